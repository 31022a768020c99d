// Randomized check of the host planner (plan.cpp), built with AddressSanitizer
// and UndefinedBehaviorSanitizer by tests/test_native_planner.py.  Fake device
// addresses are used: the planner never dereferences them.
#include <cstdint>
#include <cstdio>
#include <random>
#include <string>
#include <vector>

#include "plan.hpp"

using namespace somaopt;

static int fails = 0;
#define EXPECT(c, ...)                                    \
    do {                                                  \
        if (!(c)) {                                       \
            std::printf("FAIL %s:%d ", __FILE__, __LINE__); \
            std::printf(__VA_ARGS__);                     \
            std::printf("\n");                            \
            ++fails;                                      \
        }                                                 \
    } while (0)

// Every segment of a built plan lies inside one included tensor, at most
// p.chunk long, in order, and the segments cover each included tensor once.
// Pass 3 (arrival) includes every trainable tensor like pass 2; its vector
// alignment is checked by check_arrival_offsets.
static void check_built(const Plan& p, const std::vector<somaopt_tensor_desc>& d, int pass) {
    const int64_t chunk = p.chunk;
    std::vector<int64_t> covered(d.size(), 0);
    std::vector<int64_t> next_off(d.size(), 0);
    for (size_t s = 0; s < p.segs.size(); ++s) {
        const PlanSeg& g = p.segs[s];
        const somaopt_tensor_desc& t = d[g.tensor];
        EXPECT(t.trainable && (pass != 1 || t.owner), "segment of an excluded tensor %lld", (long long)g.tensor);
        EXPECT(g.numel <= chunk && g.numel > 0, "segment size %lld", (long long)g.numel);
        EXPECT(g.numel == g.head + g.nvec * g.vec + g.tail, "segment arithmetic");
        EXPECT(g.offset == next_off[g.tensor], "segments out of order or overlapping");
        next_off[g.tensor] = g.offset + g.numel;
        covered[g.tensor] += g.numel;
        EXPECT(16 * g.nvec < (int64_t(1) << 31), "segment body of %lld bytes", (long long)(16 * g.nvec));
        if (pass != 3 && g.vec && g.nvec > 0) {
            const int64_t gsz = grad_elem_bytes(t.grad_dtype);
            const int64_t start = g.offset + g.head;
            if (pass == 1) {
                EXPECT((reinterpret_cast<uintptr_t>(t.grad) + start * gsz) % 16 == 0,
                       "pass-1 vector misaligned: tensor %lld off %lld head %d nvec %lld grad %% 16 = %llu dtype %d",
                       (long long)g.tensor, (long long)g.offset, g.head, (long long)g.nvec,
                       (unsigned long long)(reinterpret_cast<uintptr_t>(t.grad) % 16), t.grad_dtype);
            } else {
                EXPECT((reinterpret_cast<uintptr_t>(t.param) + start * 4) % 16 == 0, "p misaligned");
                EXPECT((reinterpret_cast<uintptr_t>(t.exp_avg) + start * 4) % 16 == 0, "m misaligned");
                EXPECT((reinterpret_cast<uintptr_t>(t.exp_avg_sq) + start * 4) % 16 == 0, "v misaligned");
                EXPECT((reinterpret_cast<uintptr_t>(t.grad) + start * gsz) % (4 * gsz) == 0, "g misaligned");
                if (t.param_lowp)
                    EXPECT((reinterpret_cast<uintptr_t>(t.param_lowp) + start * 2) % 8 == 0, "copy misaligned");
            }
        }
        EXPECT(g.block >= 0 && g.block < p.n_blocks(), "block index");
        EXPECT(p.block_first[g.block] <= s && s < p.block_first[g.block + 1], "block table");
    }
    for (size_t i = 0; i < d.size(); ++i) {
        const bool want = d[i].trainable && d[i].numel > 0 && (pass != 1 || d[i].owner);
        EXPECT(covered[i] == (want ? d[i].numel : 0), "tensor %zu covered %lld of %lld", i,
               (long long)covered[i], (long long)d[i].numel);
    }
}

static void check_plan(const std::vector<somaopt_tensor_desc>& d, int pass, int64_t chunk) {
    const Plan p = build_plan(d.data(), (int64_t)d.size(), pass, chunk);
    EXPECT(p.chunk == chunk, "plan chunk %lld, asked %lld", (long long)p.chunk, (long long)chunk);
    check_built(p, d, pass);
}

// The update plan the library builds by default: 4096-element segments, or
// 2048 when that plan streams; an explicit chunk is kept.
static void check_update_plan(const std::vector<somaopt_tensor_desc>& d) {
    const int64_t n = (int64_t)d.size();
    const bool streams = streaming_plan(build_plan(d.data(), n, 2, kDefaultPass2Chunk, kUpdateSegmentCost));
    const Plan p = build_update_plan(d.data(), n, 0, kUpdateSegmentCost);
    EXPECT(p.chunk == (streams ? kStreamingPass2Chunk : kDefaultPass2Chunk), "update plan chunk %lld",
           (long long)p.chunk);
    check_built(p, d, 2);
    const Plan q = build_update_plan(d.data(), n, 3000, kUpdateSegmentCost);
    EXPECT(q.chunk == 3000, "explicit update chunk became %lld", (long long)q.chunk);
    check_built(q, d, 2);
}

// The arrival pass addresses each segment's vector body (16-byte vectors of
// the gradient and of its arriving buffer) with 32-bit buffer offsets: at the
// largest norm-pass chunk a normaliser allows, every arrival segment must
// still span fewer than 2^31 bytes.  Gradients may not overlap for arrival,
// and arriving buffers sit in an arena of their own.
static void check_arrival_offsets(const std::vector<somaopt_tensor_desc>& d, std::mt19937_64& rng, bool full) {
    std::vector<somaopt_tensor_desc> big = d;
    std::vector<const void*> inc(d.size(), nullptr);
    uintptr_t ga = 6ull << 40, ia = 7ull << 40;
    for (size_t i = 0; i < big.size(); ++i) {
        somaopt_tensor_desc& t = big[i];
        const int64_t gsz = grad_elem_bytes(t.grad_dtype);
        if (rng() % 4 == 0) t.numel = (int64_t)1 << 28;   // one huge tensor in four
        t.grad = reinterpret_cast<void*>(ga);
        ga = (ga + gsz * (uintptr_t)t.numel + 512) & ~uintptr_t(255);
        inc[i] = reinterpret_cast<void*>(ia + gsz * (uintptr_t)(rng() % 3));
        ia = (ia + gsz * (uintptr_t)t.numel + 512) & ~uintptr_t(255);
    }
    const int64_t chunk = arrival_chunk(normalise_chunk(int64_t(1) << 40, kDefaultPass1Chunk));
    EXPECT(chunk <= kMaxChunk, "arrival chunk %lld above the buffer-offset limit", (long long)chunk);
    Plan p = build_plan(big.data(), (int64_t)big.size(), 3, chunk, kSegmentCost, inc.data());
    for (const PlanSeg& g : p.segs) {
        EXPECT(g.numel <= chunk, "arrival segment of %lld elements", (long long)g.numel);
        EXPECT(16 * g.nvec < (int64_t(1) << 31), "arrival segment body of %lld bytes", (long long)(16 * g.nvec));
    }
    if (!full) return;
    // the arrival plan the library builds by default: the norm pass's chunk,
    // at most kStreamingPass3Chunk when that plan streams
    const Plan a = build_arrival_plan(big.data(), (int64_t)big.size(), kDefaultPass1Chunk, 0, inc.data());
    const bool streams = streaming_plan(build_plan(big.data(), (int64_t)big.size(), 3, kDefaultPass1Chunk,
                                                   kSegmentCost, inc.data()));
    EXPECT(a.chunk == (streams ? kStreamingPass3Chunk : kDefaultPass1Chunk), "arrival plan chunk %lld",
           (long long)a.chunk);
    check_built(a, big, 3);
}

int main() {
    std::mt19937_64 rng(12345);
    for (int trial = 0; trial < 400; ++trial) {
        const int n = 1 + (int)(rng() % 60);
        std::vector<somaopt_tensor_desc> d(n);
        uintptr_t arena[5] = {1ull << 40, 2ull << 40, 3ull << 40, 4ull << 40, 5ull << 40};
        for (int i = 0; i < n; ++i) {
            somaopt_tensor_desc& t = d[i];
            t = somaopt_tensor_desc{};
            const int64_t big = (rng() % 8 == 0) ? 200000 : 9000;
            t.numel = (int64_t)(rng() % big);
            t.grad_dtype = (int32_t)(rng() % 3);
            t.group = (int32_t)(rng() % 3);
            t.trainable = (rng() % 5) != 0;
            t.owner = (rng() % 4) != 0;
            const int64_t gsz = grad_elem_bytes(t.grad_dtype);
            auto place = [&](int k, int64_t esz) {
                const uintptr_t a = arena[k] + esz * (uintptr_t)(rng() % 5);
                arena[k] = (a + esz * (uintptr_t)t.numel + 512) & ~uintptr_t(255);
                return reinterpret_cast<void*>(a);
            };
            t.param = place(0, 4);
            t.exp_avg = place(1, 4);
            t.exp_avg_sq = place(2, 4);
            t.grad = place(3, gsz);
            if (rng() % 3 == 0) {
                t.param_lowp = place(4, 2);
                t.lowp_dtype = (rng() % 2) ? SOMAOPT_BF16 : SOMAOPT_F16;
            }
        }
        std::string err;
        Counts c;
        const int rc = validate_host(d.data(), n, 3, err, &c);
        EXPECT(rc == SOMAOPT_OK, "valid table rejected: %s", err.c_str());
        const int64_t ch1 = normalise_chunk((int64_t)(rng() % 20000), kDefaultPass1Chunk);
        const int64_t ch2 = normalise_chunk((int64_t)(rng() % 20000), kDefaultPass2Chunk);
        check_plan(d, 1, ch1);
        check_plan(d, 2, ch2);
        check_update_plan(d);
        check_arrival_offsets(d, rng, trial % 10 == 0);
        // a corrupted copy of the table must be rejected
        std::vector<somaopt_tensor_desc> bad = d;
        const int j = (int)(rng() % n);
        bad[j].trainable = 1;
        bad[j].numel = bad[j].numel ? bad[j].numel : 1;
        switch (rng() % 4) {
            case 0: bad[j].group = 3; break;
            case 1: bad[j].grad_dtype = 9; break;
            case 2: bad[j].exp_avg = bad[j].param; break;
            default: bad[j].param = nullptr; break;
        }
        EXPECT(validate_host(bad.data(), n, 3, err, nullptr) == SOMAOPT_E_INVALID, "corrupted table accepted");
    }
    std::printf("%s (%d failures)\n", fails ? "FAILED" : "ok", fails);
    return fails ? 1 : 0;
}
