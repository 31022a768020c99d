// Tensor-table planner (host only, no HIP calls).  See plan.hpp.
#include "plan.hpp"

#include <algorithm>
#include <cstdio>
#include <limits>

namespace somaopt {

namespace {

struct Interval {
    uintptr_t lo, hi;   // [lo, hi)
    int64_t tensor;
    int kind;           // 0 p, 1 m, 2 v, 3 g, 4 working copy, 5 arriving gradient
};

const char* kKindName[6] = {"param", "exp_avg", "exp_avg_sq", "grad", "param_lowp", "incoming"};

// Sorted sweep over [lo, hi) intervals: a writable interval may overlap
// nothing; a read-only one may overlap other read-only ones only.
int check_overlaps(std::vector<Interval>& iv, int readonly_kind, std::string& err) {
    std::sort(iv.begin(), iv.end(), [](const Interval& x, const Interval& y) {
        return x.lo < y.lo || (x.lo == y.lo && x.hi < y.hi);
    });
    // Keep the interval with the furthest end among writable ones and among
    // read-only ones separately.
    uintptr_t w_end = 0, r_end = 0;
    int64_t w_t = -1, r_t = -1;
    int w_k = 0, r_k = 0;
    for (const Interval& x : iv) {
        const bool writable = x.kind != readonly_kind;
        if (w_t >= 0 && x.lo < w_end) {
            err = std::string("buffers overlap: tensor ") + std::to_string(x.tensor) + " " + kKindName[x.kind] +
                  " and tensor " + std::to_string(w_t) + " " + kKindName[w_k];
            return SOMAOPT_E_INVALID;
        }
        if (writable && r_t >= 0 && x.lo < r_end) {
            err = std::string("buffers overlap: tensor ") + std::to_string(x.tensor) + " " + kKindName[x.kind] +
                  " and tensor " + std::to_string(r_t) + " " + kKindName[r_k];
            return SOMAOPT_E_INVALID;
        }
        if (writable) {
            if (x.hi > w_end || w_t < 0) { w_end = x.hi; w_t = x.tensor; w_k = x.kind; }
        } else {
            if (x.hi > r_end || r_t < 0) { r_end = x.hi; r_t = x.tensor; r_k = x.kind; }
        }
    }
    return SOMAOPT_OK;
}

std::string fmt(const char* f, long long a = 0, long long b = 0, long long c = 0) {
    char buf[256];
    std::snprintf(buf, sizeof(buf), f, a, b, c);
    return buf;
}

}  // namespace

int64_t normalise_chunk(int64_t requested, int64_t dflt, int64_t max_chunk) {
    int64_t c = requested > 0 ? requested : dflt;
    c = (c / 8) * 8;
    if (c < 256) c = 256;
    if (c > max_chunk) c = max_chunk;
    return c;
}

int validate_host(const somaopt_tensor_desc* d, int64_t n, int32_t n_groups, std::string& err,
                  Counts* counts) {
    if (n < 0) { err = "n_tensors < 0"; return SOMAOPT_E_INVALID; }
    if (n > 0 && d == nullptr) { err = "descs is NULL"; return SOMAOPT_E_INVALID; }
    if (n_groups < 1 || n_groups > SOMAOPT_MAX_GROUPS) {
        err = fmt("n_groups=%lld outside [1, %lld]", n_groups, SOMAOPT_MAX_GROUPS);
        return SOMAOPT_E_INVALID;
    }
    Counts c;
    std::vector<Interval> iv;
    for (int64_t i = 0; i < n; ++i) {
        const somaopt_tensor_desc& t = d[i];
        if (t.trainable != 0 && t.trainable != 1) {
            err = fmt("tensor %lld: trainable must be 0 or 1", i);
            return SOMAOPT_E_INVALID;
        }
        if (!t.trainable) continue;   // frozen: never read, never validated further
        if (t.owner != 0 && t.owner != 1) {
            err = fmt("tensor %lld: owner must be 0 or 1", i);
            return SOMAOPT_E_INVALID;
        }
        if (t.numel < 0) { err = fmt("tensor %lld: numel %lld < 0", i, t.numel); return SOMAOPT_E_INVALID; }
        if (t.numel > (int64_t(1) << 40)) { err = fmt("tensor %lld: numel too large", i); return SOMAOPT_E_INVALID; }
        if (t.grad_dtype != SOMAOPT_F32 && t.grad_dtype != SOMAOPT_BF16 && t.grad_dtype != SOMAOPT_F16) {
            err = fmt("tensor %lld: unknown grad_dtype %lld", i, t.grad_dtype);
            return SOMAOPT_E_INVALID;
        }
        if (t.param_lowp && t.lowp_dtype != SOMAOPT_BF16 && t.lowp_dtype != SOMAOPT_F16) {
            err = fmt("tensor %lld: lowp_dtype %lld must be bf16 or fp16", i, t.lowp_dtype);
            return SOMAOPT_E_INVALID;
        }
        if (t.reserved != 0) {
            err = fmt("tensor %lld: reserved field must be 0", i);
            return SOMAOPT_E_INVALID;
        }
        if (t.group < 0 || t.group >= n_groups) {
            err = fmt("tensor %lld: group %lld outside [0, %lld)", i, t.group, n_groups);
            return SOMAOPT_E_INVALID;
        }
        c.n_trainable++;
        c.trainable_numel += t.numel;
        if (t.owner) c.owned_numel += t.numel;
        if (t.numel == 0) continue;
        const void* ptrs[5] = {t.param, t.exp_avg, t.exp_avg_sq, t.grad, t.param_lowp};
        const int64_t esz[5] = {4, 4, 4, grad_elem_bytes(t.grad_dtype), 2};
        const int nbuf = t.param_lowp ? 5 : 4;
        for (int k = 0; k < nbuf; ++k) {
            uintptr_t a = reinterpret_cast<uintptr_t>(ptrs[k]);
            if (a == 0) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] + " pointer is NULL";
                return SOMAOPT_E_INVALID;
            }
            if (a % (uintptr_t)esz[k]) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] +
                      " pointer is not aligned to its element size";
                return SOMAOPT_E_INVALID;
            }
            uintptr_t bytes = (uintptr_t)t.numel * (uintptr_t)esz[k];
            if (a + bytes < a) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] + " range wraps";
                return SOMAOPT_E_INVALID;
            }
            iv.push_back(Interval{a, a + bytes, i, k});
        }
    }
    // Overlap check: written buffers (p, m, v, working copy) may overlap
    // nothing; gradients may overlap other gradients (both read only) but no
    // written buffer.
    if (check_overlaps(iv, 3, err) != SOMAOPT_OK) return SOMAOPT_E_INVALID;
    if (counts) *counts = c;
    return SOMAOPT_OK;
}

int validate_arrival(const somaopt_tensor_desc* d, int64_t n, const void* const* incoming, std::string& err) {
    if (n > 0 && incoming == nullptr) { err = "incoming is NULL"; return SOMAOPT_E_INVALID; }
    std::vector<Interval> iv;
    for (int64_t i = 0; i < n; ++i) {
        const somaopt_tensor_desc& t = d[i];
        if (!t.trainable || t.numel == 0) continue;
        const void* ptrs[6] = {t.param, t.exp_avg, t.exp_avg_sq, t.grad, t.param_lowp, incoming[i]};
        const int64_t gsz = grad_elem_bytes(t.grad_dtype);
        const int64_t esz[6] = {4, 4, 4, gsz, 2, gsz};
        for (int k = 0; k < 6; ++k) {
            if (k == 4 && !t.param_lowp) continue;
            const uintptr_t a = reinterpret_cast<uintptr_t>(ptrs[k]);
            if (a == 0) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] + " pointer is NULL";
                return SOMAOPT_E_INVALID;
            }
            if (a % (uintptr_t)esz[k]) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] +
                      " pointer is not aligned to its element size";
                return SOMAOPT_E_INVALID;
            }
            const uintptr_t bytes = (uintptr_t)t.numel * (uintptr_t)esz[k];
            if (a + bytes < a) {
                err = std::string("tensor ") + std::to_string(i) + ": " + kKindName[k] + " range wraps";
                return SOMAOPT_E_INVALID;
            }
            iv.push_back(Interval{a, a + bytes, i, k});
        }
    }
    return check_overlaps(iv, 5, err);
}

namespace {

// Smallest e in [0, vec) such that every listed address, advanced by e
// elements of its size, is aligned to `vec * size`; -1 if none exists.
int64_t common_head(const uintptr_t* addr, const int64_t* esz, int n, int64_t vec) {
    for (int64_t e = 0; e < vec; ++e) {
        bool ok = true;
        for (int k = 0; k < n && ok; ++k) {
            uintptr_t need = (uintptr_t)(vec * esz[k]);
            ok = ((addr[k] + (uintptr_t)(e * esz[k])) % need) == 0;
        }
        if (ok) return e;
    }
    return -1;
}

}  // namespace

Plan build_plan(const somaopt_tensor_desc* d, int64_t n, int pass, int64_t chunk, int64_t segment_cost,
                const void* const* incoming) {
    Plan plan;
    plan.chunk = chunk;
    for (int64_t i = 0; i < n; ++i) {
        const somaopt_tensor_desc& t = d[i];
        if (!t.trainable || t.numel == 0) continue;
        if (pass == 1 && !t.owner) continue;
        const int64_t gsz = grad_elem_bytes(t.grad_dtype);
        int64_t vec, head;
        if (pass == 1) {
            vec = 16 / gsz;
            uintptr_t a[1] = {reinterpret_cast<uintptr_t>(t.grad)};
            int64_t s[1] = {gsz};
            head = common_head(a, s, 1, vec);
        } else if (pass == 3) {
            vec = 16 / gsz;
            uintptr_t a[2] = {reinterpret_cast<uintptr_t>(t.grad), reinterpret_cast<uintptr_t>(incoming[i])};
            int64_t s[2] = {gsz, gsz};
            head = common_head(a, s, 2, vec);
        } else {
            vec = 4;
            uintptr_t a[5] = {reinterpret_cast<uintptr_t>(t.param), reinterpret_cast<uintptr_t>(t.exp_avg),
                              reinterpret_cast<uintptr_t>(t.exp_avg_sq), reinterpret_cast<uintptr_t>(t.grad),
                              reinterpret_cast<uintptr_t>(t.param_lowp)};
            int64_t s[5] = {4, 4, 4, gsz, 2};
            head = common_head(a, s, t.param_lowp ? 5 : 4, vec);
        }
        if (head < 0) {
            // No common alignment: the whole tensor takes the scalar path.
            for (int64_t off = 0; off < t.numel; off += chunk) {
                int64_t len = std::min(chunk, t.numel - off);
                plan.segs.push_back(PlanSeg{i, off, len, 0, (int32_t)len, 0, 0, -1});
            }
            continue;
        }
        head = std::min(head, t.numel);
        int64_t off = 0;
        bool first = true;
        while (off < t.numel) {
            int64_t h = first ? head : 0;
            int64_t room = first ? ((chunk - h) / vec) * vec : chunk;   // body capacity
            int64_t body = std::min(room, t.numel - off - h);
            int64_t nv = body / vec;
            int64_t tl = body - nv * vec;
            int64_t len = h + body;
            plan.segs.push_back(PlanSeg{i, off, len, nv, (int32_t)h, (int32_t)tl, (int32_t)vec, -1});
            off += len;
            first = false;
        }
    }
    // Pack consecutive segments into workgroups of bounded cost.
    if (segment_cost < 0) segment_cost = default_segment_cost(pass);
    plan.block_first.clear();
    int64_t cost = 0;
    for (size_t s = 0; s < plan.segs.size(); ++s) {
        int64_t c = plan.segs[s].numel + segment_cost;
        if (plan.block_first.empty() || cost + c > chunk + segment_cost) {
            plan.block_first.push_back((uint32_t)s);
            cost = 0;
        }
        cost += c;
        plan.segs[s].block = (int32_t)(plan.block_first.size() - 1);
    }
    plan.block_first.push_back((uint32_t)plan.segs.size());
    if (plan.segs.empty()) plan.block_first.assign(1, 0);
    return plan;
}

bool streaming_plan(const Plan& p) {
    int64_t total = 0, full = 0;
    for (const PlanSeg& s : p.segs) {
        total += s.numel;
        if (s.numel == p.chunk) full += s.numel;
    }
    return total > 0 && 2 * full >= total;
}

Plan build_arrival_plan(const somaopt_tensor_desc* d, int64_t n, int64_t pass1_chunk, int64_t requested,
                        const void* const* incoming) {
    if (requested > 0)
        return build_plan(d, n, 3, normalise_chunk(requested, kDefaultPass1Chunk), kSegmentCost, incoming);
    const int64_t chunk = arrival_chunk(pass1_chunk);
    Plan p = build_plan(d, n, 3, chunk, kSegmentCost, incoming);
    if (streaming_plan(p) && chunk > kStreamingPass3Chunk)
        p = build_plan(d, n, 3, kStreamingPass3Chunk, kSegmentCost, incoming);
    return p;
}

Plan build_update_plan(const somaopt_tensor_desc* d, int64_t n, int64_t requested, int64_t segment_cost) {
    if (requested > 0) return build_plan(d, n, 2, normalise_chunk(requested, kDefaultPass2Chunk), segment_cost);
    Plan p = build_plan(d, n, 2, kDefaultPass2Chunk, segment_cost);
    if (streaming_plan(p)) p = build_plan(d, n, 2, kStreamingPass2Chunk, segment_cost);
    return p;
}

}  // namespace somaopt
