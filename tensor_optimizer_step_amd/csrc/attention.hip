// Tiled attention over frozen and trainable keys (gfx950, bf16 MFMA, fp32
// accumulation).
//
// SomaSpeed landing page, paragraph 5: queries from the trainable action
// computation read the context keys/values tile by tile, the full score
// matrix is never stored, and frozen inputs get no gradient work.  Here the
// keys of every (batch, head) are a frozen source followed by a trainable one:
// the backward produces dQ for every query and dK/dV only for the trainable
// keys -- the frozen tiles cost three products per tile (S, dP, dQ) instead of
// five.  dK/dV come out of the dQ kernel itself when one workgroup holds all
// queries of a (batch, head) (at most 64), else from a second kernel launched
// over the trainable keys only.
//
// Layout: Q, K, V, O, dO are bf16 [B][H][L][D], rows contiguous; LSE and
// delta fp32 [B][H][Lq]; dQ fp32 [B][H][Lq][D]; dK, dV fp32 [B][H][Lk-Lf][D].
//
// Every workgroup is 4 waves; a wave owns 16 rows (queries, or keys in the
// dK/dV kernel).  All products are v_mfma_f32_16x16x32_bf16: with 16 lanes
// r = lane % 16 and 4 groups g = lane / 16, a lane holds A[r][8g..8g+7] and
// B[8g..8g+7][r] and receives C[4g+i][r], i = 0..3.  Computing S^T = K Q^T
// leaves each lane with four consecutive keys of one query -- the operand P^T
// needs for O^T = V^T P^T -- so no register shuffles are needed between the
// two products, and each lane owns one query row's softmax state.  The second
// product reduces over two such 16-key blocks at once: a lane's eight B
// values are its keys 4g..4g+3 of both blocks, and its A operand reads the
// same eight keys from a transposed LDS tile (the order of the terms inside
// one product's reduction is free).
#include <hip/hip_runtime.h>

#include "attention.hpp"

namespace somaopt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kRows = 64;          // rows staged per tile (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kPadRow = 8;         // bf16 padding of a row-major LDS row read by rows
constexpr int kPadTr = 16;         // bf16 padding of a row-major LDS row read transposed
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}
__device__ __forceinline__ float bf16_at(uint32_t w, int half) {
    return __uint_as_float(half ? (w & 0xffff0000u) : (w << 16));
}

// 2^x with the hardware v_exp_f32: results below 2^-126 flush to zero, which
// is immaterial for softmax weights (every argument here is <= 0 or -inf).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum / max over the four lanes r, r+16, r+32, r+48 that share a row.
__device__ __forceinline__ float group_sum(float x) {
    x += __shfl_xor(x, 16);
    x += __shfl_xor(x, 32);
    return x;
}
__device__ __forceinline__ float group_max(float x) {
    x = fmaxf(x, __shfl_xor(x, 16));
    x = fmaxf(x, __shfl_xor(x, 32));
    return x;
}

// Raw buffer resource over one (batch, head) matrix of `rows` x D bf16
// values: the hardware bounds-checks every access, so rows at or past the end
// read as zero without a branch (and the compiler keeps exact counts of the
// loads in flight).  Word 3 selects the 32-bit data format untyped buffer
// accesses require on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t mat_rsrc(const uint16_t* base, int rows) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(base), (short)0, rows * D * 2, kRsrcWord3);
}
// 16 bytes (8 bf16) of row `row`, starting at column `col`.
template <int D>
__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, int row, int col) {
    return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (row * D + col) * 2, 0, 0));
}

// Rows [row0, row0 + 64) of a [L][D] bf16 matrix, as held by one thread
// between its global loads and its LDS stores (so the loads of later tiles
// can be in flight while the current tile is computed).  Each wave reads
// whole rows: lanes 16 apart take consecutive 16-byte chunks of one row.
template <int D>
struct RowChunks {
    static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
    static constexpr int kPer = kRows * kChunks / kThreads;  // chunks per thread
    u32x4 c[kPer];
    __device__ __forceinline__ void load(__amdgpu_buffer_rsrc_t src, int row0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + kThreads * j;
            c[j] = bload16<D>(src, row0 + i / kChunks, (i % kChunks) * 8);
        }
    }
    template <int P>
    __device__ __forceinline__ void store(uint16_t (*dst)[P]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + kThreads * j;
            *reinterpret_cast<u32x4*>(&dst[i / kChunks][(i % kChunks) * 8]) = c[j];
        }
    }
};

// Transposed read of a row-major LDS tile with gfx950's ds_read_b64_tr_b16:
// within each 16-lane group, lane m supplies the address of columns
// d0 + 4 (m % 4) .. + 3 of row k0 + m / 4, and lane r receives rows
// k0 .. k0 + 3 of column d0 + r (four bf16 in row order) -- the operand layout
// of a product that reduces over the rows.  With a row pitch of D + 16 bf16 the
// 64 lanes' reads are spread evenly over the LDS banks.
template <int P>
__device__ __forceinline__ u32x2 tr_rows4(const uint16_t (*t)[P], int k0, int d0, int r) {
    typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;
    const uint16_t* p = &t[k0 + (r >> 2)][d0 + 4 * (r & 3)];
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4*)p));
}
// A operand of a 16x16x32 product from a row-major tile: column d0 + r, the
// four rows from k0 and the four from k1.
template <int P>
__device__ __forceinline__ u32x4 tr_pair(const uint16_t (*t)[P], int k0, int k1, int d0, int r) {
    const u32x2 lo = tr_rows4(t, k0, d0, r);
    const u32x2 hi = tr_rows4(t, k1, d0, r);
    return u32x4{lo.x, lo.y, hi.x, hi.y};
}

// Pipeline over a sequence of n_tiles 64-row tiles: two register stages, so
// while tile t is computed from LDS the loads of tiles t + 1 and t + 2 are in
// flight.  `load(stage, t)` issues tile t's global loads into a stage,
// `store(stage)` writes a stage to LDS, `compute(t)` runs tile t's products
// from LDS.  The loads are unconditional: tiles past the end lie outside the
// buffer resources, so they read zero without touching memory.  Tiles are
// processed in pairs (an odd last tile is paired with an all-padding tile
// whose keys the products mask out), so the loop body is straight-line and
// every path into the loop head has the same loads outstanding: the compiler
// then waits for just the older stage.
template <class Stage, class Load, class Store, class Compute>
__device__ __forceinline__ void two_stage_tiles(int n_tiles, Stage& s0, Stage& s1, Load load, Store store,
                                                Compute compute) {
    // The scheduling barriers keep each stage's loads together and in program
    // order (otherwise the two prologue stages interleave and the first
    // stage's wait would cover both).
    load(s0, 0);
    __builtin_amdgcn_sched_barrier(0);
    load(s1, 1);
    __builtin_amdgcn_sched_barrier(0);
    for (int t = 0; t < n_tiles; t += 2) {
        __syncthreads();
        store(s0);
        __syncthreads();
        load(s0, t + 2);
        __builtin_amdgcn_sched_barrier(0);
        compute(t);
        __syncthreads();
        store(s1);
        __syncthreads();
        load(s1, t + 3);
        __builtin_amdgcn_sched_barrier(0);
        compute(t + 1);
    }
}

// Workgroup coordinates (query block, head, batch) grouped by XCD.  The
// hardware hands consecutive workgroups to the eight XCDs in turn, each with
// its own L2; this bijection gives every XCD one contiguous run of the
// logical order, in which the query batches that share one context batch
// (ctx_share of them, same head) are adjacent -- so a shared context is read
// from HBM into one XCD's L2 and reused there; so are the query blocks of
// one (batch, head), which read the same keys (measured on MI355X, 64 query
// batches, 960 context keys: contexts shared by 2 over 12 heads 71.6 -> 61.3
// us; 128 queries per head 90.2 -> 79.8 us, 256 queries 165 -> 130 us).  With
// one query block and no sharing nothing is reused and the plain order is
// kept.  Only placement depends on the dispatch order; any order computes the
// same result.
struct WgCoord {
    int x, h, b;
};
__device__ __forceinline__ WgCoord xcd_grouped(int share) {
    if (share <= 1 && gridDim.x == 1) return WgCoord{(int)blockIdx.x, (int)blockIdx.y, (int)blockIdx.z};
    // 64-bit: a grid of up to 2^16 x 2^16 x 2^16 workgroups
    const uint64_t nx = gridDim.x, nh = gridDim.y, nb = gridDim.z;
    const uint64_t n = nx * nh * nb;
    const uint64_t l = blockIdx.x + nx * (blockIdx.y + nh * (uint64_t)blockIdx.z);
    const uint64_t xcd = l % 8, local = l / 8, per = n / 8, rem = n % 8;
    uint64_t t = xcd * per + (xcd < rem ? xcd : rem) + local;   // logical index
    WgCoord c;
    c.x = (int)(t % nx);
    t /= nx;
    const uint64_t sh = (uint64_t)share;
    const uint64_t m = t % sh;
    t /= sh;
    c.h = (int)(t % nh);
    c.b = (int)((t / nh) * sh + m);
    return c;
}

// The key tiles of one (batch, head), source by source.  Resources are built
// once; picking one per tile is a uniform (scalar) choice.
template <int D>
//
// The frozen source comes first, or, with trainable_first, the trainable
// one: the forward visits the trainable tiles first, and so does the dQ
// kernel that also produces dK/dV, so that their extra products overlap the
// loads of the frozen tiles instead of trailing after the last load.
struct KeyTiles {
    __amdgpu_buffer_rsrc_t k[2], v[2];
    int rows[2];
    int first, nf, n;   // source visited first, its tile count, tiles in total
    __device__ __forceinline__ KeyTiles(const AttnArgs& a, int b, int h, bool trainable_first = false) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const KeySrc& src = a.src[s];
            const size_t off = ((size_t)(b / src.share) * a.heads + h) * (size_t)src.stride * D;
            k[s] = mat_rsrc<D>(static_cast<const uint16_t*>(src.k) + off, src.rows);
            v[s] = mat_rsrc<D>(static_cast<const uint16_t*>(src.v) + off, src.rows);
            rows[s] = src.rows;
        }
        first = trainable_first ? 1 : 0;
        nf = (rows[first] + kRows - 1) / kRows;
        n = nf + (rows[1 - first] + kRows - 1) / kRows;
    }
    // Source and first row of tile t (tiles past the end fall past the end
    // of the source visited second).
    __device__ __forceinline__ int src_of(int t) const { return t < nf ? first : 1 - first; }
    __device__ __forceinline__ int row_of(int t) const { return (t < nf ? t : t - nf) * kRows; }
    __device__ __forceinline__ int bound_of(int t) const { return rows[src_of(t)]; }
};

// ------------------------------------------------------------------ forward

template <int D>
struct FwdLds {
    uint16_t k[kRows][D + kPadRow];   // K tile, row-major (read by rows)
    uint16_t v[kRows][D + kPadTr];    // V tile, row-major (read transposed)
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd(AttnArgs a) {
    __shared__ FwdLds<D> s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const WgCoord wc = xcd_grouped(a.src[0].share);
    const size_t bh = (size_t)wc.b * a.heads + wc.h;
    const auto Q = mat_rsrc<D>(static_cast<const uint16_t*>(a.q) + bh * a.lq * D, a.lq);
    // The trainable keys' tiles first: a workgroup then ends on its frozen
    // context's sequential stream rather than on a separate buffer (measured
    // on MI355X, 64 batches x 8 heads, 64 queries, 960 context + 64 action
    // keys: 57.4 -> 55.3 us; 448 or 1984 context keys, or a context shared by
    // 4 query batches: 2-4 us less; 128 queries per head unchanged).
    const KeyTiles<D> kt(a, wc.b, wc.h, true);
    const int q = wc.x * kRows + 16 * w + r;
    const bool qv = q < a.lq;
    // B operand of S^T = K Q^T: Q[q][32 kk + 8 g .. + 7] (zero past the last query)
    u32x4 qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) qb[kk] = bload16<D>(Q, q, 32 * kk + 8 * g);
    const float sc = a.scale * kLog2e;   // scores in log2 units
    float m = -INFINITY, lsum = 0.0f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Products of one staged 64-key tile: the tile's scores, one max and one
    // rescale of the accumulator per tile, then O^T += V^T P^T over two
    // 32-key halves.
    auto tile = [&](int t) {
        // A wave computing a tile takes issue priority over the waves of the
        // other workgroup on its SIMD, which are then storing or waiting for
        // loads.  Measured on MI355X (64 query batches, 960 context + 64
        // action keys): 57.5 -> 55.2 us over 8 heads, 40.7 -> 36.2 us with a
        // context shared by 4 over 6 heads, 2-4 us less at 448 or 1984 keys,
        // 128 queries, 12 or 16 heads; 62.9 -> 64.5 us over 12 heads sharing
        // by 2, the one shape measured slower.  The backward is unchanged by it.
        __builtin_amdgcn_s_setprio(1);
        const int key0 = kt.row_of(t), bound = kt.bound_of(t);
        f32x4 st[kRows / 16];
#pragma unroll
        for (int kb = 0; kb < kRows / 16; ++kb) {
            st[kb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                st[kb] = mfma32(*reinterpret_cast<const u32x4*>(&s.k[16 * kb + r][32 * kk + 8 * g]), qb[kk], st[kb]);
        }
        float bm = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < kRows / 16; ++kb) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + 16 * kb + 4 * g + i;
                st[kb][i] = key < bound ? st[kb][i] * sc : -INFINITY;
                bm = fmaxf(bm, st[kb][i]);
            }
        }
        bm = group_max(bm);
        // The first tile always holds a key (row 0 of the first source that
        // has keys), so mn is finite from then on; a padding tile (every key
        // masked) leaves m unchanged and alpha = 1.
        const float mn = fmaxf(m, bm);
        const float alpha = exp2_hw(m - mn);
        m = mn;
        float ps = 0.0f;
        u32x2 pb[kRows / 16];
#pragma unroll
        for (int kb = 0; kb < kRows / 16; ++kb) {
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = exp2_hw(st[kb][i] - mn);
            ps += (p[0] + p[1]) + (p[2] + p[3]);
            pb[kb] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
        }
        lsum = lsum * alpha + ps;
#pragma unroll
        for (int nb = 0; nb < D / 16; ++nb) acc[nb] *= alpha;
#pragma unroll
        for (int h = 0; h < kRows / 32; ++h) {
            const u32x4 bop = {pb[2 * h].x, pb[2 * h].y, pb[2 * h + 1].x, pb[2 * h + 1].y};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb)
                acc[nb] = mfma32(tr_pair(s.v, 32 * h + 4 * g, 32 * h + 16 + 4 * g, 16 * nb, r), bop, acc[nb]);
        }
        __builtin_amdgcn_s_setprio(0);
    };
    struct KV {
        RowChunks<D> k, v;
    } st0, st1;
    two_stage_tiles(
        kt.n, st0, st1,
        [&](KV& x, int t) {
            const int src = kt.src_of(t), row0 = kt.row_of(t);
            x.k.load(kt.k[src], row0);
            x.v.load(kt.v[src], row0);
        },
        [&](const KV& x) {
            x.k.store(s.k);
            x.v.store(s.v);
        },
        tile);
    const float total = group_sum(lsum);
    if (!qv) return;
    const float inv = 1.0f / total;
    uint16_t* O = static_cast<uint16_t*>(a.o) + bh * a.lq * D + (size_t)q * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
        const u32x2 out = {pack_bf16(acc[nb][0] * inv, acc[nb][1] * inv), pack_bf16(acc[nb][2] * inv, acc[nb][3] * inv)};
        *reinterpret_cast<u32x2*>(O + 16 * nb + 4 * g) = out;
    }
    if (g == 0) a.lse[bh * a.lq + q] = (m + log2f(total)) * kLn2;
}

// ------------------------------------------------------- backward: dQ, delta

template <int D>
struct DqLds {
    uint16_t k[kRows][D + kPadRow];   // K tile, read by rows (A of S^T)
    uint16_t kr[kRows][D + kPadTr];   // the same K tile, read transposed (A of dQ^T)
    uint16_t v[kRows][D + kPadRow];   // V tile, read by rows (A of dP^T)
};
// With every query of the (batch, head) in the workgroup, the same memory
// holds, after a trainable tile's dQ products, the workgroup's Q and dO rows
// (one pitch, read both ways) and their log-sum-exp and delta for the tile's
// dK and dV.
template <int D>
struct DqKvLds {
    uint16_t q[kRows][D + kPadTr];
    uint16_t d_o[kRows][D + kPadTr];
    float lse2[kRows];
    float delta[kRows];
};
template <int D>
union DqShared {
    DqLds<D> t;
    DqKvLds<D> x;
};

// FUSE_KV (the workgroup holds every query of its (batch, head), i.e.
// lq <= 64): after the dQ products of each trainable tile, the workgroup also
// produces that tile's dK and dV -- complete, since no other workgroup holds
// queries of this (batch, head) -- in place of the separate dK/dV kernel,
// which would read Q, dO, K and V again.  Wave w takes keys 16 w .. + 15 of the
// tile; the products are those of attn_bwd_dkdv over the 64 queries.
template <int D, bool FUSE_KV>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq(AttnArgs a) {
    __shared__ DqShared<D> su;
    DqLds<D>& s = su.t;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const WgCoord wc = xcd_grouped(a.src[0].share);
    const size_t bh = (size_t)wc.b * a.heads + wc.h;
    const auto Q = mat_rsrc<D>(static_cast<const uint16_t*>(a.q) + bh * a.lq * D, a.lq);
    const auto dO = mat_rsrc<D>(static_cast<const uint16_t*>(a.d_o) + bh * a.lq * D, a.lq);
    const auto O = mat_rsrc<D>(static_cast<const uint16_t*>(a.o) + bh * a.lq * D, a.lq);
    const KeyTiles<D> kt(a, wc.b, wc.h, FUSE_KV);
    const int q = wc.x * kRows + 16 * w + r;
    const bool qv = q < a.lq;
    u32x4 qb[D / 32], db[D / 32];
    float dot = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        qb[kk] = bload16<D>(Q, q, 32 * kk + 8 * g);
        db[kk] = bload16<D>(dO, q, 32 * kk + 8 * g);
        const u32x4 ov = bload16<D>(O, q, 32 * kk + 8 * g);
#pragma unroll
        for (int e = 0; e < 8; ++e) dot += bf16_at(db[kk][e / 2], e & 1) * bf16_at(ov[e / 2], e & 1);
    }
    const float delta = group_sum(dot);   // sum_c dO[q][c] O[q][c]
    if (qv && g == 0) a.delta[bh * a.lq + q] = delta;
    const float lse2 = qv ? a.lse[bh * a.lq + q] * kLog2e : INFINITY;
    const float sc = a.scale * kLog2e;
    f32x4 acc[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // dK and dV of one staged trainable tile (FUSE_KV only); key0 is the
    // tile's first trainable key, bound the trainable key count.
    auto tile_dkdv = [&](int key0, int bound) {
        // B operands from the staged tile: K[key][32 kk + 8 g ..], V[key][..]
        u32x4 kb_[D / 32], vb_[D / 32];
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            kb_[kk] = *reinterpret_cast<const u32x4*>(&s.k[16 * w + r][32 * kk + 8 * g]);
            vb_[kk] = *reinterpret_cast<const u32x4*>(&s.v[16 * w + r][32 * kk + 8 * g]);
        }
        __syncthreads();   // every wave is done with the K / V tiles
        // each wave publishes its 16 query rows of Q and dO, LSE and delta
#pragma unroll
        for (int kk = 0; kk < D / 32; ++kk) {
            *reinterpret_cast<u32x4*>(&su.x.q[16 * w + r][32 * kk + 8 * g]) = qb[kk];
            *reinterpret_cast<u32x4*>(&su.x.d_o[16 * w + r][32 * kk + 8 * g]) = db[kk];
        }
        if (g == 0) {
            su.x.lse2[16 * w + r] = lse2;
            su.x.delta[16 * w + r] = qv ? delta : 0.0f;
        }
        __syncthreads();
        u32x2 pb[kRows / 16], dsq[kRows / 16];
#pragma unroll
        for (int qb_ = 0; qb_ < kRows / 16; ++qb_) {
            // S = Q K^T and dP = dO V^T: lane holds [query 16 qb_ + 4 g + i][key r]
            f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                st = mfma32(*reinterpret_cast<const u32x4*>(&su.x.q[16 * qb_ + r][32 * kk + 8 * g]), kb_[kk], st);
                dpt = mfma32(*reinterpret_cast<const u32x4*>(&su.x.d_o[16 * qb_ + r][32 * kk + 8 * g]), vb_[kk], dpt);
            }
            float pr[4], dsr[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qi = 16 * qb_ + 4 * g + i;
                pr[i] = exp2_hw(st[i] * sc - su.x.lse2[qi]);
                dsr[i] = pr[i] * (dpt[i] - su.x.delta[qi]);
            }
            pb[qb_] = u32x2{pack_bf16(pr[0], pr[1]), pack_bf16(pr[2], pr[3])};
            dsq[qb_] = u32x2{pack_bf16(dsr[0], dsr[1]), pack_bf16(dsr[2], dsr[3])};
        }
        // dV^T = dO^T P, then dK^T = Q^T dS, over two 32-query halves (one
        // accumulator set live at a time keeps the register count of the
        // streaming loop)
        const int j = key0 + 16 * w + r;   // trainable key index
        const size_t row = (bh * (size_t)bound + j) * D;
#pragma unroll 1
        for (int which = 0; which < 2; ++which) {
            const u32x2* op = which == 0 ? pb : dsq;
            f32x4 c[D / 16];
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) c[nb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int h = 0; h < kRows / 32; ++h) {
                const u32x4 bop = {op[2 * h].x, op[2 * h].y, op[2 * h + 1].x, op[2 * h + 1].y};
#pragma unroll
                for (int nb = 0; nb < D / 16; ++nb) {
                    const int k0 = 32 * h + 4 * g, k1 = 32 * h + 16 + 4 * g;
                    const u32x4 aop = which == 0 ? tr_pair(su.x.d_o, k0, k1, 16 * nb, r)
                                                 : tr_pair(su.x.q, k0, k1, 16 * nb, r);
                    c[nb] = mfma32(aop, bop, c[nb]);
                }
            }
            if (j < bound) {
                float* out = (which == 0 ? a.dv : a.dk) + row;
                const float f = which == 0 ? 1.0f : a.scale;
#pragma unroll
                for (int nb = 0; nb < D / 16; ++nb) *reinterpret_cast<f32x4*>(out + 16 * nb + 4 * g) = c[nb] * f;
            }
        }
    };
    auto tile = [&](int t) {
        const int key0 = kt.row_of(t), bound = kt.bound_of(t);
        u32x2 dsb[kRows / 16];
#pragma unroll
        for (int kb = 0; kb < kRows / 16; ++kb) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                st = mfma32(*reinterpret_cast<const u32x4*>(&s.k[16 * kb + r][32 * kk + 8 * g]), qb[kk], st);
                dpt = mfma32(*reinterpret_cast<const u32x4*>(&s.v[16 * kb + r][32 * kk + 8 * g]), db[kk], dpt);
            }
            float ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + 16 * kb + 4 * g + i;
                const float p = key < bound ? exp2_hw(st[i] * sc - lse2) : 0.0f;
                ds[i] = p * (dpt[i] - delta);
            }
            dsb[kb] = u32x2{pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
        }
        // dQ^T += K^T dS^T over two 32-key halves
#pragma unroll
        for (int h = 0; h < kRows / 32; ++h) {
            const u32x4 bop = {dsb[2 * h].x, dsb[2 * h].y, dsb[2 * h + 1].x, dsb[2 * h + 1].y};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb)
                acc[nb] = mfma32(tr_pair(s.kr, 32 * h + 4 * g, 32 * h + 16 + 4 * g, 16 * nb, r), bop, acc[nb]);
        }
        if constexpr (FUSE_KV) {
            if (t < kt.n && kt.src_of(t) == 1) tile_dkdv(key0, bound);
        }
    };
    // K is loaded once and written twice, at the pitch of each way it is read.
    struct KV {
        RowChunks<D> k, v;
    } st0, st1;
    two_stage_tiles(
        kt.n, st0, st1,
        [&](KV& x, int t) {
            const int src = kt.src_of(t), row0 = kt.row_of(t);
            x.k.load(kt.k[src], row0);
            x.v.load(kt.v[src], row0);
        },
        [&](const KV& x) {
            x.k.store(s.k);
            x.k.store(s.kr);
            x.v.store(s.v);
        },
        tile);
    if (!qv) return;
    float* dQ = a.dq + bh * a.lq * D + (size_t)q * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) *reinterpret_cast<f32x4*>(dQ + 16 * nb + 4 * g) = acc[nb] * a.scale;
}

// ------------------------------------------ backward: dK, dV of trainable keys

template <int D>
struct DkvLds {
    uint16_t q[kRows][D + kPadRow];    // Q chunk, read by rows (A of S)
    uint16_t d_o[kRows][D + kPadRow];  // dO chunk, read by rows (A of dP)
    uint16_t qr[kRows][D + kPadTr];    // the same Q chunk, read transposed (A of dK^T)
    uint16_t dor[kRows][D + kPadTr];   // the same dO chunk, read transposed (A of dV^T)
    float lse2[kRows];
    float delta[kRows];
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv(AttnArgs a) {
    __shared__ DkvLds<D> s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const WgCoord wc = xcd_grouped(1);   // key blocks of one (batch, head) share its Q and dO
    const size_t bh = (size_t)wc.b * a.heads + wc.h;
    const KeySrc& src = a.src[1];
    const int lt = src.rows;
    const auto Q = mat_rsrc<D>(static_cast<const uint16_t*>(a.q) + bh * a.lq * D, a.lq);
    const auto dO = mat_rsrc<D>(static_cast<const uint16_t*>(a.d_o) + bh * a.lq * D, a.lq);
    const size_t koff = ((size_t)(wc.b / src.share) * a.heads + wc.h) * (size_t)src.stride * D;
    const auto K = mat_rsrc<D>(static_cast<const uint16_t*>(src.k) + koff, lt);
    const auto V = mat_rsrc<D>(static_cast<const uint16_t*>(src.v) + koff, lt);
    const int j = wc.x * kRows + 16 * w + r;   // trainable key index
    const bool kv = j < lt;
    const int key = j;
    // B operands: K[key][32 kk + 8 g ..], V[key][32 kk + 8 g ..] (zero past the last key)
    u32x4 kb_[D / 32], vb_[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        kb_[kk] = bload16<D>(K, key, 32 * kk + 8 * g);
        vb_[kk] = bload16<D>(V, key, 32 * kk + 8 * g);
    }
    const float sc = a.scale * kLog2e;
    f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) dk[nb] = dv[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int q0 = 0; q0 < a.lq; q0 += kRows) {
        __syncthreads();
        {
            RowChunks<D> tq, tdo;
            tq.load(Q, q0);
            tdo.load(dO, q0);
            tq.store(s.q);
            tq.store(s.qr);
            tdo.store(s.d_o);
            tdo.store(s.dor);
        }
        if (threadIdx.x < kRows) {
            const int qq = q0 + threadIdx.x;
            s.lse2[threadIdx.x] = qq < a.lq ? a.lse[bh * a.lq + qq] * kLog2e : INFINITY;
            s.delta[threadIdx.x] = qq < a.lq ? a.delta[bh * a.lq + qq] : 0.0f;
        }
        __syncthreads();
        u32x2 pb[kRows / 16], dsb[kRows / 16];
#pragma unroll
        for (int qb = 0; qb < kRows / 16; ++qb) {
            // S = Q K^T and dP = dO V^T: lane holds [query 16 qb + 4 g + i][key r]
            f32x4 st = {0.f, 0.f, 0.f, 0.f}, dpt = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk) {
                st = mfma32(*reinterpret_cast<const u32x4*>(&s.q[16 * qb + r][32 * kk + 8 * g]), kb_[kk], st);
                dpt = mfma32(*reinterpret_cast<const u32x4*>(&s.d_o[16 * qb + r][32 * kk + 8 * g]), vb_[kk], dpt);
            }
            float p[4], ds[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int qi = 16 * qb + 4 * g + i;
                p[i] = exp2_hw(st[i] * sc - s.lse2[qi]);
                ds[i] = p[i] * (dpt[i] - s.delta[qi]);
            }
            pb[qb] = u32x2{pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            dsb[qb] = u32x2{pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
        }
        // dV^T += dO^T P and dK^T += Q^T dS over two 32-query halves
#pragma unroll
        for (int h = 0; h < kRows / 32; ++h) {
            const u32x4 pop = {pb[2 * h].x, pb[2 * h].y, pb[2 * h + 1].x, pb[2 * h + 1].y};
            const u32x4 dop = {dsb[2 * h].x, dsb[2 * h].y, dsb[2 * h + 1].x, dsb[2 * h + 1].y};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const int k0 = 32 * h + 4 * g, k1 = 32 * h + 16 + 4 * g;
                dv[nb] = mfma32(tr_pair(s.dor, k0, k1, 16 * nb, r), pop, dv[nb]);
                dk[nb] = mfma32(tr_pair(s.qr, k0, k1, 16 * nb, r), dop, dk[nb]);
            }
        }
    }
    if (!kv) return;
    float* dK = a.dk + (bh * lt + j) * D;
    float* dV = a.dv + (bh * lt + j) * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) {
        *reinterpret_cast<f32x4*>(dK + 16 * nb + 4 * g) = dk[nb] * a.scale;
        *reinterpret_cast<f32x4*>(dV + 16 * nb + 4 * g) = dv[nb];
    }
}

template <int D>
hipError_t launch_fwd(const AttnArgs& a, hipStream_t st) {
    dim3 grid((a.lq + kRows - 1) / kRows, a.heads, a.batch);
    hipLaunchKernelGGL(attn_fwd<D>, grid, dim3(kThreads), 0, st, a);
    return hipGetLastError();
}

template <int D>
hipError_t launch_bwd(const AttnArgs& a, hipStream_t st) {
    dim3 grid_q((a.lq + kRows - 1) / kRows, a.heads, a.batch);
    const int lt = a.src[1].rows;
    if (a.lq <= kRows && lt > 0) {
        // one workgroup holds every query of its (batch, head): dK and dV
        // come out of the same kernel
        hipLaunchKernelGGL((attn_bwd_dq<D, true>), grid_q, dim3(kThreads), 0, st, a);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((attn_bwd_dq<D, false>), grid_q, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (lt > 0) {
        dim3 grid_k((lt + kRows - 1) / kRows, a.heads, a.batch);
        hipLaunchKernelGGL(attn_bwd_dkdv<D>, grid_k, dim3(kThreads), 0, st, a);
        e = hipGetLastError();
    }
    return e;
}

}  // namespace

hipError_t launch_attention_forward(const AttnArgs& a, hipStream_t s) {
    return a.head_dim == 64 ? launch_fwd<64>(a, s) : launch_fwd<128>(a, s);
}

hipError_t launch_attention_backward(const AttnArgs& a, hipStream_t s) {
    return a.head_dim == 64 ? launch_bwd<64>(a, s) : launch_bwd<128>(a, s);
}

}  // namespace somaopt
