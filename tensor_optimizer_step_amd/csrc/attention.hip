// Tiled attention over frozen and trainable keys (gfx950, bf16 MFMA, fp32
// accumulation).
//
// SomaSpeed landing page, paragraph 5: queries from the trainable action
// computation read the context keys/values tile by tile, the full score
// matrix is never stored, and frozen inputs get no gradient work.  Here the
// first lk_frozen keys of every (batch, head) are frozen: the backward produces
// dQ for every query and dK/dV only for the trainable keys -- the frozen
// tiles cost three products per tile (S, dP, dQ) instead of five, and the
// dK/dV kernel is never launched over them.
//
// Layout: Q, K, V, O, dO are bf16 [B][H][L][D], rows contiguous; LSE and
// delta fp32 [B][H][Lq]; dQ fp32 [B][H][Lq][D]; dK, dV fp32 [B][H][Lk-Lf][D].
//
// Every workgroup is 4 waves; a wave owns 16 rows (queries, or keys in the
// dK/dV kernel).  MFMA operand layouts (16 lanes r = lane % 16, 4 groups
// g = lane / 16): for v_mfma_f32_16x16x32_bf16, lane holds A[r][8g..8g+7] and
// B[8g..8g+7][r]; for v_mfma_f32_16x16x16_bf16, A[r][4g..4g+3] and
// B[4g..4g+3][r]; both return C[4g+i][r], i = 0..3.  Computing S^T = K Q^T
// leaves each lane with four consecutive keys of one query -- exactly the
// operand P^T needs for O^T = V^T P^T -- so no register shuffles are needed
// between the two products, and each lane owns one query row's softmax state.
#include <hip/hip_runtime.h>

#include "attention.hpp"

namespace somaopt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kRows = 64;          // rows staged per tile (4 waves x 16)
constexpr int kThreads = 256;
constexpr int kPadRow = 8;         // bf16 padding of a row-major LDS row
constexpr int kPitchT = kRows + 4; // bf16 pitch of a transposed LDS row (8-byte aligned reads)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ f32x4 mfma32(const u32x4& a, const u32x4& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b),
                                                   c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16(const u32x2& a, const u32x2& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a), __builtin_bit_cast(s16x4, b),
                                                     c, 0, 0, 0);
}

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
           ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}
__device__ __forceinline__ float bf16_at(uint32_t w, int half) {
    return __uint_as_float(half ? (w & 0xffff0000u) : (w << 16));
}

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

__device__ __forceinline__ u32x4 load16(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }

// Rows [row0, row0 + 64) of a [L][D] bf16 matrix, as held by one thread
// between its global loads and its LDS stores (so the loads of the next tile
// can be in flight while the current tile is computed).  Rows at or past L
// are zero.
template <int D>
struct RowChunks {
    static constexpr int kChunks = D / 8;                    // 16-byte chunks per row
    static constexpr int kPer = kRows * kChunks / kThreads;  // chunks per thread
    u32x4 c[kPer];
    __device__ __forceinline__ void load(const uint16_t* src, int L, int row0) {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + kThreads * j;
            const int row = i / kChunks, col = (i % kChunks) * 8;
            c[j] = (row0 + row < L) ? load16(src + (size_t)(row0 + row) * D + col) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(uint16_t (*dst)[D + kPadRow]) const {
#pragma unroll
        for (int j = 0; j < kPer; ++j) {
            const int i = threadIdx.x + kThreads * j;
            *reinterpret_cast<u32x4*>(&dst[i / kChunks][(i % kChunks) * 8]) = c[j];
        }
    }
};

// The same rows for a transposed LDS tile dst[d][row]: thread t holds the row
// pair (2 (t % 32), 2 (t % 32) + 1) over D/8 consecutive columns and writes
// each column's pair as one 32-bit word.
template <int D>
struct PairChunks {
    static constexpr int kCols = D / 8;
    u32x4 a[kCols / 8], b[kCols / 8];
    __device__ __forceinline__ void load(const uint16_t* src, int L, int row0) {
        const int kp = threadIdx.x % 32, c0 = (threadIdx.x / 32) * kCols;
        const int ra = row0 + 2 * kp, rb = ra + 1;
#pragma unroll
        for (int j = 0; j < kCols / 8; ++j) {
            a[j] = (ra < L) ? load16(src + (size_t)ra * D + c0 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
            b[j] = (rb < L) ? load16(src + (size_t)rb * D + c0 + 8 * j) : u32x4{0u, 0u, 0u, 0u};
        }
    }
    // The same rows, row-major (no second global load of the tile).
    __device__ __forceinline__ void store_rows(uint16_t (*dst)[D + kPadRow]) const {
        const int kp = threadIdx.x % 32, c0 = (threadIdx.x / 32) * kCols;
#pragma unroll
        for (int j = 0; j < kCols / 8; ++j) {
            *reinterpret_cast<u32x4*>(&dst[2 * kp][c0 + 8 * j]) = a[j];
            *reinterpret_cast<u32x4*>(&dst[2 * kp + 1][c0 + 8 * j]) = b[j];
        }
    }
    __device__ __forceinline__ void store(uint16_t (*dst)[kPitchT]) const {
        const int kp = threadIdx.x % 32, c0 = (threadIdx.x / 32) * kCols;
#pragma unroll
        for (int j = 0; j < kCols / 8; ++j) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const uint32_t wa = a[j][e / 2], wb = b[j][e / 2];
                const uint32_t lo = (e & 1) ? (wa >> 16) : (wa & 0xffffu);
                const uint32_t hi = (e & 1) ? (wb & 0xffff0000u) : (wb << 16);
                *reinterpret_cast<uint32_t*>(&dst[c0 + 8 * j + e][2 * kp]) = lo | hi;
            }
        }
    }
};

template <int D>
__device__ __forceinline__ void stage_rows(const uint16_t* src, int L, int row0, uint16_t (*dst)[D + kPadRow]) {
    RowChunks<D> t;
    t.load(src, L, row0);
    t.store(dst);
}

template <int D>
__device__ __forceinline__ void stage_transposed(const uint16_t* src, int L, int row0, uint16_t (*dst)[kPitchT]) {
    PairChunks<D> t;
    t.load(src, L, row0);
    t.store(dst);
}

// ------------------------------------------------------------------ forward

template <int D>
struct FwdLds {
    uint16_t k[kRows][D + kPadRow];   // K tile, row-major
    uint16_t vt[D][kPitchT];          // V tile, transposed
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_fwd(AttnArgs a) {
    __shared__ FwdLds<D> s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const size_t bh = (size_t)blockIdx.z * a.heads + blockIdx.y;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + bh * a.lq * D;
    const uint16_t* K = static_cast<const uint16_t*>(a.k) + bh * a.lk * D;
    const uint16_t* V = static_cast<const uint16_t*>(a.v) + bh * a.lk * D;
    const int q = blockIdx.x * kRows + 16 * w + r;
    const bool qv = q < a.lq;
    // B operand of S^T = K Q^T: Q[q][32 kk + 8 g .. + 7]
    u32x4 qb[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk)
        qb[kk] = qv ? load16(Q + (size_t)q * D + 32 * kk + 8 * g) : u32x4{0u, 0u, 0u, 0u};
    const float sc = a.scale * kLog2e;   // scores in log2 units
    float m = -INFINITY, lsum = 0.0f;
    f32x4 acc[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) acc[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    // Products of one staged 64-key tile.
    auto tile = [&](int key0) {
#pragma unroll
        for (int kb = 0; kb < kRows / 16; ++kb) {
            f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
            for (int kk = 0; kk < D / 32; ++kk)
                st = mfma32(*reinterpret_cast<const u32x4*>(&s.k[16 * kb + r][32 * kk + 8 * g]), qb[kk], st);
            float x[4];
            float bm = -INFINITY;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int key = key0 + 16 * kb + 4 * g + i;
                x[i] = key < a.lk ? st[i] * sc : -INFINITY;
                bm = fmaxf(bm, x[i]);
            }
            bm = group_max(bm);
            const float mn = fmaxf(m, bm);
            const float alpha = exp2f(m - mn);   // m = -inf only before the first key
            m = mn;
            float p[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) p[i] = exp2f(x[i] - mn);
            lsum = lsum * alpha + (p[0] + p[1]) + (p[2] + p[3]);
            const u32x2 pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                acc[nb] *= alpha;
                const u32x2 va = *reinterpret_cast<const u32x2*>(&s.vt[16 * nb + r][16 * kb + 4 * g]);
                acc[nb] = mfma16(va, pb, acc[nb]);
            }
        }
    };
    // The next tile's global loads are issued before this tile's products,
    // so they overlap the MFMA work.
    RowChunks<D> kn;
    PairChunks<D> vn;
    kn.load(K, a.lk, 0);
    vn.load(V, a.lk, 0);
    for (int key0 = 0; key0 < a.lk; key0 += kRows) {
        __syncthreads();
        kn.store(s.k);
        vn.store(s.vt);
        __syncthreads();
        if (key0 + kRows < a.lk) {
            kn.load(K, a.lk, key0 + kRows);
            vn.load(V, a.lk, key0 + kRows);
        }
        tile(key0);
    }
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
    uint16_t k[kRows][D + kPadRow];   // K tile, row-major (A of S^T)
    uint16_t kt[D][kPitchT];          // K tile, transposed (A of dQ^T)
    uint16_t v[kRows][D + kPadRow];   // V tile, row-major (A of dP^T)
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dq(AttnArgs a) {
    __shared__ DqLds<D> s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const size_t bh = (size_t)blockIdx.z * a.heads + blockIdx.y;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + bh * a.lq * D;
    const uint16_t* dO = static_cast<const uint16_t*>(a.d_o) + bh * a.lq * D;
    const uint16_t* O = static_cast<const uint16_t*>(a.o) + bh * a.lq * D;
    const uint16_t* K = static_cast<const uint16_t*>(a.k) + bh * a.lk * D;
    const uint16_t* V = static_cast<const uint16_t*>(a.v) + bh * a.lk * D;
    const int q = blockIdx.x * kRows + 16 * w + r;
    const bool qv = q < a.lq;
    u32x4 qb[D / 32], db[D / 32];
    float dot = 0.0f;
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const size_t off = (size_t)q * D + 32 * kk + 8 * g;
        qb[kk] = qv ? load16(Q + off) : u32x4{0u, 0u, 0u, 0u};
        db[kk] = qv ? load16(dO + off) : u32x4{0u, 0u, 0u, 0u};
        const u32x4 ov = qv ? load16(O + off) : u32x4{0u, 0u, 0u, 0u};
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

    auto tile = [&](int key0) {
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
                const float p = key < a.lk ? exp2f(st[i] * sc - lse2) : 0.0f;
                ds[i] = p * (dpt[i] - delta);
            }
            const u32x2 dsb = {pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const u32x2 ka = *reinterpret_cast<const u32x2*>(&s.kt[16 * nb + r][16 * kb + 4 * g]);
                acc[nb] = mfma16(ka, dsb, acc[nb]);
            }
        }
    };
    // K is loaded once as row pairs and written both row-major and
    // transposed; the next tile's loads overlap this tile's products.
    PairChunks<D> kn;
    RowChunks<D> vn;
    kn.load(K, a.lk, 0);
    vn.load(V, a.lk, 0);
    for (int key0 = 0; key0 < a.lk; key0 += kRows) {
        __syncthreads();
        kn.store_rows(s.k);
        kn.store(s.kt);
        vn.store(s.v);
        __syncthreads();
        if (key0 + kRows < a.lk) {
            kn.load(K, a.lk, key0 + kRows);
            vn.load(V, a.lk, key0 + kRows);
        }
        tile(key0);
    }
    if (!qv) return;
    float* dQ = a.dq + bh * a.lq * D + (size_t)q * D;
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) *reinterpret_cast<f32x4*>(dQ + 16 * nb + 4 * g) = acc[nb] * a.scale;
}

// ------------------------------------------ backward: dK, dV of trainable keys

template <int D>
struct DkvLds {
    uint16_t q[kRows][D + kPadRow];    // Q chunk, row-major (A of S)
    uint16_t d_o[kRows][D + kPadRow];  // dO chunk, row-major (A of dP)
    uint16_t qt[D][kPitchT];           // Q chunk, transposed (A of dK^T)
    uint16_t dot[D][kPitchT];          // dO chunk, transposed (A of dV^T)
    float lse2[kRows];
    float delta[kRows];
};

template <int D>
__global__ __launch_bounds__(kThreads) void attn_bwd_dkdv(AttnArgs a) {
    __shared__ DkvLds<D> s;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int r = lane & 15, g = lane >> 4;
    const size_t bh = (size_t)blockIdx.z * a.heads + blockIdx.y;
    const int lt = a.lk - a.lk_frozen;
    const uint16_t* Q = static_cast<const uint16_t*>(a.q) + bh * a.lq * D;
    const uint16_t* dO = static_cast<const uint16_t*>(a.d_o) + bh * a.lq * D;
    const uint16_t* K = static_cast<const uint16_t*>(a.k) + bh * a.lk * D;
    const uint16_t* V = static_cast<const uint16_t*>(a.v) + bh * a.lk * D;
    const int j = blockIdx.x * kRows + 16 * w + r;   // trainable key index
    const bool kv = j < lt;
    const int key = a.lk_frozen + j;
    // B operands: K[key][32 kk + 8 g ..], V[key][32 kk + 8 g ..]
    u32x4 kb_[D / 32], vb_[D / 32];
#pragma unroll
    for (int kk = 0; kk < D / 32; ++kk) {
        const size_t off = (size_t)key * D + 32 * kk + 8 * g;
        kb_[kk] = kv ? load16(K + off) : u32x4{0u, 0u, 0u, 0u};
        vb_[kk] = kv ? load16(V + off) : u32x4{0u, 0u, 0u, 0u};
    }
    const float sc = a.scale * kLog2e;
    f32x4 dk[D / 16], dv[D / 16];
#pragma unroll
    for (int nb = 0; nb < D / 16; ++nb) dk[nb] = dv[nb] = f32x4{0.f, 0.f, 0.f, 0.f};

    for (int q0 = 0; q0 < a.lq; q0 += kRows) {
        __syncthreads();
        stage_rows<D>(Q, a.lq, q0, s.q);
        stage_rows<D>(dO, a.lq, q0, s.d_o);
        stage_transposed<D>(Q, a.lq, q0, s.qt);
        stage_transposed<D>(dO, a.lq, q0, s.dot);
        if (threadIdx.x < kRows) {
            const int qq = q0 + threadIdx.x;
            s.lse2[threadIdx.x] = qq < a.lq ? a.lse[bh * a.lq + qq] * kLog2e : INFINITY;
            s.delta[threadIdx.x] = qq < a.lq ? a.delta[bh * a.lq + qq] : 0.0f;
        }
        __syncthreads();
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
                p[i] = exp2f(st[i] * sc - s.lse2[qi]);
                ds[i] = p[i] * (dpt[i] - s.delta[qi]);
            }
            const u32x2 pb = {pack_bf16(p[0], p[1]), pack_bf16(p[2], p[3])};
            const u32x2 dsb = {pack_bf16(ds[0], ds[1]), pack_bf16(ds[2], ds[3])};
#pragma unroll
            for (int nb = 0; nb < D / 16; ++nb) {
                const u32x2 da = *reinterpret_cast<const u32x2*>(&s.dot[16 * nb + r][16 * qb + 4 * g]);
                const u32x2 qa = *reinterpret_cast<const u32x2*>(&s.qt[16 * nb + r][16 * qb + 4 * g]);
                dv[nb] = mfma16(da, pb, dv[nb]);    // dV^T += dO^T P
                dk[nb] = mfma16(qa, dsb, dk[nb]);   // dK^T += Q^T dS
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
    hipLaunchKernelGGL(attn_bwd_dq<D>, grid_q, dim3(kThreads), 0, st, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int lt = a.lk - a.lk_frozen;
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
