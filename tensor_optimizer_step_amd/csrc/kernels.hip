// gfx950 kernels of the fused clip + AdamW optimizer step.
//
// Pass 1 (norm pass): every workgroup streams the owned gradient segments of
// its block with 16-byte loads, squares and accumulates in fp64, reduces across
// the wavefront with DPP row permutes and across waves through LDS, and stores
// one partial per workgroup.  A one-workgroup finalize kernel then adds the
// partials in a fixed order (through one intermediate level of fixed-order
// workgroup sums for large tables), so the global sum is bitwise reproducible, and
// derives the norm, the clip coefficient and each group's bias-corrected
// constants on the device (no host synchronization).  SomaSpeed landing page,
// paragraph 8: the statistics for one global clip decision, with every
// gradient shard counted once.
//
// Pass 2 (update pass): a streaming elementwise kernel over every trainable
// segment that reads g, p, m, v and writes p, m, v in one pass, applying the
// effective-batch normalization, the clip coefficient and decoupled AdamW
// together from the unmodified gradients (same paragraph).  HBM-bound, so
// plain fp32 FMA arithmetic, no matrix cores.
//
// Arrival pass (the step before the path): rewrites every trainable gradient
// from the buffer whose already-reduced values arrive for it (copy, or fp32
// sum rounded once to the gradient dtype) and produces the norm pass's
// partials from the new values in the same sweep, so the norm needs no second
// read of the gradients.
#include <hip/hip_runtime.h>
#include <algorithm>

#include "kernels.hpp"

namespace somaopt {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// Address spaces: tensor data is global memory (global_load/store with a
// scalar base); the descriptor tables and the optimizer state are read through
// the constant space so that they arrive by scalar loads into SGPRs.
#define AS_GLOBAL __attribute__((address_space(1)))
#define AS_CONST __attribute__((address_space(4)))

template <typename T>
__device__ __forceinline__ AS_GLOBAL T* gptr(const void* p) {
    return (AS_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ const AS_CONST T* cptr(const void* p) {
    return (const AS_CONST T*)(p);
}
// Copy a table entry out of the constant space (scalar loads).  The host pass
// of the single-source compile cannot copy across address spaces and never
// runs this code, so it only sees a stand-in.
template <typename T>
__device__ __forceinline__ T cload(const AS_CONST T* p) {
#if defined(__HIP_DEVICE_COMPILE__)
    return *p;
#else
    (void)p;
    return T{};
#endif
}

// Exact widening of 16-bit gradients: bf16 is the top half of a binary32;
// binary16 converts exactly with the hardware conversion.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
__device__ __forceinline__ float bf16_one(uint16_t h) { return __uint_as_float((uint32_t)h << 16); }
__device__ __forceinline__ float f16_one(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

template <int DT>
__device__ __forceinline__ float widen16(uint16_t h) {
    if constexpr (DT == SOMAOPT_BF16) return bf16_one(h);
    else return f16_one(h);
}
template <int DT>
__device__ __forceinline__ float widen_lo(uint32_t w) {
    if constexpr (DT == SOMAOPT_BF16) return bf16_lo(w);
    else return f16_one((uint16_t)(w & 0xffffu));
}
template <int DT>
__device__ __forceinline__ float widen_hi(uint32_t w) {
    if constexpr (DT == SOMAOPT_BF16) return bf16_hi(w);
    else return f16_one((uint16_t)(w >> 16));
}

// Working copy of an fp32 master weight: round to nearest, ties to even.
template <int DT>
__device__ __forceinline__ uint16_t narrow16(float x) {
    if constexpr (DT == SOMAOPT_BF16) return __builtin_bit_cast(uint16_t, (__bf16)x);
    else return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// ---------------------------------------------------------------- reductions

// Move a double across lanes with one DPP control (applied to both halves).
template <int CTRL>
__device__ __forceinline__ double dpp_double(double x) {
    int lo = __double2loint(x);
    int hi = __double2hiint(x);
    lo = __builtin_amdgcn_update_dpp(0, lo, CTRL, 0xF, 0xF, false);
    hi = __builtin_amdgcn_update_dpp(0, hi, CTRL, 0xF, 0xF, false);
    return __hiloint2double(hi, lo);
}

__device__ __forceinline__ double readlane_double(double x, int lane) {
    int lo = __builtin_amdgcn_readlane(__double2loint(x), lane);
    int hi = __builtin_amdgcn_readlane(__double2hiint(x), lane);
    return __hiloint2double(hi, lo);
}

// Sum over the 64 lanes of a wavefront, identical in every lane, fixed order.
// Inside each 16-lane row: swap neighbours (quad_perm 1,0,3,2), swap pairs
// (quad_perm 2,3,0,1), mirror half-rows, mirror the row; then the four row
// sums are read from lanes 0, 16, 32, 48 and added as (r0 + r1) + (r2 + r3).
// Must be called with all 64 lanes active.
__device__ __forceinline__ double wave_sum(double x) {
    x += dpp_double<0xB1>(x);    // quad_perm [1,0,3,2]
    x += dpp_double<0x4E>(x);    // quad_perm [2,3,0,1]
    x += dpp_double<0x141>(x);   // row_half_mirror
    x += dpp_double<0x140>(x);   // row_mirror
    const double r0 = readlane_double(x, 0);
    const double r1 = readlane_double(x, 16);
    const double r2 = readlane_double(x, 32);
    const double r3 = readlane_double(x, 48);
    return (r0 + r1) + (r2 + r3);
}

// Workgroup sum (valid in thread 0); waves are added in index order.
template <int BS>
__device__ __forceinline__ double block_sum(double x, double* lds) {
    constexpr int kWaves = BS / 64;
    const double w = wave_sum(x);
    if ((threadIdx.x & 63) == 0) lds[threadIdx.x >> 6] = w;
    __syncthreads();
    double s = 0.0;
    if (threadIdx.x == 0) {
#pragma unroll
        for (int k = 0; k < kWaves; ++k) s += lds[k];
    }
    return s;
}

// ------------------------------------------------- buffer-instruction access

// Buffer resource over `bytes` bytes at `base` (raw addressing, stride 0):
// the hardware bounds-checks every access against the segment, so a load past
// the end returns zero and a store past it is dropped.  Word 3 selects the
// 32-bit data format that untyped buffer accesses require on gfx9-family parts.
constexpr int kRsrcWord3 = 0x00020000;
__device__ __forceinline__ __amdgpu_buffer_rsrc_t seg_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kRsrcWord3);
}
// Cache-policy operand of the streaming buffer accesses: nt (nontemporal).
// Every byte is used exactly once per step; on gfx950 the hint raises the
// sustained bandwidth of this 4-read / 3-write stream by about a tenth over
// plain accesses.
constexpr int kLdPolicy = 2;
constexpr int kStPolicy = 2;

__device__ __forceinline__ f32x4 bload4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kLdPolicy));
}
__device__ __forceinline__ u32x2 bload2(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_bit_cast(u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, (int)off, 0, kLdPolicy));
}
__device__ __forceinline__ void bstore4(__amdgpu_buffer_rsrc_t r, uint32_t off, const f32x4& x) {
    __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), r, (int)off, 0, kStPolicy);
}
__device__ __forceinline__ void bstore2(__amdgpu_buffer_rsrc_t r, uint32_t off, const u32x2& x) {
    __builtin_amdgcn_raw_buffer_store_b64(x, r, (int)off, 0, kStPolicy);
}

// ------------------------------------------------------------------ pass 1

// Sum of squares of one gradient segment: a scalar head (fewer elements than
// a 16-byte vector), a body of 16-byte vectors and a scalar tail.  The body is
// read through a buffer resource bounded by its own bytes, kPass1Batch vectors
// per thread per round with every load of a round issued before the first
// square (lanes past the end read zero, which adds an exact zero), so a short
// segment costs one memory latency however many vectors per thread it has up
// to kPass1Batch.  The head and tail elements are requested before the body
// through a resource bounded by the whole segment and squared after it.
constexpr int kPass1Batch = 4;
// Cache policy of the norm pass's loads: the default one.  Nontemporal loads
// here make the update pass that follows 6-7% slower on MI355X (measured in
// one process on the action expert and the 7B state), although the norm pass
// itself is no slower with them.
constexpr int kNormLdPolicy = 0;
// Descriptors fetched together by a workgroup of several segments (at most
// 8 with the default packing cost; later ones are fetched one by one).
constexpr int kPrefetchSegs = 8;
constexpr uint32_t kOutOfRange = 0x7fffffffu;   // a buffer offset past every segment

template <int DT>
__device__ __forceinline__ double widen_elem(uint32_t raw) {
    if constexpr (DT == SOMAOPT_F32) return __uint_as_float(raw);
    else return widen16<DT>((uint16_t)raw);
}

template <int DT>
__device__ __forceinline__ uint32_t bload_elem(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    if constexpr (DT == SOMAOPT_F32) return __builtin_amdgcn_raw_buffer_load_b32(r, (int)off, 0, kNormLdPolicy);
    else return __builtin_amdgcn_raw_buffer_load_b16(r, (int)off, 0, kNormLdPolicy);
}

template <int DT>
__device__ __forceinline__ void square_vec(const u32x4& q, double& a0, double& a1) {
    if constexpr (DT == SOMAOPT_F32) {
        double x;
        x = __uint_as_float(q.x); a0 = fma(x, x, a0);
        x = __uint_as_float(q.y); a1 = fma(x, x, a1);
        x = __uint_as_float(q.z); a0 = fma(x, x, a0);
        x = __uint_as_float(q.w); a1 = fma(x, x, a1);
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const double lo = widen_lo<DT>(q[k]);
            const double hi = widen_hi<DT>(q[k]);
            a0 = fma(lo, lo, a0);
            a1 = fma(hi, hi, a1);
        }
    }
}

template <int BS, int DT>
__device__ __forceinline__ void segment_sumsq_t(const Seg1& sg, int tid, double& a0, double& a1) {
    constexpr uint32_t esz = DT == SOMAOPT_F32 ? 4u : 2u;
    const char* g = static_cast<const char*>(sg.g);
    const uint32_t body = sg.head * esz;
    const uint32_t tail0 = body + 16u * sg.nvec;
    const __amdgpu_buffer_rsrc_t rs = seg_rsrc(g, tail0 + sg.tail * esz);
    const __amdgpu_buffer_rsrc_t rv = seg_rsrc(g + body, 16u * sg.nvec);
    // a head or a tail has fewer elements than a 16-byte vector: one per thread at most
    const uint32_t hraw = bload_elem<DT>(rs, (uint32_t)tid < sg.head ? tid * esz : kOutOfRange);
    const uint32_t traw = bload_elem<DT>(rs, (uint32_t)tid < sg.tail ? tail0 + tid * esz : kOutOfRange);
    for (uint32_t base = 0; base < sg.nvec; base += kPass1Batch * BS) {
        u32x4 q[kPass1Batch];
#pragma unroll
        for (int u = 0; u < kPass1Batch; ++u)
            q[u] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                                 rv, (int)(16u * (base + u * BS + tid)), 0, kNormLdPolicy));
        __builtin_amdgcn_sched_barrier(0);   // every load of the round before the first square
#pragma unroll
        for (int u = 0; u < kPass1Batch; ++u) square_vec<DT>(q[u], a0, a1);
    }
    const double h = widen_elem<DT>(hraw);
    const double t = widen_elem<DT>(traw);
    a0 = fma(h, h, a0);
    a1 = fma(t, t, a1);
}

template <int BS>
__device__ __forceinline__ void segment_sumsq(const Seg1& sg, int tid, double& a0, double& a1) {
    if (sg.dtype == SOMAOPT_BF16)
        segment_sumsq_t<BS, SOMAOPT_BF16>(sg, tid, a0, a1);
    else if (sg.dtype == SOMAOPT_F16)
        segment_sumsq_t<BS, SOMAOPT_F16>(sg, tid, a0, a1);
    else
        segment_sumsq_t<BS, SOMAOPT_F32>(sg, tid, a0, a1);
}

// Statistics of the pending update, computed once in fp64 by one thread.
__device__ void finalize_stats(DevState* st, double sumsq) {
    const double D = st->grad_divisor;
    const double M = st->max_norm;
    const double norm = sqrt(sumsq) / D;
    const double raw = M / (norm + 1e-6);
    const double coef = (raw > 1.0) ? 1.0 : raw;   // NaN stays NaN
    const double scale = coef / D;
    st->stats.sumsq = sumsq;
    st->stats.norm = norm;
    st->stats.clip_coef = coef;
    st->stats.grad_scale = scale;
    st->stats.nonfinite = isfinite(sumsq) ? 0 : 1;
    st->stats.n_groups = st->n_groups;
    st->grad_scale_f32 = (float)scale;
}

// beta^t for an integer t >= 0 by binary exponentiation in fp64: at most
// 2 log2(t) roundings, far below the fp32 rounding of the derived constants,
// and much shorter than a general power function on the critical path.
__device__ __forceinline__ double int_pow(double b, int64_t t) {
    double r = 1.0;
    while (t > 0) {
        if (t & 1) r *= b;
        b *= b;
        t >>= 1;
    }
    return r;
}

// The learning rate of update t under an on-device schedule (fp64); `lr` is
// the group's own value, used when the group has none.  The definitions are
// those of somaopt_set_schedules.
__device__ double scheduled_lr(const somaopt_schedule& s, int64_t t, double lr) {
    if (s.kind == SOMAOPT_SCHED_NONE) return lr;
    const int64_t w = s.kind == SOMAOPT_SCHED_COSINE ? 0 : s.warmup;   // >= 1 for the warm-up kinds
    if (s.kind == SOMAOPT_SCHED_LINEAR_WARMUP || (w > 0 && t <= w)) {
        const int64_t tt = t < w ? (t < 0 ? 0 : t) : w;
        return s.peak_lr * (double)tt / (double)w;
    }
    const int64_t span = s.total - w;
    int64_t k = t - w - 1;
    k = k < 0 ? 0 : (k > span ? span : k);
    return s.floor_lr + (s.peak_lr - s.floor_lr) * 0.5 * (1.0 + cos(M_PI * (double)k / (double)span));
}

// Group k's update count and bias-corrected constants (fp64, rounded once).
__device__ void finalize_group(DevState* st, int k, int advance) {
    int64_t t = st->step[k];
    if (advance) {
        t += 1;
        st->step[k] = t;
    }
    const somaopt_group h = st->hyper[k];
    const double lr = scheduled_lr(st->sched[k], t, h.lr);
    const double bc1 = 1.0 - int_pow(h.beta1, t);
    const double bc2 = 1.0 - int_pow(h.beta2, t);
    GroupConst c;
    c.step_size = (float)(lr / bc1);
    c.inv_sqrt_bc2 = (float)(1.0 / sqrt(bc2));
    c.lr_wd = (float)(lr * h.weight_decay);
    c.beta1 = (float)h.beta1;
    c.one_minus_beta1 = (float)(1.0 - h.beta1);
    c.beta2 = (float)h.beta2;
    c.one_minus_beta2 = (float)(1.0 - h.beta2);
    c.eps = (float)h.eps;
    st->gconst[k] = c;
}

template <int BS>
__global__ __launch_bounds__(BS) void sqnorm_pass1(Pass1Args a) {
    __shared__ double lds[BS / 64];
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const AS_CONST uint32_t* blk = cptr<uint32_t>(a.blk_first);
    const AS_CONST Seg1* segs = cptr<Seg1>(a.segs);
    const uint32_t s0 = blk[b];
    const uint32_t s1 = blk[b + 1];
    double a0 = 0.0, a1 = 0.0;
    if (s1 == s0 + 1) {
        segment_sumsq<BS>(cload(segs + s0), tid, a0, a1);
    } else if (s1 > s0) {
        // Several short segments: every descriptor of the block is requested
        // at once (scalar loads complete in any order, so a descriptor
        // fetched per segment would cost one wait each), then the segments
        // are read from registers.
        const uint32_t ns = s1 - s0;
        Seg1 d[kPrefetchSegs];
#pragma unroll
        for (int j = 0; j < kPrefetchSegs; ++j) d[j] = cload(segs + s0 + min((uint32_t)j, ns - 1));
#pragma unroll
        for (int j = 0; j < kPrefetchSegs; ++j)
            if ((uint32_t)j < ns) segment_sumsq<BS>(d[j], tid, a0, a1);
        for (uint32_t s = s0 + kPrefetchSegs; s < s1; ++s) segment_sumsq<BS>(cload(segs + s), tid, a0, a1);
    }
    const double part = block_sum<BS>(a0 + a1, lds);
    if (tid == 0) a.partials[b] = part;
}

// Fixed-order sum of n doubles by one workgroup (valid in thread 0): thread t
// adds elements t, t + BS, t + 2 BS, ... in increasing order, then the fixed
// wave/LDS tree.  Sixteen loads go out together; positions past n add an
// exact zero, so a thread with fewer than sixteen elements (every thread of
// the first-level reduction, which sums 1024 partials with 256 threads) still
// waits for one memory latency rather than one per element.
template <int BS>
__device__ __forceinline__ double fixed_order_sum(const AS_GLOBAL double* part, uint32_t n, double* lds) {
    constexpr int kLoads = 16;
    const uint32_t tid = threadIdx.x;
    double acc = 0.0;
    for (uint32_t i = tid; i < n; i += kLoads * BS) {
        double x[kLoads];
#pragma unroll
        for (int k = 0; k < kLoads; ++k) {
            const uint32_t j = i + k * BS;
            x[k] = j < n ? part[j] : 0.0;
        }
#pragma unroll
        for (int k = 0; k < kLoads; ++k) acc += x[k];
    }
    return block_sum<BS>(acc, lds);
}

// First level for large tables: workgroup j sums partials
// [j * kReduceSpan, (j + 1) * kReduceSpan) in fixed order.
template <int BS>
__global__ __launch_bounds__(BS) void reduce_partials(Pass1Args a) {
    __shared__ double lds[BS / 64];
    const uint32_t j = blockIdx.x;
    const uint32_t first = j * kReduceSpan;
    const uint32_t n = min(kReduceSpan, a.n_blocks - first);
    const double s = fixed_order_sum<BS>(gptr<double>(a.partials) + first, n, lds);
    if (threadIdx.x == 0) a.partials2[j] = s;
}

// One workgroup: fixed-order sum of the (first- or second-level) partials,
// then the statistics and the per-group constants of the pending update.  The
// kernel boundary after the norm pass makes every partial visible without any
// cache maintenance.
template <int BS>
__global__ __launch_bounds__(BS) void sqnorm_finalize(Pass1Args a) {
    __shared__ double lds[BS / 64];
    const int tid = threadIdx.x;
    const bool two = a.n_blocks > kTwoLevelAbove;
    const double* src = two ? a.partials2 : a.partials;
    const uint32_t n = two ? (a.n_blocks + kReduceSpan - 1) / kReduceSpan : a.n_blocks;
    const double total = fixed_order_sum<BS>(gptr<double>(src), n, lds);
    if (tid == 0) finalize_stats(a.state, total);
    if (tid < a.n_groups) finalize_group(a.state, tid, a.advance);
}

// ------------------------------------------------------------------ pass 2

// One element of the fused update: normalize + clip (scale = c / D), AdamW
// moments, bias-corrected step, decoupled decay of the pre-update weight.
// p is written as p + (-lr*wd*p - u) with the bracket in one fma, so the
// weight takes a single rounding at its own scale.
__device__ __forceinline__ void adamw_elem(float& p, float& m, float& v, float g, const GroupConst& c,
                                           float scale) {
    const float gh = g * scale;
    m = fmaf(c.beta1, m, c.one_minus_beta1 * gh);
    v = fmaf(c.beta2, v, (c.one_minus_beta2 * gh) * gh);
    const float denom = fmaf(sqrtf(v), c.inv_sqrt_bc2, c.eps);
    const float u = c.step_size * (m / denom);
    p = p + fmaf(-c.lr_wd, p, -u);
}

__device__ __forceinline__ void adamw_vec(f32x4& p, f32x4& m, f32x4& v, const f32x4& g,
                                          const GroupConst& c, float scale) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float pk = p[k], mk = m[k], vk = v[k];
        adamw_elem(pk, mk, vk, g[k], c, scale);
        p[k] = pk;
        m[k] = mk;
        v[k] = vk;
    }
}

template <int GDT>
__device__ __forceinline__ float load_g1(const AS_GLOBAL char* gbase, size_t i) {
    if constexpr (GDT == SOMAOPT_F32) return ((const AS_GLOBAL float*)gbase)[i];
    else return widen16<GDT>(((const AS_GLOBAL uint16_t*)gbase)[i]);
}

template <int LDT>
__device__ __forceinline__ u32x2 narrow4(const f32x4& p) {
    u32x2 r;
    r.x = (uint32_t)narrow16<LDT>(p.x) | ((uint32_t)narrow16<LDT>(p.y) << 16);
    r.y = (uint32_t)narrow16<LDT>(p.z) | ((uint32_t)narrow16<LDT>(p.w) << 16);
    return r;
}

constexpr int kNoLowp = -1;

template <int GDT>
__device__ __forceinline__ f32x4 widen_g4_buf(__amdgpu_buffer_rsrc_t r, uint32_t i) {
    if constexpr (GDT == SOMAOPT_F32) {
        return bload4(r, 16u * i);
    } else {
        const u32x2 w = bload2(r, 8u * i);
        f32x4 x;
        x.x = widen_lo<GDT>(w.x);
        x.y = widen_hi<GDT>(w.x);
        x.z = widen_lo<GDT>(w.y);
        x.w = widen_hi<GDT>(w.y);
        return x;
    }
}

// One segment of the update pass.  Each thread takes kVecsPerThread vectors
// spaced BS apart and issues all of their loads before any arithmetic, so a
// wave keeps 4 x (3 x 16 + 8 or 16) bytes per lane in flight; a segment of at
// most BS * kVecsPerThread vectors is a single batch.  The vector body goes
// through buffer instructions with one resource per array and segment: the
// addresses are a 32-bit lane offset on a scalar base, and lanes past the end
// of the body need no branch (their loads read zero, their stores are
// dropped).  GDT is the gradient dtype, LDT the working-copy dtype (kNoLowp:
// none).
template <int BS, int GDT, int LDT>
__device__ __forceinline__ void update_segment(const Seg2& sg, const GroupConst& c, float scale, int tid) {
    constexpr int U = kVecsPerThread;
    constexpr uint32_t kGsz = GDT == SOMAOPT_F32 ? 4 : 2;
    AS_GLOBAL float* p = gptr<float>(sg.p);
    AS_GLOBAL float* m = gptr<float>(sg.m);
    AS_GLOBAL float* v = gptr<float>(sg.v);
    const AS_GLOBAL char* gb = gptr<char>(sg.g);
    AS_GLOBAL uint16_t* lp = gptr<uint16_t>(sg.lowp);
    // Scalar head: a few elements before the first aligned vector, or the
    // whole segment when p, m, v, g (and the working copy) share no alignment.
    for (uint32_t k = tid; k < sg.head; k += BS) {
        float pp = p[k], mm = m[k], vq = v[k];
        adamw_elem(pp, mm, vq, load_g1<GDT>(gb, k), c, scale);
        p[k] = pp;
        m[k] = mm;
        v[k] = vq;
        if constexpr (LDT != kNoLowp) lp[k] = narrow16<LDT>(pp);
    }
    const uint32_t nvec = sg.nvec;
    const __amdgpu_buffer_rsrc_t rp = seg_rsrc((const void*)(p + sg.head), 16u * nvec);
    const __amdgpu_buffer_rsrc_t rm = seg_rsrc((const void*)(m + sg.head), 16u * nvec);
    const __amdgpu_buffer_rsrc_t rv = seg_rsrc((const void*)(v + sg.head), 16u * nvec);
    const __amdgpu_buffer_rsrc_t rg = seg_rsrc((const void*)(gb + sg.head * kGsz), 4u * kGsz * nvec);
    __amdgpu_buffer_rsrc_t rl;
    bool pair16 = false;
    if constexpr (LDT != kNoLowp) {
        rl = seg_rsrc((const void*)(lp + sg.head), 8u * nvec);
        pair16 = ((uintptr_t)(lp + sg.head) & 15u) == 0;
    }
    for (uint32_t base = 0; base < nvec; base += BS * U) {
        f32x4 pr[U], mr[U], vr[U], gr[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = base + u * BS + tid;
            pr[u] = bload4(rp, 16u * i);
            mr[u] = bload4(rm, 16u * i);
            vr[u] = bload4(rv, 16u * i);
            gr[u] = widen_g4_buf<GDT>(rg, i);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const uint32_t i = base + u * BS + tid;
            adamw_vec(pr[u], mr[u], vr[u], gr[u], c, scale);
            bstore4(rp, 16u * i, pr[u]);
            bstore4(rm, 16u * i, mr[u]);
            bstore4(rv, 16u * i, vr[u]);
        }
        if constexpr (LDT != kNoLowp) {
            // Working copy, after the fp32 stores.  Lanes 2j and 2j + 1 hold
            // adjacent vectors, so where the copy's vector body is 16-byte
            // aligned the even lane writes both halves (8 narrowed values)
            // with one 16-byte store, 2% faster than an 8-byte store per lane;
            // a last vector without a partner (odd vector count) is written
            // alone.
            if (pair16) {
#pragma unroll
                for (int u = 0; u < U; ++u) {
                    const uint32_t i = base + u * BS + tid;
                    const u32x2 w = narrow4<LDT>(pr[u]);
                    const uint32_t nx = (uint32_t)__shfl_xor((int)w.x, 1);
                    const uint32_t ny = (uint32_t)__shfl_xor((int)w.y, 1);
                    if ((tid & 1) == 0) {
                        if (i + 1 < nvec)
                            __builtin_amdgcn_raw_buffer_store_b128(u32x4{w.x, w.y, nx, ny}, rl, (int)(8u * i), 0,
                                                                   kStPolicy);
                        else
                            bstore2(rl, 8u * i, w);
                    }
                }
            } else {
#pragma unroll
                for (int u = 0; u < U; ++u) bstore2(rl, 8u * (base + u * BS + tid), narrow4<LDT>(pr[u]));
            }
        }
    }
    if ((uint32_t)tid < sg.tail) {
        const size_t k = sg.head + 4 * (size_t)nvec + tid;
        float pp = p[k], mm = m[k], vq = v[k];
        adamw_elem(pp, mm, vq, load_g1<GDT>(gb, k), c, scale);
        p[k] = pp;
        m[k] = mm;
        v[k] = vq;
        if constexpr (LDT != kNoLowp) lp[k] = narrow16<LDT>(pp);
    }
}

template <int BS, int GDT>
__device__ __forceinline__ void update_segment_any(const Seg2& sg, const GroupConst& c, float scale, int tid) {
    if (sg.lowp == nullptr)
        update_segment<BS, GDT, kNoLowp>(sg, c, scale, tid);
    else if (sg.lowp_dtype == SOMAOPT_BF16)
        update_segment<BS, GDT, SOMAOPT_BF16>(sg, c, scale, tid);
    else
        update_segment<BS, GDT, SOMAOPT_F16>(sg, c, scale, tid);
}

template <int BS>
__global__ __launch_bounds__(BS) void adamw_pass2(Pass2Args a) {
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const AS_CONST DevState* st = cptr<DevState>(a.state);
    const AS_CONST uint32_t* blk = cptr<uint32_t>(a.blk_first);
    const AS_CONST Seg2* segs = cptr<Seg2>(a.segs);
    const float scale = st->grad_scale_f32;
    const uint32_t s0 = blk[b];
    const uint32_t s1 = blk[b + 1];
    for (uint32_t s = s0; s < s1; ++s) {
        const Seg2 sg = cload(segs + s);
        const GroupConst c = cload(&st->gconst[sg.group]);
        if (sg.dtype == SOMAOPT_BF16)
            update_segment_any<BS, SOMAOPT_BF16>(sg, c, scale, tid);
        else if (sg.dtype == SOMAOPT_F16)
            update_segment_any<BS, SOMAOPT_F16>(sg, c, scale, tid);
        else
            update_segment_any<BS, SOMAOPT_F32>(sg, c, scale, tid);
    }
}

// ------------------------------------------------------------------ arrival

// Cache policy of the arrival pass's gradient stores: sc1, written through to
// memory.  Measured on MI355X (302M-element action expert, bf16 gradients):
// with nontemporal or plain stores the rewritten gradients linger dirty in the
// 256 MB memory-side cache and the update pass that follows pays for their
// write-back (1.29-1.34 ms instead of 1.20 ms); written through, arrival plus
// update take 1.53 ms per step against 1.60-1.65 ms.
constexpr int kArrivalStorePolicy = 16;

// One arriving 16-bit value: the fp32 sum with the held value, rounded once
// to the storage dtype (nearest, ties to even), or the arriving bits as they
// are when nothing is accumulated.
template <int DT>
__device__ __forceinline__ uint16_t arrive16(uint16_t held, uint16_t inc) {
    return narrow16<DT>(widen16<DT>(held) + widen16<DT>(inc));
}
template <int DT>
__device__ __forceinline__ uint32_t arrive_word(uint32_t held, uint32_t inc) {
    const uint16_t lo = narrow16<DT>(widen_lo<DT>(held) + widen_lo<DT>(inc));
    const uint16_t hi = narrow16<DT>(widen_hi<DT>(held) + widen_hi<DT>(inc));
    return (uint32_t)lo | ((uint32_t)hi << 16);
}

// Arrival over one 16-bit-gradient segment; squares of the stored values are
// accumulated in fp64 when the segment is owned.
template <int BS, int DT>
__device__ __forceinline__ void arrive16_segment(const Seg3& sg, int tid, bool acc, double& a0, double& a1) {
    AS_GLOBAL uint16_t* g = gptr<uint16_t>(sg.g);
    const AS_GLOBAL uint16_t* in = gptr<uint16_t>(sg.inc);
    const bool own = sg.owner != 0;
    for (uint32_t k = tid; k < sg.head; k += BS) {
        const uint16_t x = acc ? arrive16<DT>(g[k], in[k]) : in[k];
        g[k] = x;
        if (own) {
            const double w = widen16<DT>(x);
            a0 = fma(w, w, a0);
        }
    }
    const __amdgpu_buffer_rsrc_t rg = seg_rsrc((const void*)(g + sg.head), 16u * sg.nvec);
    const __amdgpu_buffer_rsrc_t ri = seg_rsrc((const void*)(in + sg.head), 16u * sg.nvec);
#pragma unroll 2
    for (uint32_t i = tid; i < sg.nvec; i += BS) {
        u32x4 x = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(ri, (int)(16u * i), 0, kLdPolicy));
        if (acc) {
            const u32x4 h = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, (int)(16u * i), 0, kLdPolicy));
#pragma unroll
            for (int k = 0; k < 4; ++k) x[k] = arrive_word<DT>(h[k], x[k]);
        }
        __builtin_amdgcn_raw_buffer_store_b128(x, rg, (int)(16u * i), 0, kArrivalStorePolicy);
        if (own) {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const double lo = widen_lo<DT>(x[k]);
                const double hi = widen_hi<DT>(x[k]);
                a0 = fma(lo, lo, a0);
                a1 = fma(hi, hi, a1);
            }
        }
    }
    if ((uint32_t)tid < sg.tail) {
        const size_t k = sg.head + 8 * (size_t)sg.nvec + tid;
        const uint16_t x = acc ? arrive16<DT>(g[k], in[k]) : in[k];
        g[k] = x;
        if (own) {
            const double w = widen16<DT>(x);
            a1 = fma(w, w, a1);
        }
    }
}

template <int BS>
__device__ __forceinline__ void arrive32_segment(const Seg3& sg, int tid, bool acc, double& a0, double& a1) {
    AS_GLOBAL float* g = gptr<float>(sg.g);
    const AS_GLOBAL float* in = gptr<float>(sg.inc);
    const bool own = sg.owner != 0;
    for (uint32_t k = tid; k < sg.head; k += BS) {
        const float x = acc ? g[k] + in[k] : in[k];
        g[k] = x;
        if (own) a0 = fma((double)x, (double)x, a0);
    }
    const __amdgpu_buffer_rsrc_t rg = seg_rsrc((const void*)(g + sg.head), 16u * sg.nvec);
    const __amdgpu_buffer_rsrc_t ri = seg_rsrc((const void*)(in + sg.head), 16u * sg.nvec);
#pragma unroll 2
    for (uint32_t i = tid; i < sg.nvec; i += BS) {
        f32x4 x = bload4(ri, 16u * i);
        if (acc) x = bload4(rg, 16u * i) + x;
        __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, x), rg, (int)(16u * i), 0,
                                               kArrivalStorePolicy);
        if (own) {
            double w;
            w = x.x; a0 = fma(w, w, a0);
            w = x.y; a1 = fma(w, w, a1);
            w = x.z; a0 = fma(w, w, a0);
            w = x.w; a1 = fma(w, w, a1);
        }
    }
    if ((uint32_t)tid < sg.tail) {
        const size_t k = sg.head + 4 * (size_t)sg.nvec + tid;
        const float x = acc ? g[k] + in[k] : in[k];
        g[k] = x;
        if (own) a1 = fma((double)x, (double)x, a1);
    }
}

template <int BS>
__global__ __launch_bounds__(BS) void arrival_pass(Pass3Args a) {
    __shared__ double lds[BS / 64];
    const int tid = threadIdx.x;
    const uint32_t b = blockIdx.x;
    const AS_CONST uint32_t* blk = cptr<uint32_t>(a.blk_first);
    const AS_CONST Seg3* segs = cptr<Seg3>(a.segs);
    const bool acc = a.accumulate != 0;
    const uint32_t s0 = blk[b];
    const uint32_t s1 = blk[b + 1];
    double a0 = 0.0, a1 = 0.0;
    for (uint32_t s = s0; s < s1; ++s) {
        const Seg3 sg = cload(segs + s);
        if (sg.dtype == SOMAOPT_BF16)
            arrive16_segment<BS, SOMAOPT_BF16>(sg, tid, acc, a0, a1);
        else if (sg.dtype == SOMAOPT_F16)
            arrive16_segment<BS, SOMAOPT_F16>(sg, tid, acc, a0, a1);
        else
            arrive32_segment<BS>(sg, tid, acc, a0, a1);
    }
    const double part = block_sum<BS>(a0 + a1, lds);
    if (tid == 0) a.partials[b] = part;
}

// ------------------------------------------------------------- small setters

__global__ void set_groups_kernel(DevState* st, GroupArgs g) {
    const int k = threadIdx.x;
    if (k < g.n) st->hyper[k] = g.g[k];
}

__global__ void set_schedules_kernel(DevState* st, ScheduleArgs a) {
    const int k = threadIdx.x;
    if (k < a.n) st->sched[k] = a.s[k];
}

__global__ void set_clip_kernel(DevState* st, double max_norm, double grad_divisor) {
    if (threadIdx.x == 0) {
        st->max_norm = max_norm;
        st->grad_divisor = grad_divisor;
    }
}

__global__ void set_step_kernel(DevState* st, int64_t step, int32_t n) {
    const int k = threadIdx.x;
    if (k < n) st->step[k] = step;
}

}  // namespace

hipError_t launch_reduce_finalize(const Pass1Args& a, hipStream_t s);

hipError_t launch_pass1(const Pass1Args& a, hipStream_t s) {
    hipLaunchKernelGGL(sqnorm_pass1<kPass1Threads>, dim3(a.n_blocks), dim3(kPass1Threads), a.lds_bytes, s, a);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    return launch_reduce_finalize(a, s);
}

// Fixed-order reduction of the per-workgroup partials and the finalize.
hipError_t launch_reduce_finalize(const Pass1Args& a, hipStream_t s) {
    if (a.n_blocks > kTwoLevelAbove) {
        const uint32_t groups = (a.n_blocks + kReduceSpan - 1) / kReduceSpan;
        hipLaunchKernelGGL(reduce_partials<kReduceThreads>, dim3(groups), dim3(kReduceThreads), 0, s, a);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(sqnorm_finalize<kFinalizeThreads>, dim3(1), dim3(kFinalizeThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_pass3(const Pass3Args& a, uint32_t per_launch, hipStream_t s) {
    const uint32_t per = per_launch == 0 ? a.n_blocks : per_launch;
    for (uint32_t first = 0; first < a.n_blocks; first += per) {
        // workgroups [first, first + n) read blk_first[first .. first + n]
        // and write partials[first .. first + n)
        Pass3Args x = a;
        x.blk_first = a.blk_first + first;
        x.partials = a.partials + first;
        x.n_blocks = std::min(per, a.n_blocks - first);
        hipLaunchKernelGGL(arrival_pass<kPass1Threads>, dim3(x.n_blocks), dim3(kPass1Threads), x.lds_bytes, s, x);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    Pass1Args r;
    r.segs = nullptr;
    r.blk_first = nullptr;
    r.n_blocks = a.n_blocks;
    r.partials = a.partials;
    r.partials2 = a.partials2;
    r.state = a.state;
    r.n_groups = a.n_groups;
    r.advance = a.advance;
    r.lds_bytes = 0;
    return launch_reduce_finalize(r, s);
}

hipError_t launch_pass2(const Pass2Args& a, hipStream_t s) {
    hipLaunchKernelGGL(adamw_pass2<kPass2Threads>, dim3(a.n_blocks), dim3(kPass2Threads), a.lds_bytes, s, a);
    return hipGetLastError();
}

hipError_t launch_set_groups(DevState* st, const GroupArgs& g, hipStream_t s) {
    hipLaunchKernelGGL(set_groups_kernel, dim3(1), dim3(SOMAOPT_MAX_GROUPS), 0, s, st, g);
    return hipGetLastError();
}

hipError_t launch_set_schedules(DevState* st, const ScheduleArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(set_schedules_kernel, dim3(1), dim3(SOMAOPT_MAX_GROUPS), 0, s, st, a);
    return hipGetLastError();
}

hipError_t launch_set_clip(DevState* st, double max_norm, double grad_divisor, hipStream_t s) {
    hipLaunchKernelGGL(set_clip_kernel, dim3(1), dim3(64), 0, s, st, max_norm, grad_divisor);
    return hipGetLastError();
}

hipError_t launch_set_step(DevState* st, int64_t step, int32_t n_groups, hipStream_t s) {
    hipLaunchKernelGGL(set_step_kernel, dim3(1), dim3(SOMAOPT_MAX_GROUPS), 0, s, st, step, n_groups);
    return hipGetLastError();
}

}  // namespace somaopt
