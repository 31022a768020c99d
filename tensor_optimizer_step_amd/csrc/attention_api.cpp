// C-ABI of the tiled attention kernels (declared in include/somaopt.h):
// shape and pointer validation, then stream-ordered launches.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdlib>
#include <cstring>
#include <string>

#include "attention.hpp"
#include "somaopt.h"

namespace somaopt {
// defined in somaopt.cpp
int set_error(int code, const std::string& msg);
}  // namespace somaopt

using namespace somaopt;

namespace {

// Rows per matrix are bounded so that every byte offset of a buffer
// resource (including the padding tiles past the end) fits in 31 bits.
constexpr int32_t kMaxRows = 1 << 22;

int check_common(int32_t batch, int32_t heads, int32_t lq, int32_t head_dim, float scale) {
    if (head_dim != 64 && head_dim != 128) return set_error(SOMAOPT_E_INVALID, "head_dim must be 64 or 128");
    if (batch < 1 || heads < 1 || batch > 65535 || heads > 65535)
        return set_error(SOMAOPT_E_INVALID, "batch and heads must be in [1, 65535]");
    if (lq < 1 || lq > kMaxRows) return set_error(SOMAOPT_E_INVALID, "lq must be in [1, 2^22]");
    if (!(scale == scale) || scale == 0.0f || scale - scale != 0.0f)
        return set_error(SOMAOPT_E_INVALID, "scale must be finite and nonzero");
    return SOMAOPT_OK;
}

int check_shape(const somaopt_attn_shape* s) {
    if (!s) return set_error(SOMAOPT_E_INVALID, "shape is NULL");
    int rc = check_common(s->batch, s->heads, s->lq, s->head_dim, s->scale);
    if (rc) return rc;
    if (s->lk < 1 || s->lk > kMaxRows) return set_error(SOMAOPT_E_INVALID, "lk must be in [1, 2^22]");
    if (s->lk_frozen < 0 || s->lk_frozen > s->lk) return set_error(SOMAOPT_E_INVALID, "lk_frozen outside [0, lk]");
    return SOMAOPT_OK;
}

int check_ctx_shape(const somaopt_attn_ctx_shape* s) {
    if (!s) return set_error(SOMAOPT_E_INVALID, "shape is NULL");
    int rc = check_common(s->batch, s->heads, s->lq, s->head_dim, s->scale);
    if (rc) return rc;
    if (s->l_ctx < 0 || s->l_ctx > kMaxRows || s->l_act < 0 || s->l_act > kMaxRows)
        return set_error(SOMAOPT_E_INVALID, "l_ctx and l_act must be in [0, 2^22]");
    if (s->l_ctx + s->l_act < 1) return set_error(SOMAOPT_E_INVALID, "l_ctx + l_act must be >= 1");
    if (s->ctx_share < 1 || s->batch % s->ctx_share != 0)
        return set_error(SOMAOPT_E_INVALID, "ctx_share must be >= 1 and divide batch");
    return SOMAOPT_OK;
}

// A buffer of `bytes` at `p`: non-NULL, aligned, device memory of the current
// device, inside one allocation.
int check_buffer(const void* p, size_t bytes, size_t align, const char* name) {
    if (!p) return set_error(SOMAOPT_E_INVALID, std::string(name) + " is NULL");
    if (reinterpret_cast<uintptr_t>(p) % align)
        return set_error(SOMAOPT_E_INVALID, std::string(name) + " is not " + std::to_string(align) + "-byte aligned");
    const char* skip = std::getenv("SOMAOPT_SKIP_POINTER_CHECK");
    if (skip && std::strcmp(skip, "1") == 0) return SOMAOPT_OK;
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) return set_error(SOMAOPT_E_HIP, "hipGetDevice failed");
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    if (hipPointerGetAttributes(&attr, p) != hipSuccess || attr.type != hipMemoryTypeDevice || attr.device != dev) {
        (void)hipGetLastError();
        return set_error(SOMAOPT_E_INVALID, std::string(name) + " is not device memory of the current device");
    }
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    if (hipMemGetAddressRange(&base, &size, const_cast<void*>(p)) != hipSuccess) {
        (void)hipGetLastError();
        return set_error(SOMAOPT_E_INVALID, std::string(name) + ": allocation range unknown to HIP");
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base), a = reinterpret_cast<uintptr_t>(p);
    if (a < lo || a + bytes > lo + size)
        return set_error(SOMAOPT_E_INVALID, std::string(name) + " runs past the end of its allocation");
    return SOMAOPT_OK;
}

AttnArgs base_args(int32_t batch, int32_t heads, int32_t lq, int32_t head_dim, float scale) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.batch = batch;
    a.heads = heads;
    a.lq = lq;
    a.head_dim = head_dim;
    a.scale = scale;
    return a;
}

// One buffer of lk keys per (batch, head): rows [0, lk_frozen) are source 0,
// rows [lk_frozen, lk) source 1, both with stride lk.
AttnArgs make_args(const somaopt_attn_shape* s, const void* k, const void* v) {
    AttnArgs a = base_args(s->batch, s->heads, s->lq, s->head_dim, s->scale);
    const size_t skip = (size_t)s->lk_frozen * s->head_dim * 2;
    a.src[0] = KeySrc{k, v, s->lk_frozen, s->lk, 1};
    a.src[1] = KeySrc{static_cast<const char*>(k) + skip, static_cast<const char*>(v) + skip, s->lk - s->lk_frozen,
                      s->lk, 1};
    return a;
}

// Separate context (shared by ctx_share consecutive query batches) and
// action buffers.  An empty source keeps a valid (unused) pointer.
AttnArgs make_ctx_args(const somaopt_attn_ctx_shape* s, const void* kc, const void* vc, const void* ka,
                       const void* va) {
    AttnArgs a = base_args(s->batch, s->heads, s->lq, s->head_dim, s->scale);
    a.src[0] = KeySrc{s->l_ctx ? kc : ka, s->l_ctx ? vc : va, s->l_ctx, s->l_ctx, s->ctx_share};
    a.src[1] = KeySrc{s->l_act ? ka : kc, s->l_act ? va : vc, s->l_act, s->l_act, 1};
    return a;
}

int launch_rc(hipError_t e, const char* what) {
    return e == hipSuccess ? SOMAOPT_OK : set_error(SOMAOPT_E_HIP, std::string(what) + ": " + hipGetErrorString(e));
}

}  // namespace

extern "C" {

int somaopt_attn_forward(const void* q, const void* k, const void* v, void* o, float* lse,
                         const somaopt_attn_shape* shape, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const size_t bh = (size_t)shape->batch * shape->heads, D = (size_t)shape->head_dim;
    const size_t nq = bh * shape->lq * D * 2, nk = bh * shape->lk * D * 2;
    if ((rc = check_buffer(q, nq, 16, "q")) || (rc = check_buffer(k, nk, 16, "k")) ||
        (rc = check_buffer(v, nk, 16, "v")) || (rc = check_buffer(o, nq, 16, "o")) ||
        (rc = check_buffer(lse, bh * shape->lq * 4, 4, "lse")))
        return rc;
    AttnArgs a = make_args(shape, k, v);
    a.q = q;
    a.o = o;
    a.lse = lse;
    return launch_rc(launch_attention_forward(a, static_cast<hipStream_t>(stream)), "attention forward launch");
}

int somaopt_attn_backward(const void* q, const void* k, const void* v, const void* o,
                          const float* lse, const void* d_o, float* dq, float* dk, float* dv,
                          float* delta, const somaopt_attn_shape* shape, void* stream) {
    int rc = check_shape(shape);
    if (rc) return rc;
    const size_t bh = (size_t)shape->batch * shape->heads, D = (size_t)shape->head_dim;
    const size_t nq = bh * shape->lq * D * 2, nk = bh * shape->lk * D * 2;
    const size_t lt = (size_t)(shape->lk - shape->lk_frozen);
    if ((rc = check_buffer(q, nq, 16, "q")) || (rc = check_buffer(k, nk, 16, "k")) ||
        (rc = check_buffer(v, nk, 16, "v")) || (rc = check_buffer(o, nq, 16, "o")) ||
        (rc = check_buffer(d_o, nq, 16, "d_o")) || (rc = check_buffer(lse, bh * shape->lq * 4, 4, "lse")) ||
        (rc = check_buffer(delta, bh * shape->lq * 4, 4, "delta")) ||
        (rc = check_buffer(dq, bh * shape->lq * D * 4, 16, "dq")))
        return rc;
    if (lt > 0 && ((rc = check_buffer(dk, bh * lt * D * 4, 16, "dk")) || (rc = check_buffer(dv, bh * lt * D * 4, 16, "dv"))))
        return rc;
    AttnArgs a = make_args(shape, k, v);
    a.q = q;
    a.o = const_cast<void*>(o);
    a.lse = const_cast<float*>(lse);
    a.d_o = d_o;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    return launch_rc(launch_attention_backward(a, static_cast<hipStream_t>(stream)), "attention backward launch");
}

int somaopt_attn_ctx_forward(const void* q, const void* k_ctx, const void* v_ctx, const void* k_act,
                             const void* v_act, void* o, float* lse, const somaopt_attn_ctx_shape* shape,
                             void* stream) {
    int rc = check_ctx_shape(shape);
    if (rc) return rc;
    const size_t bh = (size_t)shape->batch * shape->heads, D = (size_t)shape->head_dim;
    const size_t nq = bh * shape->lq * D * 2;
    const size_t nc = bh / shape->ctx_share * shape->l_ctx * D * 2, na = bh * shape->l_act * D * 2;
    if ((rc = check_buffer(q, nq, 16, "q")) || (rc = check_buffer(o, nq, 16, "o")) ||
        (rc = check_buffer(lse, bh * shape->lq * 4, 4, "lse")))
        return rc;
    if (shape->l_ctx && ((rc = check_buffer(k_ctx, nc, 16, "k_ctx")) || (rc = check_buffer(v_ctx, nc, 16, "v_ctx"))))
        return rc;
    if (shape->l_act && ((rc = check_buffer(k_act, na, 16, "k_act")) || (rc = check_buffer(v_act, na, 16, "v_act"))))
        return rc;
    AttnArgs a = make_ctx_args(shape, k_ctx, v_ctx, k_act, v_act);
    a.q = q;
    a.o = o;
    a.lse = lse;
    return launch_rc(launch_attention_forward(a, static_cast<hipStream_t>(stream)), "attention forward launch");
}

int somaopt_attn_ctx_backward(const void* q, const void* k_ctx, const void* v_ctx, const void* k_act,
                              const void* v_act, const void* o, const float* lse, const void* d_o, float* dq,
                              float* dk_act, float* dv_act, float* delta, const somaopt_attn_ctx_shape* shape,
                              void* stream) {
    int rc = check_ctx_shape(shape);
    if (rc) return rc;
    const size_t bh = (size_t)shape->batch * shape->heads, D = (size_t)shape->head_dim;
    const size_t nq = bh * shape->lq * D * 2;
    const size_t nc = bh / shape->ctx_share * shape->l_ctx * D * 2, na = bh * shape->l_act * D * 2;
    if ((rc = check_buffer(q, nq, 16, "q")) || (rc = check_buffer(o, nq, 16, "o")) ||
        (rc = check_buffer(d_o, nq, 16, "d_o")) || (rc = check_buffer(lse, bh * shape->lq * 4, 4, "lse")) ||
        (rc = check_buffer(delta, bh * shape->lq * 4, 4, "delta")) ||
        (rc = check_buffer(dq, bh * shape->lq * D * 4, 16, "dq")))
        return rc;
    if (shape->l_ctx && ((rc = check_buffer(k_ctx, nc, 16, "k_ctx")) || (rc = check_buffer(v_ctx, nc, 16, "v_ctx"))))
        return rc;
    if (shape->l_act && ((rc = check_buffer(k_act, na, 16, "k_act")) || (rc = check_buffer(v_act, na, 16, "v_act")) ||
                         (rc = check_buffer(dk_act, na * 2, 16, "dk_act")) ||
                         (rc = check_buffer(dv_act, na * 2, 16, "dv_act"))))
        return rc;
    AttnArgs a = make_ctx_args(shape, k_ctx, v_ctx, k_act, v_act);
    a.q = q;
    a.o = const_cast<void*>(o);
    a.lse = const_cast<float*>(lse);
    a.d_o = d_o;
    a.dq = dq;
    a.dk = dk_act;
    a.dv = dv_act;
    a.delta = delta;
    return launch_rc(launch_attention_backward(a, static_cast<hipStream_t>(stream)), "attention backward launch");
}

}  // extern "C"
