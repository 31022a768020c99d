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

int check_shape(const somaopt_attn_shape* s) {
    if (!s) return set_error(SOMAOPT_E_INVALID, "shape is NULL");
    if (s->head_dim != 64 && s->head_dim != 128) return set_error(SOMAOPT_E_INVALID, "head_dim must be 64 or 128");
    if (s->batch < 1 || s->heads < 1 || s->batch > 65535 || s->heads > 65535)
        return set_error(SOMAOPT_E_INVALID, "batch and heads must be in [1, 65535]");
    if (s->lq < 1 || s->lk < 1) return set_error(SOMAOPT_E_INVALID, "lq and lk must be >= 1");
    if (s->lk_frozen < 0 || s->lk_frozen > s->lk) return set_error(SOMAOPT_E_INVALID, "lk_frozen outside [0, lk]");
    if (!(s->scale == s->scale) || s->scale == 0.0f) return set_error(SOMAOPT_E_INVALID, "scale must be finite and nonzero");
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

AttnArgs make_args(const somaopt_attn_shape* s) {
    AttnArgs a;
    std::memset(&a, 0, sizeof(a));
    a.batch = s->batch;
    a.heads = s->heads;
    a.lq = s->lq;
    a.lk = s->lk;
    a.lk_frozen = s->lk_frozen;
    a.head_dim = s->head_dim;
    a.scale = s->scale;
    return a;
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
    AttnArgs a = make_args(shape);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = o;
    a.lse = lse;
    hipError_t e = launch_attention_forward(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK
                           : set_error(SOMAOPT_E_HIP, std::string("attention forward launch: ") + hipGetErrorString(e));
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
    AttnArgs a = make_args(shape);
    a.q = q;
    a.k = k;
    a.v = v;
    a.o = const_cast<void*>(o);
    a.lse = const_cast<float*>(lse);
    a.d_o = d_o;
    a.dq = dq;
    a.dk = dk;
    a.dv = dv;
    a.delta = delta;
    hipError_t e = launch_attention_backward(a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK
                           : set_error(SOMAOPT_E_HIP, std::string("attention backward launch: ") + hipGetErrorString(e));
}

}  // extern "C"
