// Launch wrappers of the tiled attention kernels (defined in attention.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace somaopt {

struct AttnArgs {
    const void* q;       // bf16 [B][H][lq][D]
    const void* k;       // bf16 [B][H][lk][D]
    const void* v;       // bf16 [B][H][lk][D]
    void* o;             // bf16 [B][H][lq][D] (forward output; backward input)
    float* lse;          // fp32 [B][H][lq]   (forward output; backward input)
    const void* d_o;     // bf16 [B][H][lq][D] (backward)
    float* dq;           // fp32 [B][H][lq][D] (backward)
    float* dk;           // fp32 [B][H][lk - lk_frozen][D] (backward, trainable keys)
    float* dv;           // fp32 [B][H][lk - lk_frozen][D]
    float* delta;        // fp32 [B][H][lq] workspace: rowsum(dO * O)
    int32_t batch, heads, lq, lk, lk_frozen, head_dim;
    float scale;
};

hipError_t launch_attention_forward(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_backward(const AttnArgs& a, hipStream_t s);

}  // namespace somaopt
