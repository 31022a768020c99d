// Launch wrappers of the tiled attention kernels (defined in attention.hip).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace somaopt {

// One source of keys and values: for query batch b and head h the kernels
// read the bf16 [rows][D] matrices at
//   k + ((b / share) * heads + h) * stride * D   (and the same offset of v).
struct KeySrc {
    const void* k;
    const void* v;
    int32_t rows;     // keys per matrix, >= 0
    int32_t stride;   // rows between consecutive (batch, head) matrices
    int32_t share;    // consecutive query batches that read the same matrices, >= 1
};

// Keys are the concatenation of src[0] (frozen: no dK/dV) and src[1]
// (trainable: dK/dV written, one matrix per query batch).
struct AttnArgs {
    const void* q;       // bf16 [B][H][lq][D]
    void* o;             // bf16 [B][H][lq][D] (forward output; backward input)
    float* lse;          // fp32 [B][H][lq]   (forward output; backward input)
    const void* d_o;     // bf16 [B][H][lq][D] (backward)
    float* dq;           // fp32 [B][H][lq][D] (backward)
    float* dk;           // fp32 [B][H][src[1].rows][D] (backward)
    float* dv;           // fp32 [B][H][src[1].rows][D]
    float* delta;        // fp32 [B][H][lq] workspace: rowsum(dO * O)
    KeySrc src[2];
    int32_t batch, heads, lq, head_dim;
    float scale;
};

hipError_t launch_attention_forward(const AttnArgs& a, hipStream_t s);
hipError_t launch_attention_backward(const AttnArgs& a, hipStream_t s);

}  // namespace somaopt
