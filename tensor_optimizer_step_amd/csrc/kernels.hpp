// Launch wrappers of the gfx950 kernels (defined in kernels.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "plan.hpp"
#include "state.hpp"

namespace somaopt {

constexpr int kPass1Threads = 256;
constexpr int kPass2Threads = 256;
constexpr int kFinalizeThreads = 1024;
// Update pass: 4-element vectors per thread per batch (see update_segment).
constexpr int kVecsPerThread = 4;

// Norm-pass tables with more partials than this are reduced in two levels:
// kReduceSpan consecutive partials per workgroup, then the finalize.
constexpr uint32_t kTwoLevelAbove = 8192;
constexpr uint32_t kReduceSpan = 1024;
constexpr int kReduceThreads = 256;

struct Pass1Args {
    const Seg1* segs;
    const uint32_t* blk_first;   // n_blocks + 1 entries
    uint32_t n_blocks;           // >= 1
    double* partials;            // n_blocks entries, one per workgroup
    double* partials2;           // ceil(n_blocks / kReduceSpan) entries (two-level only)
    DevState* state;
    int32_t n_groups;
    int32_t advance;             // 1: this pass opens a new update (t += 1)
};

struct Pass2Args {
    const Seg2* segs;
    const uint32_t* blk_first;
    uint32_t n_blocks;           // >= 1
    const DevState* state;
};

hipError_t launch_pass1(const Pass1Args& a, hipStream_t s);
hipError_t launch_pass2(const Pass2Args& a, hipStream_t s);
hipError_t launch_set_groups(DevState* st, const GroupArgs& g, hipStream_t s);
hipError_t launch_set_clip(DevState* st, double max_norm, double grad_divisor, hipStream_t s);
hipError_t launch_set_step(DevState* st, int64_t step, int32_t n_groups, hipStream_t s);

}  // namespace somaopt
