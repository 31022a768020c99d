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

// Resident workgroups per compute unit.  Both streaming passes use no LDS for
// data; a launch reserves a share of the CU's LDS so that no more than this
// many workgroups are resident at once.  Measured on MI355X:
//  - tables of large tensors (a workgroup streams one full segment): the
//    4-read / 3-write update stream sustains its highest HBM bandwidth with
//    about 114 KB of loads in flight per CU: two 256-thread workgroups per CU
//    over 4096-element segments were about 10% above the
//    unrestricted occupancy of five, because fewer concurrent streams keep
//    DRAM rows open longer; four per CU over the half-length segments of
//    kStreamingPass2Chunk (the same bytes in flight) are another 1.5% faster
//    at 7B scale (three or more per CU over 4096 elements: 8-9% slower); the
//    read-only norm pass prefers six (7% faster on 7B-scale state);
//  - tables of many small tensors (a workgroup walks several short segments,
//    each starting with dependent descriptor loads): the update pass needs
//    four per CU to hide those latencies, and the norm pass no limit.
constexpr int kPass1WgPerCuStreaming = 6;
// The arrival pass over a streaming table (4096-element segments,
// kStreamingPass3Chunk): no limit when it copies the arriving values (one
// read, one write per element), six per CU when it accumulates (two reads,
// one write).  Measured on MI355X, 6.7e9 bf16 gradients: accumulated 6.25 ms
// at six, 6.71 at eight, 6.83 unlimited, 7.38 at four; copied 4.04 ms
// unlimited, 4.13 at eight, 4.32 at six.  302M elements: accumulated 0.272 ms
// at six, 0.284 unlimited; copied 0.176 ms unlimited, 0.194 at six.  (Over
// the previous 8192-element segments: four and six per CU respectively.)
constexpr int kPass3WgPerCuAccumulate = 6;
constexpr int kPass3WgPerCuCopy = 0;
constexpr int kPass2WgPerCuStreaming = 4;
constexpr int kPass2WgPerCuPacked = 4;
// Workgroups per update-pass launch.  A larger pass is split into consecutive
// launches of about this many workgroups each, on the same stream.  The
// hardware deals workgroups to the 8 XCDs in turn and each XCD then works
// through its share at its own pace; over a long launch the XCDs drift apart,
// so the single front of addresses that all CUs stream through splits into
// eight, and DRAM rows whose data is spread over several XCDs' workgroups are
// opened more than once.  A launch boundary brings the XCDs back together.
// Measured on MI355X over 6.7e9 elements in 4096-element workgroups (1.65M,
// 28.9 ms in one launch): 27.72 ms at 131072 per launch, 27.70 at 65536, 27.97
// at 16384 (each boundary costs about 4 us of ramp-down and ramp-up); in
// 2048-element workgroups 262144 and 131072 per launch give the same time
// (27.457 and 27.461 ms), so a launch keeps covering about 5.4e8 elements; a
// 302M-element table (147,559 workgroups) stays one launch.
constexpr uint32_t kPass2SliceBlocks = 262144;
// Workgroups per arrival-pass launch, for the same reason: the arrival pass
// reads and writes like the update pass.  Measured on MI355X, 6.7e9 bf16
// gradients accumulated in 8,192-element workgroups (822K): 7.01 ms in one
// launch, 6.86 at 131072 per launch, 6.81 at 65536, 6.78 at 32768.  With
// 4,096-element workgroups a launch of 131072 keeps covering about 5.4e8
// elements; the 302M-element table (73,780 workgroups) stays one launch.
constexpr uint32_t kPass3SliceBlocks = 131072;
// Number of launches for `n_blocks` workgroups at `per_launch` per launch
// (0: one launch); every launch gets the same count, the last possibly fewer.
inline int64_t update_launches(int64_t n_blocks, int64_t per_launch) {
    if (n_blocks <= 0) return 0;
    if (per_launch <= 0 || n_blocks <= per_launch) return 1;
    return (n_blocks + per_launch - 1) / per_launch;
}
// LDS bytes to reserve per workgroup for `wg_per_cu` resident workgroups on a
// CU with `lds_per_cu` bytes (2 KiB granules, so that allocation rounding
// never lowers the count); 0 if the device reports no LDS size.
inline uint32_t occupancy_lds(int64_t lds_per_cu, int wg_per_cu) {
    if (lds_per_cu <= 0 || wg_per_cu <= 0) return 0;
    const int64_t granule = 2048;
    const int64_t per = (lds_per_cu / wg_per_cu) / granule * granule;
    const int64_t max_per_wg = 64 * 1024;
    return (uint32_t)(per > max_per_wg ? max_per_wg : per);
}

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
    uint32_t lds_bytes;          // LDS reserved per workgroup (occupancy limit)
};

// Arrival pass: rewrites every trainable gradient from its arriving buffer
// and writes one owned sum-of-squares partial per workgroup; the reduction and
// finalize of the norm pass then run on those partials.
struct Pass3Args {
    const Seg3* segs;
    const uint32_t* blk_first;   // n_blocks + 1 entries
    uint32_t n_blocks;           // >= 1
    double* partials;            // n_blocks entries
    double* partials2;           // ceil(n_blocks / kReduceSpan) entries (two-level only)
    DevState* state;
    int32_t n_groups;
    int32_t advance;             // 1: this pass opens a new update (t += 1)
    int32_t accumulate;          // 1: g = round(g + incoming); 0: g = incoming
    uint32_t lds_bytes;          // LDS reserved per workgroup (occupancy limit)
};

struct Pass2Args {
    const Seg2* segs;
    const uint32_t* blk_first;
    uint32_t n_blocks;           // >= 1
    const DevState* state;
    uint32_t lds_bytes;          // LDS reserved per workgroup (occupancy limit)
};

hipError_t launch_pass1(const Pass1Args& a, hipStream_t s);
hipError_t launch_pass2(const Pass2Args& a, hipStream_t s);
// The arrival pass as ceil(n_blocks / per_launch) launches over consecutive
// ranges of its workgroups (per_launch 0: one launch), then the reduction of
// all n_blocks partials.
hipError_t launch_pass3(const Pass3Args& a, uint32_t per_launch, hipStream_t s);
hipError_t launch_set_groups(DevState* st, const GroupArgs& g, hipStream_t s);
hipError_t launch_set_schedules(DevState* st, const ScheduleArgs& a, hipStream_t s);
hipError_t launch_set_clip(DevState* st, double max_norm, double grad_divisor, hipStream_t s);
hipError_t launch_set_step(DevState* st, int64_t step, int32_t n_groups, hipStream_t s);

}  // namespace somaopt
