// Host-side tensor-table planner: validation, frozen-tensor removal, alignment
// analysis and the split of every tensor into workgroup-sized segments.
//
// The landing page's fused optimizer (paragraph 8) batches the norm and update
// work across tensors instead of launching per tensor; here that batching is a
// device-resident segment table plus a block table, built once by this
// planner.
#pragma once

#include <cstdint>
#include <string>
#include <vector>

#include "somaopt.h"

namespace somaopt {

// Device layout of a norm-pass segment: a contiguous run of one owned gradient.
struct alignas(8) Seg1 {
    const void* g;      // first element of the segment
    uint32_t head;      // scalar elements before the first 16-byte vector
    uint32_t nvec;      // 16-byte vectors (4 fp32 or 8 bf16 elements)
    uint32_t tail;      // scalar elements after the last vector
    uint32_t dtype;     // somaopt_dtype
};
static_assert(sizeof(Seg1) == 24, "Seg1 layout");

// Device layout of an arrival-pass segment: a contiguous run of one trainable
// gradient and of the buffer whose values arrive for it.
struct alignas(16) Seg3 {
    void* g;            // gradient, rewritten by the pass
    const void* inc;    // arriving values (same dtype and element order)
    uint32_t head;      // scalar elements before the first 16-byte vector
    uint32_t nvec;      // 16-byte vectors of both buffers
    uint32_t tail;      // scalar elements after the last vector
    uint16_t dtype;     // gradient somaopt_dtype
    uint16_t owner;     // 1: the segment enters the sum of squares
};
static_assert(sizeof(Seg3) == 32, "Seg3 layout");

// Device layout of an update-pass segment: the same run of p, m, v, g and the
// optional low-precision working copy.
struct alignas(16) Seg2 {
    float* p;
    float* m;
    float* v;
    const void* g;
    void* lowp;         // bf16/fp16 working copy or NULL
    uint32_t head;      // scalar elements before the first 4-element vector
    uint32_t nvec;      // 4-element vectors (16 bytes of p/m/v, 8 or 16 of g)
    uint32_t tail;      // scalar elements after the last vector
    uint16_t group;
    uint8_t dtype;      // gradient somaopt_dtype
    uint8_t lowp_dtype; // working-copy somaopt_dtype (when lowp is set)
};
static_assert(sizeof(Seg2) == 64, "Seg2 layout");

// Elements per workgroup.  Measured on MI355X: short workgroups (8192 gradient
// elements in the norm pass, 4096 = 256 threads x 4 vectors x 4 elements in the
// update pass) keep concurrently streamed addresses close together and beat
// longer or persistent workgroups by 10-20% in sustained HBM bandwidth.
constexpr int64_t kDefaultPass1Chunk = 8192;
constexpr int64_t kDefaultPass2Chunk = 4096;
// Update-pass segments of a streaming table (most elements in full-length
// segments): half a batch, so that each thread's four vectors are two real
// ones and two that the buffer bounds turn into no memory access, at four
// resident workgroups per CU instead of two: the same bytes in flight per CU
// in twice as many shorter workgroups.  Measured on MI355X in one process
// against 4096 at two per CU, four times on two boxes: the 7B update pass
// 27.28-27.46 against 27.74-27.89 ms (1.5-1.7%), the 302M-element one 0.3-1.5%
// faster; 3072 at three per CU and kernels built for exactly two vectors per
// thread or 128-thread workgroups were 4-13% slower.  Tables of small
// tensors keep 4096 (at 2048 the 20,000-tensor update pass took 134.5 against
// 128.0 us).
constexpr int64_t kStreamingPass2Chunk = 2048;
// Packing cost of one segment, in elements: a segment costs about one memory
// latency before its loads are in flight.  Measured on MI355X: for the norm
// (and arrival) pass 1024 beats 64 by 3% per step on the 20,000-tensor
// workload; for the update pass 4096, which keeps about one segment per
// workgroup, beats 1024 by 4% there and halves the 64-tensor workload's
// update pass (more workgroups each wait on one segment instead of a few
// walking several in turn).  Tables of full-length segments are unaffected.
constexpr int64_t kSegmentCost = 1024;
constexpr int64_t kUpdateSegmentCost = 4096;
// Packing cost used by build_plan for `pass` when the caller gives none.
inline int64_t default_segment_cost(int pass) { return pass == 2 ? kUpdateSegmentCost : kSegmentCost; }

struct PlanSeg {
    int64_t tensor;
    int64_t offset;
    int64_t numel;
    int64_t nvec;
    int32_t head;
    int32_t tail;
    int32_t vec;      // elements per vector, 0 = scalar only
    int32_t block;
};

struct Plan {
    std::vector<PlanSeg> segs;
    std::vector<uint32_t> block_first;   // n_blocks + 1 entries
    int64_t chunk = 0;
    int64_t n_blocks() const { return (int64_t)block_first.size() - 1; }
};

struct Counts {
    int64_t n_trainable = 0, trainable_numel = 0, owned_numel = 0;
};

// Validation that needs no device.  Returns SOMAOPT_OK or SOMAOPT_E_INVALID with
// `err` set.
int validate_host(const somaopt_tensor_desc* d, int64_t n, int32_t n_groups, std::string& err,
                  Counts* counts);

// Validation of the arriving-gradient buffers of an arrival pass: for every
// trainable tensor with numel > 0, incoming[i] is non-NULL and aligned to the
// gradient's element size; the pass writes the gradients, so gradients must not
// overlap one another nor any p, m, v or working copy, and no arriving buffer
// may overlap a written buffer (arriving buffers may overlap each other).
int validate_arrival(const somaopt_tensor_desc* d, int64_t n, const void* const* incoming, std::string& err);

// pass = 1 (owned gradient segments), 2 (all trainable segments, aligned for
// p/m/v/g) or 3 (all trainable segments, aligned for g and incoming[i]).
// segment_cost < 0: default_segment_cost(pass).
Plan build_plan(const somaopt_tensor_desc* d, int64_t n, int pass, int64_t chunk,
                int64_t segment_cost = -1, const void* const* incoming = nullptr);

// Largest segment of any pass: every kernel addresses a segment's vector body
// through a buffer resource whose size and lane offsets are 32-bit byte counts
// (at 2^30 fp32 elements a segment's 2^32 bytes would wrap to 0); 2^26
// elements keep every segment below 2^28 bytes.
constexpr int64_t kMaxChunk = int64_t(1) << 26;

// Normalise a requested chunk: positive multiple of 8, at least 256 elements,
// at most `max_chunk`.
int64_t normalise_chunk(int64_t requested, int64_t dflt, int64_t max_chunk = kMaxChunk);

// Segment length of the arrival pass: the norm pass's chunk (kept within
// kMaxChunk here too, for a chunk given from elsewhere).
inline int64_t arrival_chunk(int64_t pass1_chunk) {
    return pass1_chunk < kMaxChunk ? pass1_chunk : kMaxChunk;
}
// Arrival-pass segments of a streaming table: half the norm pass's, for the
// reason the update pass uses half batches (more, shorter workgroups with the
// same bytes in flight).  Measured on MI355X in one process against 8192:
// accumulating, 7B state 6.25 against 6.45 ms and 302M elements 0.272 against
// 0.290 ms; copying 4.04 against 4.15 ms and 0.176 against 0.179 ms (with the
// occupancy limits of kernels.hpp).
constexpr int64_t kStreamingPass3Chunk = 4096;

// True when at least half of the plan's elements lie in segments of the full
// chunk length, i.e. most workgroups stream one long run of one tensor.
bool streaming_plan(const Plan& p);

// The update pass's plan.  `requested` > 0: segments of that many elements
// (normalised).  Otherwise segments of kDefaultPass2Chunk, re-planned with
// kStreamingPass2Chunk when that plan streams.
Plan build_update_plan(const somaopt_tensor_desc* d, int64_t n, int64_t requested, int64_t segment_cost);

// The arrival pass's plan.  `requested` > 0: segments of that many elements
// (normalised).  Otherwise segments of arrival_chunk(pass1_chunk), re-planned
// with at most kStreamingPass3Chunk when that plan streams.
Plan build_arrival_plan(const somaopt_tensor_desc* d, int64_t n, int64_t pass1_chunk, int64_t requested,
                        const void* const* incoming);

inline int64_t grad_elem_bytes(int32_t dtype) { return dtype == SOMAOPT_F32 ? 4 : 2; }

}  // namespace somaopt
