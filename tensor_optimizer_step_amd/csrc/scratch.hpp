// Internal interface between the handle code (somaopt.cpp) and the
// file-scope device scratch array behind somaopt_init_tensor_table_noalloc
// (noalloc.hip).
#pragma once

#include <cstddef>
#include <cstdint>

#include "somaopt.h"

namespace somaopt {

// Bytes of the per-device scratch array (SOMAOPT_NOALLOC_SCRATCH_BYTES).
size_t scratch_capacity();

// Device address of the scratch array on `dev` (which must be the current
// device), looked up once per device and cached.  SOMAOPT_OK or SOMAOPT_E_HIP.
int scratch_base(int dev, char** base);

// Current generation of `dev`'s scratch array, and a new one for a handle
// that is about to overwrite it (every handle built on an older generation
// is superseded from then on).
uint64_t scratch_generation(int dev);
uint64_t scratch_claim(int dev);

// The table build shared by somaopt_init_tensor_table (from_scratch = false:
// every device buffer from hipMalloc) and somaopt_init_tensor_table_noalloc
// (from_scratch = true: every device buffer carved from the scratch array;
// no device allocation at all).
int init_table(const somaopt_tensor_desc* descs, int64_t n_tensors, const somaopt_group* groups,
               int32_t n_groups, double max_norm, double grad_divisor, int64_t initial_step, void* stream,
               somaopt_handle** out, bool from_scratch);

}  // namespace somaopt
