// The no-allocation table build: somaopt_init_tensor_table_noalloc places a
// handle's device tables, norm-pass partials and optimizer state in one
// file-scope device array instead of hipMalloc'd buffers, for callers that
// cannot allocate device memory.
//
// In host code the array's name stands for a host-side shadow, not a device
// address: its device address is looked up once per device with
// hipGetSymbolAddress (the device current) and only that address is ever
// handed to a kernel or a copy.  Every device has its own copy of the array,
// held until the process ends.  All no-allocation handles of a device share
// it: each build overwrites it and supersedes the handles built before it on
// that device (they refuse every call from then on).
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <string>

#include "scratch.hpp"
#include "somaopt.h"

#define SOMAOPT_NOALLOC_SCRATCH_BYTES (32u << 20)

static __device__ __align__(256) unsigned char scratch[SOMAOPT_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
char* g_base[kMaxDevices] = {};
std::atomic<uint64_t> g_generation[kMaxDevices];

}  // namespace

namespace somaopt {

int set_error(int code, const std::string& msg);

size_t scratch_capacity() { return SOMAOPT_NOALLOC_SCRATCH_BYTES; }

int scratch_base(int dev, char** base) {
    if (dev < 0 || dev >= kMaxDevices) return set_error(SOMAOPT_E_INVALID, "device index out of range for the scratch table");
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_base[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || p == nullptr)
            return set_error(SOMAOPT_E_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorName(e));
        g_base[dev] = static_cast<char*>(p);
    }
    *base = g_base[dev];
    return SOMAOPT_OK;
}

uint64_t scratch_generation(int dev) {
    return (dev >= 0 && dev < kMaxDevices) ? g_generation[dev].load(std::memory_order_acquire) : 0;
}

uint64_t scratch_claim(int dev) { return g_generation[dev].fetch_add(1, std::memory_order_acq_rel) + 1; }

}  // namespace somaopt

extern "C" int somaopt_init_tensor_table_noalloc(const somaopt_tensor_desc* descs, int64_t n_tensors,
                                                 const somaopt_group* groups, int32_t n_groups,
                                                 double max_norm, double grad_divisor, int64_t initial_step,
                                                 void* stream, somaopt_handle** out) {
    return somaopt::init_table(descs, n_tensors, groups, n_groups, max_norm, grad_divisor, initial_step, stream,
                               out, true);
}
