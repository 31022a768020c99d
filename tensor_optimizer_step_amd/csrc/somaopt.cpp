// C-ABI of the fused clip + AdamW optimizer step (declared in include/somaopt.h).
//
// Host side only: argument validation, the device tables built once at init,
// stream-ordered launches of the two passes and of the small setters, and the
// HIP-graph capture / replay of a whole step.  All arithmetic of the step runs
// in the kernels (kernels.hip).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kernels.hpp"
#include "plan.hpp"
#include "scratch.hpp"
#include "somaopt.h"
#include "state.hpp"

namespace somaopt {
int set_error(int code, const std::string& msg);
}  // namespace somaopt

using namespace somaopt;

struct somaopt_handle {
    int device = -1;
    int32_t n_groups = 0;
    somaopt_plan_info info{};
    Seg1* d_seg1 = nullptr;
    uint32_t* d_blk1 = nullptr;
    uint32_t nblk1 = 0;
    Seg2* d_seg2 = nullptr;
    uint32_t* d_blk2 = nullptr;
    uint32_t nblk2 = 0;
    uint32_t lds1 = 0;             // LDS reserved per norm-pass workgroup
    uint32_t lds2 = 0;             // LDS reserved per update-pass workgroup
    double* d_partials = nullptr;
    double* d_partials2 = nullptr;
    DevState* d_state = nullptr;
    // arrival pass (registered once by somaopt_register_arrival)
    std::vector<somaopt_tensor_desc> descs;   // the table given at init
    Seg3* d_seg3 = nullptr;
    uint32_t* d_blk3 = nullptr;
    uint32_t nblk3 = 0;
    uint32_t lds3 = 0;             // LDS reserved per arrival-pass workgroup, copying
    uint32_t lds3_acc = 0;         // and accumulating
    uint32_t per3 = 0;             // arrival-pass workgroups per launch (0: one launch)
    double* d_partials3 = nullptr;
    double* d_partials3b = nullptr;
    int64_t pass1_chunk = 0;
    bool pending = false;          // a norm pass opened an update not yet applied
    hipStream_t cap_stream = nullptr;
    hipGraphExec_t exec = nullptr;
    // Built by somaopt_init_tensor_table_noalloc: the tables, partials and
    // state live in the device scratch array (never freed), valid while the
    // device's scratch generation is still this one.
    bool scratch = false;
    uint64_t scratch_gen = 0;
};

namespace {

thread_local std::string g_last_error;

int fail(int code, const std::string& msg) {
    g_last_error = msg;
    return code;
}

int hip_fail(hipError_t e, const char* what) {
    return fail(SOMAOPT_E_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                   hipGetErrorString(e) + ")");
}

// Makes the handle's device current for the duration of a call.
class DeviceGuard {
   public:
    explicit DeviceGuard(int dev) {
        if (hipGetDevice(&prev_) != hipSuccess) prev_ = -1;
        if (prev_ != dev) ok_ = hipSetDevice(dev) == hipSuccess;
        restore_ = prev_ >= 0 && prev_ != dev;
    }
    ~DeviceGuard() {
        if (restore_) (void)hipSetDevice(prev_);
    }
    bool ok() const { return ok_; }

   private:
    int prev_ = -1;
    bool ok_ = true;
    bool restore_ = false;
};

bool finite(double x) { return std::isfinite(x); }

int check_groups(const somaopt_group* g, int32_t n) {
    if (n < 1 || n > SOMAOPT_MAX_GROUPS)
        return fail(SOMAOPT_E_INVALID, "n_groups must be in [1, " + std::to_string(SOMAOPT_MAX_GROUPS) + "]");
    if (!g) return fail(SOMAOPT_E_INVALID, "groups is NULL");
    for (int32_t k = 0; k < n; ++k) {
        const somaopt_group& h = g[k];
        const std::string at = "group " + std::to_string(k) + ": ";
        if (!finite(h.lr)) return fail(SOMAOPT_E_INVALID, at + "lr is not finite");
        if (!finite(h.weight_decay)) return fail(SOMAOPT_E_INVALID, at + "weight_decay is not finite");
        if (!(h.beta1 >= 0.0 && h.beta1 < 1.0)) return fail(SOMAOPT_E_INVALID, at + "beta1 outside [0, 1)");
        if (!(h.beta2 >= 0.0 && h.beta2 < 1.0)) return fail(SOMAOPT_E_INVALID, at + "beta2 outside [0, 1)");
        if (!(h.eps >= 0.0) || !finite(h.eps)) return fail(SOMAOPT_E_INVALID, at + "eps must be finite and >= 0");
    }
    return SOMAOPT_OK;
}

int check_clip(double max_norm, double grad_divisor) {
    if (!(max_norm > 0.0) || !finite(max_norm)) return fail(SOMAOPT_E_INVALID, "max_norm must be finite and > 0");
    if (!(grad_divisor > 0.0) || !finite(grad_divisor))
        return fail(SOMAOPT_E_INVALID, "grad_divisor must be finite and > 0");
    return SOMAOPT_OK;
}

int64_t env_int(const char* name, int64_t dflt) {
    const char* s = std::getenv(name);
    if (!s || !*s) return dflt;
    char* end = nullptr;
    long long v = std::strtoll(s, &end, 10);
    return (end && *end == 0) ? (int64_t)v : dflt;
}

// `bytes` at `p` must be device memory of `dev` inside one HIP allocation.
int check_device_range(const void* p, uintptr_t bytes, int dev, const std::string& at) {
    hipPointerAttribute_t attr;
    std::memset(&attr, 0, sizeof(attr));
    hipError_t e = hipPointerGetAttributes(&attr, p);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SOMAOPT_E_INVALID, at + "not a HIP device pointer");
    }
    if (attr.type != hipMemoryTypeDevice || attr.device != dev)
        return fail(SOMAOPT_E_INVALID, at + "not device memory of the current device");
    hipDeviceptr_t base = nullptr;
    size_t size = 0;
    e = hipMemGetAddressRange(&base, &size, const_cast<void*>(p));
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return fail(SOMAOPT_E_INVALID, at + "allocation range unknown to HIP");
    }
    const uintptr_t lo = reinterpret_cast<uintptr_t>(base);
    const uintptr_t a = reinterpret_cast<uintptr_t>(p);
    if (a < lo || a + bytes > lo + size) return fail(SOMAOPT_E_INVALID, at + "runs past the end of its allocation");
    return SOMAOPT_OK;
}

bool skip_pointer_check() {
    const char* skip = std::getenv("SOMAOPT_SKIP_POINTER_CHECK");
    return skip && std::strcmp(skip, "1") == 0;
}

// Every trainable buffer must be device memory of `dev` and lie inside one
// allocation, so that no kernel can address memory it was not given.
int check_pointers(const somaopt_tensor_desc* d, int64_t n, int dev) {
    if (skip_pointer_check()) return SOMAOPT_OK;
    static const char* kind[5] = {"param", "exp_avg", "exp_avg_sq", "grad", "param_lowp"};
    for (int64_t i = 0; i < n; ++i) {
        const somaopt_tensor_desc& t = d[i];
        if (!t.trainable || t.numel == 0) continue;
        const void* ptrs[5] = {t.param, t.exp_avg, t.exp_avg_sq, t.grad, t.param_lowp};
        const size_t esz[5] = {4, 4, 4, (size_t)grad_elem_bytes(t.grad_dtype), 2};
        const int nbuf = t.param_lowp ? 5 : 4;
        for (int k = 0; k < nbuf; ++k) {
            const std::string at = "tensor " + std::to_string(i) + " " + kind[k] + ": ";
            int rc = check_device_range(ptrs[k], (uintptr_t)t.numel * esz[k], dev, at);
            if (rc) return rc;
        }
    }
    return SOMAOPT_OK;
}

void free_handle(somaopt_handle* h) {
    if (!h) return;
    if (h->exec) (void)hipGraphExecDestroy(h->exec);
    if (h->cap_stream) (void)hipStreamDestroy(h->cap_stream);
    void* init_bufs[] = {h->d_seg1, h->d_blk1, h->d_seg2, h->d_blk2, h->d_partials, h->d_partials2, h->d_state};
    if (!h->scratch)
        for (void* p : init_bufs)
            if (p) (void)hipFree(p);
    void* arrival_bufs[] = {h->d_seg3, h->d_blk3, h->d_partials3, h->d_partials3b};
    for (void* p : arrival_bufs)
        if (p) (void)hipFree(p);
    delete h;
}

// NULL, or a no-allocation handle whose scratch tables a later no-allocation
// init on the same device has overwritten: refused before any work.
int check_handle(const somaopt_handle* h) {
    if (!h) return fail(SOMAOPT_E_INVALID, "handle is NULL");
    if (h->scratch && h->scratch_gen != scratch_generation(h->device))
        return fail(SOMAOPT_E_STATE,
                    "superseded: a later somaopt_init_tensor_table_noalloc on this device has overwritten the "
                    "device scratch array that held this handle's tables");
    return SOMAOPT_OK;
}

// Where the device buffers of a table build go: hipMalloc per buffer, or
// consecutive 256-byte-aligned pieces of a region (the scratch array); in
// counting mode (no region, counting = true) only the bytes are added up.
struct Placer {
    char* region = nullptr;
    bool counting = false;
    size_t used = 0;
    hipError_t get(void** dst, size_t bytes) {
        if (!region && !counting) return hipMalloc(dst, bytes);
        used = (used + 255) & ~size_t(255);
        *dst = region ? region + used : nullptr;
        used += bytes;
        return hipSuccess;
    }
};

template <typename T>
hipError_t alloc_upload(T** dst, const std::vector<T>& src, hipStream_t s, Placer& where) {
    const size_t bytes = std::max<size_t>(src.size(), 1) * sizeof(T);
    hipError_t e = where.get(reinterpret_cast<void**>(dst), bytes);
    if (e != hipSuccess || where.counting) return e;
    if (!src.empty()) e = hipMemcpyAsync(*dst, src.data(), src.size() * sizeof(T), hipMemcpyHostToDevice, s);
    return e;
}

template <typename T>
hipError_t alloc_upload(T** dst, const std::vector<T>& src, hipStream_t s) {
    Placer malloc_each;
    return alloc_upload(dst, src, s, malloc_each);
}

void fill_info(somaopt_plan_info* info, int64_t n_tensors, const Counts& c, const Plan& p1, const Plan& p2) {
    std::memset(info, 0, sizeof(*info));
    info->n_tensors = n_tensors;
    info->n_trainable = c.n_trainable;
    info->trainable_numel = c.trainable_numel;
    info->owned_numel = c.owned_numel;
    info->pass1_segments = (int64_t)p1.segs.size();
    info->pass1_blocks = p1.n_blocks();
    info->pass2_segments = (int64_t)p2.segs.size();
    info->pass2_blocks = p2.n_blocks();
    int64_t scal = 0;
    for (const PlanSeg& s : p2.segs) scal += (s.vec == 0);
    info->scalar_segments = scal;
    info->pass1_chunk = p1.chunk;
    info->pass2_chunk = p2.chunk;
    info->table_bytes = (int64_t)(p1.segs.size() * sizeof(Seg1) + p2.segs.size() * sizeof(Seg2) +
                                  (p1.block_first.size() + p2.block_first.size()) * sizeof(uint32_t));
    info->pass1_wg_per_cu = streaming_plan(p1) ? kPass1WgPerCuStreaming : 0;
    info->pass2_wg_per_cu = streaming_plan(p2) ? kPass2WgPerCuStreaming : kPass2WgPerCuPacked;
    info->pass2_launches = update_launches(p2.n_blocks(), kPass2SliceBlocks);
}

int launch_norm_pass(somaopt_handle* h, int advance, hipStream_t s) {
    Pass1Args a;
    a.segs = h->d_seg1;
    a.blk_first = h->d_blk1;
    a.n_blocks = h->nblk1;
    a.partials = h->d_partials;
    a.partials2 = h->d_partials2;
    a.state = h->d_state;
    a.n_groups = h->n_groups;
    a.advance = advance;
    a.lds_bytes = h->lds1;
    hipError_t e = launch_pass1(a, s);
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "norm pass launch");
}

// The update pass as info.pass2_launches launches over consecutive ranges of
// its workgroups.  A launch over workgroups [first, first + n) reads
// blk_first[first .. first + n], inside the nblk2 + 1 entries of the table.
int launch_update_pass(somaopt_handle* h, hipStream_t s) {
    if (h->nblk2 == 0) return SOMAOPT_OK;
    const uint32_t nl = (uint32_t)std::max<int64_t>(h->info.pass2_launches, 1);
    const uint32_t per = (h->nblk2 + nl - 1) / nl;
    Pass2Args a;
    a.segs = h->d_seg2;
    a.state = h->d_state;
    a.lds_bytes = h->lds2;
    for (uint32_t first = 0; first < h->nblk2; first += per) {
        a.blk_first = h->d_blk2 + first;
        a.n_blocks = std::min(per, h->nblk2 - first);
        hipError_t e = launch_pass2(a, s);
        if (e != hipSuccess) return hip_fail(e, "update pass launch");
    }
    return SOMAOPT_OK;
}

}  // namespace

int somaopt::set_error(int code, const std::string& msg) { return fail(code, msg); }

namespace {
int launch_arrival_pass(somaopt_handle* h, int advance, int32_t accumulate, hipStream_t s);
}  // namespace

extern "C" {

const char* somaopt_last_error(void) { return g_last_error.c_str(); }

const char* somaopt_version(void) { return "somaopt 0.1.0 (gfx950)"; }

int64_t somaopt_debug_plan(const somaopt_tensor_desc* descs, int64_t n_tensors, int32_t n_groups,
                           int32_t pass, int64_t pass1_chunk, int64_t pass2_chunk,
                           somaopt_plan_segment* segs, int64_t cap, somaopt_plan_info* info) {
    if (pass != 1 && pass != 2) return fail(SOMAOPT_E_INVALID, "pass must be 1 or 2");
    if (cap < 0) return fail(SOMAOPT_E_INVALID, "cap < 0");
    std::string err;
    Counts c;
    int rc = validate_host(descs, n_tensors, n_groups, err, &c);
    if (rc != SOMAOPT_OK) return fail(rc, err);
    const int64_t ch1 = normalise_chunk(pass1_chunk, kDefaultPass1Chunk);
    Plan p1 = build_plan(descs, n_tensors, 1, ch1);
    Plan p2 = build_update_plan(descs, n_tensors, pass2_chunk, kUpdateSegmentCost);
    if (info) fill_info(info, n_tensors, c, p1, p2);
    const Plan& p = pass == 1 ? p1 : p2;
    if (segs) {
        for (int64_t i = 0; i < (int64_t)p.segs.size() && i < cap; ++i) {
            const PlanSeg& s = p.segs[i];
            segs[i].tensor = s.tensor;
            segs[i].offset = s.offset;
            segs[i].numel = s.numel;
            segs[i].nvec = s.nvec;
            segs[i].head = s.head;
            segs[i].tail = s.tail;
            segs[i].vec_elems = s.vec;
            segs[i].block = s.block;
        }
    }
    return (int64_t)p.segs.size();
}

int somaopt_init_tensor_table(const somaopt_tensor_desc* descs, int64_t n_tensors,
                              const somaopt_group* groups, int32_t n_groups, double max_norm,
                              double grad_divisor, int64_t initial_step, void* stream,
                              somaopt_handle** out) {
    return init_table(descs, n_tensors, groups, n_groups, max_norm, grad_divisor, initial_step, stream, out,
                      false);
}

}  // extern "C"

// The table build behind both init calls.  With from_scratch, every device
// buffer is a piece of the scratch array: the bytes are counted first and a
// table that does not fit is refused before anything touches the device.
int somaopt::init_table(const somaopt_tensor_desc* descs, int64_t n_tensors, const somaopt_group* groups,
                        int32_t n_groups, double max_norm, double grad_divisor, int64_t initial_step,
                        void* stream, somaopt_handle** out, bool from_scratch) {
    if (!out) return fail(SOMAOPT_E_INVALID, "out is NULL");
    *out = nullptr;
    int rc = check_groups(groups, n_groups);
    if (rc) return rc;
    if ((rc = check_clip(max_norm, grad_divisor))) return rc;
    if (initial_step < 0) return fail(SOMAOPT_E_INVALID, "initial_step < 0");
    std::string err;
    Counts counts;
    rc = validate_host(descs, n_tensors, n_groups, err, &counts);
    if (rc) return fail(rc, err);
    const int64_t ch1 = normalise_chunk(env_int("SOMAOPT_PASS1_CHUNK", 0), kDefaultPass1Chunk);
    const int64_t cost1 = std::max<int64_t>(0, env_int("SOMAOPT_SEGMENT_COST", kSegmentCost));
    const int64_t cost2 = std::max<int64_t>(0, env_int("SOMAOPT_UPDATE_SEGMENT_COST", kUpdateSegmentCost));
    Plan p1 = build_plan(descs, n_tensors, 1, ch1, cost1);
    Plan p2 = build_update_plan(descs, n_tensors, env_int("SOMAOPT_PASS2_CHUNK", 0), cost2);
    if (p1.segs.size() >= 0xFFFFFFFFull || p2.segs.size() >= 0xFFFFFFFFull)
        return fail(SOMAOPT_E_INVALID, "too many segments for 32-bit indices");
    // A dispatch holds fewer than 2^32 work-items.
    if ((uint64_t)p1.n_blocks() * kPass1Threads >= 0xFFFFFFFFull ||
        (uint64_t)p2.n_blocks() * kPass2Threads >= 0xFFFFFFFFull)
        return fail(SOMAOPT_E_INVALID, "table too large for one dispatch (raise SOMAOPT_PASS*_CHUNK)");
    // The norm pass always runs at least one workgroup so that the statistics
    // are produced even when nothing is owned.
    if (p1.block_first.size() < 2) p1.block_first = {0u, 0u};

    std::vector<Seg1> s1(p1.segs.size());
    for (size_t i = 0; i < p1.segs.size(); ++i) {
        const PlanSeg& s = p1.segs[i];
        const somaopt_tensor_desc& t = descs[s.tensor];
        const size_t gsz = (size_t)grad_elem_bytes(t.grad_dtype);
        s1[i].g = static_cast<const char*>(t.grad) + (size_t)s.offset * gsz;
        s1[i].head = (uint32_t)s.head;
        s1[i].nvec = (uint32_t)s.nvec;
        s1[i].tail = (uint32_t)s.tail;
        s1[i].dtype = (uint32_t)t.grad_dtype;
    }
    std::vector<Seg2> s2(p2.segs.size());
    for (size_t i = 0; i < p2.segs.size(); ++i) {
        const PlanSeg& s = p2.segs[i];
        const somaopt_tensor_desc& t = descs[s.tensor];
        const size_t gsz = (size_t)grad_elem_bytes(t.grad_dtype);
        s2[i].p = static_cast<float*>(t.param) + s.offset;
        s2[i].m = static_cast<float*>(t.exp_avg) + s.offset;
        s2[i].v = static_cast<float*>(t.exp_avg_sq) + s.offset;
        s2[i].g = static_cast<const char*>(t.grad) + (size_t)s.offset * gsz;
        s2[i].lowp = t.param_lowp ? static_cast<char*>(t.param_lowp) + (size_t)s.offset * 2 : nullptr;
        s2[i].head = (uint32_t)s.head;
        s2[i].nvec = (uint32_t)s.nvec;
        s2[i].tail = (uint32_t)s.tail;
        s2[i].group = (uint16_t)t.group;
        s2[i].dtype = (uint8_t)t.grad_dtype;
        s2[i].lowp_dtype = (uint8_t)(t.param_lowp ? t.lowp_dtype : 0);
    }

    // Device bytes of the table build (the order of place_buffers below).
    const uint32_t nblk1 = (uint32_t)(p1.block_first.size() - 1);
    auto place_buffers = [&](somaopt_handle* hh, Placer& where, hipStream_t s,
                             const std::vector<DevState>& stv) -> hipError_t {
        hipError_t e;
        if ((e = alloc_upload(&hh->d_seg1, s1, s, where)) != hipSuccess ||
            (e = alloc_upload(&hh->d_blk1, p1.block_first, s, where)) != hipSuccess ||
            (e = alloc_upload(&hh->d_seg2, s2, s, where)) != hipSuccess ||
            (e = alloc_upload(&hh->d_blk2, p2.block_first, s, where)) != hipSuccess ||
            (e = alloc_upload(&hh->d_state, stv, s, where)) != hipSuccess ||
            (e = where.get(reinterpret_cast<void**>(&hh->d_partials),
                           sizeof(double) * std::max<uint32_t>(nblk1, 1))) != hipSuccess ||
            (e = where.get(reinterpret_cast<void**>(&hh->d_partials2),
                           sizeof(double) * ((nblk1 + kReduceSpan - 1) / kReduceSpan + 1))) != hipSuccess)
            return e;
        return hipSuccess;
    };
    if (from_scratch) {
        somaopt_handle probe;
        Placer count;
        count.counting = true;
        (void)place_buffers(&probe, count, nullptr, std::vector<DevState>(1));
        if (count.used > scratch_capacity())
            return fail(SOMAOPT_E_INVALID, "the table needs " + std::to_string(count.used) +
                                               " bytes of device scratch; the no-allocation entry point holds at most " +
                                               std::to_string(scratch_capacity()) + " (use somaopt_init_tensor_table)");
    }
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
    if ((rc = check_pointers(descs, n_tensors, dev))) return rc;

    DevState st;
    std::memset(&st, 0, sizeof(st));
    st.n_groups = n_groups;
    st.stats.n_groups = n_groups;
    st.max_norm = max_norm;
    st.grad_divisor = grad_divisor;
    for (int32_t k = 0; k < n_groups; ++k) {
        st.step[k] = initial_step;
        st.hyper[k] = groups[k];
    }

    somaopt_handle* h = new (std::nothrow) somaopt_handle();
    if (!h) return fail(SOMAOPT_E_NOMEM, "host allocation failed");
    h->device = dev;
    h->n_groups = n_groups;
    h->descs.assign(descs, descs + n_tensors);
    h->pass1_chunk = ch1;
    fill_info(&h->info, n_tensors, counts, p1, p2);
    h->nblk1 = (uint32_t)(p1.block_first.size() - 1);
    h->nblk2 = (uint32_t)p2.n_blocks();
    int lds_per_cu = 0;
    if ((e = hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev)) !=
        hipSuccess) {
        free_handle(h);
        return hip_fail(e, "hipDeviceGetAttribute(LDS per CU)");
    }
    // Overrides for tuning on other parts: 0 lifts the limit, unset keeps the
    // choice made from the table shape.
    const int64_t w1 = env_int("SOMAOPT_PASS1_WG_PER_CU", -1), w2 = env_int("SOMAOPT_PASS2_WG_PER_CU", -1);
    if (w1 >= 0) h->info.pass1_wg_per_cu = std::min<int64_t>(w1, 64);
    if (w2 >= 0) h->info.pass2_wg_per_cu = std::min<int64_t>(w2, 64);
    h->lds1 = occupancy_lds(lds_per_cu, (int)h->info.pass1_wg_per_cu);
    h->lds2 = occupancy_lds(lds_per_cu, (int)h->info.pass2_wg_per_cu);
    const int64_t slice = env_int("SOMAOPT_PASS2_SLICE_BLOCKS", -1);
    if (slice >= 0) h->info.pass2_launches = update_launches(h->nblk2, slice);
    hipStream_t s = static_cast<hipStream_t>(stream);

    Placer where;
    if (from_scratch) {
        if ((rc = scratch_base(dev, &where.region)) != SOMAOPT_OK) {
            free_handle(h);
            return rc;
        }
        // From here on the scratch array is overwritten: every handle built
        // on it earlier is superseded.
        h->scratch = true;
        h->scratch_gen = scratch_claim(dev);
    }
    // The whole state block is uploaded (every field that must start at zero
    // is zero in it); the partials are written by each norm pass before they
    // are read, so they need no clearing.
    const std::vector<DevState> stv(1, st);
    if ((e = place_buffers(h, where, s, stv)) != hipSuccess || (e = hipStreamSynchronize(s)) != hipSuccess) {
        free_handle(h);
        return e == hipErrorOutOfMemory ? fail(SOMAOPT_E_NOMEM, "device allocation of the tables failed")
                                        : hip_fail(e, "table upload");
    }
    *out = h;
    return SOMAOPT_OK;
}

extern "C" {


int somaopt_grad_sqnorm(somaopt_handle* h, void* stream) {
    if (int bad = check_handle(h)) return bad;
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    int rc = launch_norm_pass(h, h->pending ? 0 : 1, static_cast<hipStream_t>(stream));
    if (rc) return rc;
    h->pending = true;
    return SOMAOPT_OK;
}

int somaopt_fused_adamw_step(somaopt_handle* h, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (!h->pending) return fail(SOMAOPT_E_STATE, "somaopt_grad_sqnorm must precede each update");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    int rc = launch_update_pass(h, static_cast<hipStream_t>(stream));
    if (rc) return rc;
    h->pending = false;
    return SOMAOPT_OK;
}

int somaopt_register_arrival(somaopt_handle* h, const void* const* incoming, int64_t n_tensors, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (h->d_seg3) return fail(SOMAOPT_E_STATE, "arriving buffers are already registered for this handle");
    if (n_tensors != (int64_t)h->descs.size())
        return fail(SOMAOPT_E_INVALID, "n_tensors differs from the table given at init");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    const somaopt_tensor_desc* d = h->descs.data();
    std::string err;
    if (validate_arrival(d, n_tensors, incoming, err) != SOMAOPT_OK) return fail(SOMAOPT_E_INVALID, err);
    if (!skip_pointer_check()) {
        for (int64_t i = 0; i < n_tensors; ++i) {
            if (!d[i].trainable || d[i].numel == 0) continue;
            int rc = check_device_range(incoming[i], (uintptr_t)d[i].numel * grad_elem_bytes(d[i].grad_dtype),
                                        h->device, "tensor " + std::to_string(i) + " incoming: ");
            if (rc) return rc;
        }
    }
    Plan p3 = build_arrival_plan(d, n_tensors, h->pass1_chunk, env_int("SOMAOPT_PASS3_CHUNK", 0), incoming);
    if (p3.segs.size() >= 0xFFFFFFFFull || (uint64_t)p3.n_blocks() * kPass1Threads >= 0xFFFFFFFFull)
        return fail(SOMAOPT_E_INVALID, "arrival table too large for one dispatch");
    if (p3.block_first.size() < 2) p3.block_first = {0u, 0u};   // statistics even when nothing is trainable
    std::vector<Seg3> s3(p3.segs.size());
    for (size_t i = 0; i < p3.segs.size(); ++i) {
        const PlanSeg& sg = p3.segs[i];
        const somaopt_tensor_desc& t = d[sg.tensor];
        const size_t gsz = (size_t)grad_elem_bytes(t.grad_dtype);
        s3[i].g = static_cast<char*>(const_cast<void*>(t.grad)) + (size_t)sg.offset * gsz;
        s3[i].inc = static_cast<const char*>(incoming[sg.tensor]) + (size_t)sg.offset * gsz;
        s3[i].head = (uint32_t)sg.head;
        s3[i].nvec = (uint32_t)sg.nvec;
        s3[i].tail = (uint32_t)sg.tail;
        s3[i].dtype = (uint16_t)t.grad_dtype;
        s3[i].owner = (uint16_t)(t.owner ? 1 : 0);
    }
    const uint32_t nblk = (uint32_t)(p3.block_first.size() - 1);
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e;
    if ((e = alloc_upload(&h->d_seg3, s3, s)) != hipSuccess ||
        (e = alloc_upload(&h->d_blk3, p3.block_first, s)) != hipSuccess ||
        (e = hipMalloc(reinterpret_cast<void**>(&h->d_partials3), sizeof(double) * nblk)) != hipSuccess ||
        (e = hipMalloc(reinterpret_cast<void**>(&h->d_partials3b),
                       sizeof(double) * ((nblk + kReduceSpan - 1) / kReduceSpan + 1))) != hipSuccess ||
        (e = hipStreamSynchronize(s)) != hipSuccess) {
        void* bufs[] = {h->d_seg3, h->d_blk3, h->d_partials3, h->d_partials3b};
        for (void* p : bufs)
            if (p) (void)hipFree(p);
        h->d_seg3 = nullptr;
        h->d_blk3 = nullptr;
        h->d_partials3 = h->d_partials3b = nullptr;
        return e == hipErrorOutOfMemory ? fail(SOMAOPT_E_NOMEM, "device allocation of the arrival table failed")
                                        : hip_fail(e, "arrival table upload");
    }
    h->nblk3 = nblk;
    int lds_per_cu = 0;
    if (hipDeviceGetAttribute(&lds_per_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, h->device) !=
        hipSuccess)
        lds_per_cu = 0;
    const int64_t w3 = env_int("SOMAOPT_PASS3_WG_PER_CU", -1);
    const bool stream3 = streaming_plan(p3);
    h->lds3 = occupancy_lds(lds_per_cu, w3 >= 0 ? (int)std::min<int64_t>(w3, 64)
                                                : (stream3 ? kPass3WgPerCuCopy : 0));
    h->lds3_acc = occupancy_lds(lds_per_cu, w3 >= 0 ? (int)std::min<int64_t>(w3, 64)
                                                    : (stream3 ? kPass3WgPerCuAccumulate : 0));
    const int64_t slice = env_int("SOMAOPT_PASS3_SLICE_BLOCKS", -1);
    h->per3 = slice >= 0 ? (uint32_t)std::min<int64_t>(slice, 0xFFFFFFFFll) : kPass3SliceBlocks;
    return SOMAOPT_OK;
}

int somaopt_arrival_sqnorm(somaopt_handle* h, int32_t accumulate, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (!h->d_seg3) return fail(SOMAOPT_E_STATE, "somaopt_register_arrival must precede the arrival pass");
    if (accumulate != 0 && accumulate != 1) return fail(SOMAOPT_E_INVALID, "accumulate must be 0 or 1");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    int rc = launch_arrival_pass(h, h->pending ? 0 : 1, accumulate, static_cast<hipStream_t>(stream));
    if (rc) return rc;
    h->pending = true;
    return SOMAOPT_OK;
}

int somaopt_set_groups(somaopt_handle* h, const somaopt_group* groups, int32_t n_groups, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (n_groups != h->n_groups) return fail(SOMAOPT_E_INVALID, "n_groups differs from the handle's");
    int rc = check_groups(groups, n_groups);
    if (rc) return rc;
    GroupArgs a;
    std::memset(&a, 0, sizeof(a));
    a.n = n_groups;
    for (int32_t k = 0; k < n_groups; ++k) a.g[k] = groups[k];
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e = launch_set_groups(h->d_state, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "set_groups launch");
}

int somaopt_set_schedules(somaopt_handle* h, const somaopt_schedule* schedules, int32_t n_groups, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (n_groups != h->n_groups) return fail(SOMAOPT_E_INVALID, "n_groups differs from the handle's");
    if (!schedules) return fail(SOMAOPT_E_INVALID, "schedules is NULL");
    ScheduleArgs a;
    std::memset(&a, 0, sizeof(a));
    a.n = n_groups;
    for (int32_t k = 0; k < n_groups; ++k) {
        const somaopt_schedule& c = schedules[k];
        const std::string at = "schedule " + std::to_string(k) + ": ";
        if (c.kind < SOMAOPT_SCHED_NONE || c.kind > SOMAOPT_SCHED_WARMUP_COSINE)
            return fail(SOMAOPT_E_INVALID, at + "unknown kind");
        if (c.kind != SOMAOPT_SCHED_NONE) {
            if (!(c.peak_lr >= 0.0) || !std::isfinite(c.peak_lr) || !(c.floor_lr >= 0.0) || !std::isfinite(c.floor_lr))
                return fail(SOMAOPT_E_INVALID, at + "peak_lr and floor_lr must be finite and >= 0");
            const bool warm = c.kind == SOMAOPT_SCHED_LINEAR_WARMUP || c.kind == SOMAOPT_SCHED_WARMUP_COSINE;
            const bool cosine = c.kind == SOMAOPT_SCHED_COSINE || c.kind == SOMAOPT_SCHED_WARMUP_COSINE;
            if (warm && c.warmup < 1) return fail(SOMAOPT_E_INVALID, at + "warmup must be >= 1");
            if (cosine && c.total < 1) return fail(SOMAOPT_E_INVALID, at + "total must be >= 1");
            if (c.kind == SOMAOPT_SCHED_WARMUP_COSINE && c.total <= c.warmup)
                return fail(SOMAOPT_E_INVALID, at + "total must exceed warmup");
        }
        a.s[k] = c;
    }
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e = launch_set_schedules(h->d_state, a, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "set_schedules launch");
}

int somaopt_set_clip(somaopt_handle* h, double max_norm, double grad_divisor, void* stream) {
    if (int bad = check_handle(h)) return bad;
    int rc = check_clip(max_norm, grad_divisor);
    if (rc) return rc;
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e = launch_set_clip(h->d_state, max_norm, grad_divisor, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "set_clip launch");
}

int somaopt_set_step(somaopt_handle* h, int64_t step, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (step < 0) return fail(SOMAOPT_E_INVALID, "step < 0");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e = launch_set_step(h->d_state, step, h->n_groups, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return hip_fail(e, "set_step launch");
    h->pending = false;
    return SOMAOPT_OK;
}

}  // extern "C"

namespace {

// Arrival pass launch (shared by the eager call and the captured step).
int launch_arrival_pass(somaopt_handle* h, int advance, int32_t accumulate, hipStream_t s) {
    Pass3Args a;
    a.segs = h->d_seg3;
    a.blk_first = h->d_blk3;
    a.n_blocks = h->nblk3;
    a.partials = h->d_partials3;
    a.partials2 = h->d_partials3b;
    a.state = h->d_state;
    a.n_groups = h->n_groups;
    a.advance = advance;
    a.accumulate = accumulate;
    a.lds_bytes = accumulate ? h->lds3_acc : h->lds3;
    hipError_t e = launch_pass3(a, h->per3, s);
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "arrival pass launch");
}

// Capture {first pass, update pass} on the handle's private stream and make
// it the handle's step graph.  `arrival` < 0: the norm pass; else the arrival
// pass with accumulate = arrival.
int capture(somaopt_handle* h, int arrival) {
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e;
    if (!h->cap_stream) {
        e = hipStreamCreateWithFlags(&h->cap_stream, hipStreamNonBlocking);
        if (e != hipSuccess) {
            h->cap_stream = nullptr;
            return hip_fail(e, "hipStreamCreateWithFlags");
        }
    }
    e = hipStreamBeginCapture(h->cap_stream, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(e, "hipStreamBeginCapture");
    int rc = arrival < 0 ? launch_norm_pass(h, 1, h->cap_stream) : launch_arrival_pass(h, 1, arrival, h->cap_stream);
    if (!rc) rc = launch_update_pass(h, h->cap_stream);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(h->cap_stream, &graph);
    if (rc) {
        if (graph) (void)hipGraphDestroy(graph);
        return rc;
    }
    if (e != hipSuccess) return hip_fail(e, "hipStreamEndCapture");
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(e, "hipGraphInstantiate");
    if (h->exec) (void)hipGraphExecDestroy(h->exec);
    h->exec = exec;
    return SOMAOPT_OK;
}

}  // namespace

extern "C" {

int somaopt_capture_step(somaopt_handle* h) {
    if (int bad = check_handle(h)) return bad;
    return capture(h, -1);
}

int somaopt_capture_arrival_step(somaopt_handle* h, int32_t accumulate) {
    if (int bad = check_handle(h)) return bad;
    if (!h->d_seg3) return fail(SOMAOPT_E_STATE, "somaopt_register_arrival must precede the capture");
    if (accumulate != 0 && accumulate != 1) return fail(SOMAOPT_E_INVALID, "accumulate must be 0 or 1");
    return capture(h, accumulate);
}

int somaopt_replay_step(somaopt_handle* h, void* stream) {
    if (int bad = check_handle(h)) return bad;
    if (!h->exec) return fail(SOMAOPT_E_STATE, "no captured step (call somaopt_capture_step)");
    if (h->pending) return fail(SOMAOPT_E_STATE, "an eager norm or arrival pass is pending; finish it with somaopt_fused_adamw_step");
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipError_t e = hipGraphLaunch(h->exec, static_cast<hipStream_t>(stream));
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "hipGraphLaunch");
}

int somaopt_device_stats(somaopt_handle* h, const void** stats_dev) {
    if (!h || !stats_dev) return fail(SOMAOPT_E_INVALID, "NULL argument");
    if (int bad = check_handle(h)) return bad;
    *stats_dev = &h->d_state->stats;
    return SOMAOPT_OK;
}

int somaopt_read_stats(somaopt_handle* h, somaopt_stats* out, int64_t* steps_out, void* stream) {
    if (!h || !out) return fail(SOMAOPT_E_INVALID, "NULL argument");
    if (int bad = check_handle(h)) return bad;
    DeviceGuard g(h->device);
    if (!g.ok()) return fail(SOMAOPT_E_HIP, "cannot select the handle's device");
    hipStream_t s = static_cast<hipStream_t>(stream);
    hipError_t e = hipMemcpyAsync(out, &h->d_state->stats, sizeof(somaopt_stats), hipMemcpyDeviceToHost, s);
    if (e == hipSuccess && steps_out)
        e = hipMemcpyAsync(steps_out, h->d_state->step, sizeof(int64_t) * h->n_groups, hipMemcpyDeviceToHost, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    return e == hipSuccess ? SOMAOPT_OK : hip_fail(e, "read_stats");
}

int somaopt_get_plan_info(const somaopt_handle* h, somaopt_plan_info* out) {
    if (!h || !out) return fail(SOMAOPT_E_INVALID, "NULL argument");
    *out = h->info;
    return SOMAOPT_OK;
}

void somaopt_destroy(somaopt_handle* h) {
    if (!h) return;
    // The caller has completed the work it enqueued with this handle (the
    // header's contract) and the handle's own stream only ever captured, so
    // nothing is waited for here; hipFree itself waits for the device.
    DeviceGuard g(h->device);
    free_handle(h);
}

}  // extern "C"
