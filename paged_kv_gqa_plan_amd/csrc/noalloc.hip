// Allocation-free attention run: the same kernel launch as fl_paged_attn_run, with every
// device buffer beyond the caller's inputs and outputs (the plan's metadata, the merge
// tickets, the fp32 partial rows and the status word) placed in one file-scope device
// array of fixed size, `scratch`, which each GPU holds from the library's first use on it
// until the process ends. For callers that cannot allocate device memory; the handle may
// be host-only (created and planned without any HIP call).
//
// The array's name is only a host-side stand-in: its device address is resolved once per
// device with hipGetSymbolAddress (with that device current) and kept; kernels receive
// that address. Every call on one GPU shares the array, so calls that overlap on one GPU
// (other streams, other threads) race; calls ordered on one stream do not.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstring>
#include <mutex>
#include <string>

#include "fl_internal.h"

namespace fl {
namespace {

constexpr int64_t kScratchBytes = 16ll << 20;  // per GPU
static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
char *g_scratch_ptr[kMaxDevices] = {};  // device address of `scratch` per device

// Merge tickets start at zero: cleared by a kernel (no memset node in a caller's stream).
__global__ __launch_bounds__(256) void zero_words(int32_t *p, int n) {
    for (int i = blockIdx.x * 256 + threadIdx.x; i < n; i += gridDim.x * 256) p[i] = 0;
}

int64_t align256(int64_t x) { return (x + 255) / 256 * 256; }

fl_status hip_fail(hipError_t e, const char *what) {
    return set_error(FL_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                     hipGetErrorString(e) + ")");
}

// The device address of `scratch` on the current device `dev` (resolved on first use).
fl_status scratch_on(int dev, char **out) {
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress (scratch)");
        if (!p) return set_error(FL_ERR_HIP, "hipGetSymbolAddress (scratch) returned NULL");
        g_scratch_ptr[dev] = (char *)p;
    }
    *out = g_scratch_ptr[dev];
    return FL_OK;
}

}  // namespace
}  // namespace fl

extern "C" fl_status fl_paged_attn_run_noalloc(fl_handle h, const void *q, const void *k_pool,
                                               const void *v_pool, void *out, float *lse,
                                               void *stream) {
    using namespace fl;
    clear_error();
    NoallocView v{};
    fl_status st = noalloc_view(h, &v);
    if (st != FL_OK) return st;
    if (!q || !k_pool || !v_pool || !out)
        return set_error(FL_ERR_INVALID_ARG, "q, k_pool, v_pool and out must not be NULL");
    if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)out) & 15)
        return set_error(FL_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");

    // layout of this call's data in the scratch array
    const int64_t off_status = 0;
    const int64_t off_rec = 256;  // plan header, then a record slot for every launched workgroup
    const int64_t rec_region = kHdrInts * 4 + (int64_t)std::max<int64_t>(v.grid, v.rec_bytes / (kRecInts * 4)) *
                                                  kRecInts * 4;
    const int64_t off_segs = align256(off_rec + rec_region);
    const int64_t off_steps = align256(off_segs + v.seg_bytes);
    const int64_t off_tickets = align256(off_steps + v.step_bytes);
    const int64_t off_part_o = align256(off_tickets + (int64_t)v.num_merges * 4);
    const int64_t off_part_lse = align256(off_part_o + v.part_rows * v.part_width * 4);
    const int64_t need = align256(off_part_lse + v.part_rows * 4);
    if (need > kScratchBytes)
        return set_error(FL_ERR_CAPACITY,
                         "the plan needs " + std::to_string(need) + " bytes of device scratch (metadata " +
                             std::to_string(off_tickets) + ", partial rows " +
                             std::to_string(need - off_part_o) + "); the allocation-free run holds " +
                             std::to_string(kScratchBytes) + " per GPU");

    int dev = v.device;
    hipError_t e;
    if (dev < 0) {
        if ((e = hipGetDevice(&dev)) != hipSuccess) return hip_fail(e, "hipGetDevice");
    } else if ((e = hipSetDevice(dev)) != hipSuccess) {
        return hip_fail(e, "hipSetDevice");
    }
    if (dev >= kMaxDevices) return set_error(FL_ERR_UNSUPPORTED, "device id >= 64");
    char *base = nullptr;
    if ((st = scratch_on(dev, &base)) != FL_OK) return st;

    // the plan's metadata, from the handle's host copy (pageable memory: each copy has
    // consumed its source when the call returns)
    hipStream_t s = (hipStream_t)stream;
    const struct {
        int64_t off;
        const void *src;
        int64_t bytes;
    } parts[] = {{off_rec, v.hdr, kHdrInts * 4},
                 {off_rec + kHdrInts * 4, v.recs, v.rec_bytes},
                 {off_segs, v.segs, v.seg_bytes},
                 {off_steps, v.steps, v.step_bytes}};
    for (const auto &pt : parts)
        if (pt.bytes > 0 &&
            (e = hipMemcpyAsync(base + pt.off, pt.src, (size_t)pt.bytes, hipMemcpyHostToDevice, s)) != hipSuccess)
            return hip_fail(e, "hipMemcpyAsync (plan metadata)");
    if (v.num_merges > 0) {
        const int blocks = std::min(1024, (v.num_merges + 255) / 256);
        hipLaunchKernelGGL(zero_words, dim3(blocks), dim3(256), 0, s, (int32_t *)(base + off_tickets),
                           v.num_merges);
        if ((e = hipGetLastError()) != hipSuccess) return hip_fail(e, "ticket clear launch");
    }

    AttnArgs a{};
    a.segs = (const int32_t *)(base + off_segs);
    a.wg_rec = (const int32_t *)(base + off_rec);
    a.step_rows = (const int32_t *)(base + off_steps);
    a.tickets = (int32_t *)(base + off_tickets);
    a.status = (int32_t *)(base + off_status);
    a.q = q;
    a.k = k_pool;
    a.v = v_pool;
    a.out = out;
    a.lse = lse;
    a.part_o = (float *)(base + off_part_o);
    a.part_lse = (float *)(base + off_part_lse);
    a.num_qo_heads = v.num_qo_heads;
    a.launch_class = v.launch_class;
    const int le = launch_attention(v.dtype, v.head_dim, v.waves, v.early, v.whole_rows, false, v.grid, a,
                                    stream);
    if (le != (int)hipSuccess) return hip_fail((hipError_t)le, "attention launch (allocation-free)");
    return FL_OK;
}
