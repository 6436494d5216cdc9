// Poisoning freed pages of the paged KV pools on gfx950 ("A library kernel for decode",
// closing paragraph: freed pages are poisoned so that a kernel still reading one produces
// NaN rather than stale numbers), and its C entry point.
//
// A page of a pool is page_size * Hkv * D contiguous elements. The page ids travel in the
// launch arguments (up to 256 per launch), so the call needs no device buffer of its own;
// workgroup (x, y) fills 16-byte chunks x * 256 + lane, stepping by the grid's x extent,
// of the y-th listed page, in both pools.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>
#include <cstring>
#include <string>

#include "fl_internal.h"
#include "fl_page_pool.h"

namespace fl {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int kMaxBlocksPerPage = 64;

struct PageIds {
    int32_t id[kPoisonIdsPerLaunch];
};

__global__ __launch_bounds__(kThreads) void kv_poison_kernel(const PageIds ids, u32x4 *__restrict__ k,
                                                             u32x4 *__restrict__ v, uint32_t page_chunks,
                                                             u32x4 pattern) {
    const int64_t base = (int64_t)ids.id[blockIdx.y] * page_chunks;
    for (uint32_t c = blockIdx.x * kThreads + threadIdx.x; c < page_chunks; c += gridDim.x * kThreads) {
        k[base + c] = pattern;
        if (v) v[base + c] = pattern;
    }
}

}  // namespace

int launch_kv_poison(const PoisonArgs &a, void *stream) {
    if (a.n <= 0) return (int)hipSuccess;
    if (a.page_bytes <= 0 || a.page_bytes % 16 || a.page_bytes / 16 > UINT32_MAX / 2)
        return (int)hipErrorInvalidValue;
    const uint32_t page_chunks = (uint32_t)(a.page_bytes / 16);
    const uint32_t bx = (uint32_t)std::min<int64_t>((page_chunks + kThreads - 1) / kThreads, kMaxBlocksPerPage);
    const u32x4 pattern = {a.pattern[0], a.pattern[1], a.pattern[2], a.pattern[3]};
    for (int32_t first = 0; first < a.n; first += kPoisonIdsPerLaunch) {
        const int32_t m = std::min<int32_t>(kPoisonIdsPerLaunch, a.n - first);
        PageIds ids;
        std::memset(&ids, 0, sizeof ids);
        std::memcpy(ids.id, a.page_ids + first, (size_t)m * 4);
        hipLaunchKernelGGL(kv_poison_kernel, dim3(bx, (unsigned)m), dim3(kThreads), 0, (hipStream_t)stream, ids,
                           (u32x4 *)a.k_pool, (u32x4 *)a.v_pool, page_chunks, pattern);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return (int)e;
    }
    return (int)hipSuccess;
}

}  // namespace fl

extern "C" fl_status fl_paged_kv_poison(int32_t dtype, int32_t page_size, int32_t num_kv_heads,
                                        int32_t head_dim, int64_t num_pages, const int32_t *page_ids,
                                        int32_t n, void *k_pool, void *v_pool, void *stream) {
    fl::clear_error();
    uint32_t word;
    int64_t elem;
    switch (dtype) {
    case FL_F16: word = 0x7E007E00u; elem = 2; break;
    case FL_BF16: word = 0x7FC07FC0u; elem = 2; break;
    case FL_F32: word = 0x7FC00000u; elem = 4; break;
    default: return fl::set_error(FL_ERR_UNSUPPORTED, "dtype must be FL_F16, FL_BF16 or FL_F32");
    }
    if (page_size < 1 || num_kv_heads < 1 || head_dim < 1 || num_pages < 1)
        return fl::set_error(FL_ERR_INVALID_ARG, "page_size, num_kv_heads, head_dim and num_pages must be >= 1");
    if (n < 0 || (n > 0 && !page_ids)) return fl::set_error(FL_ERR_INVALID_ARG, "n < 0 or page_ids is NULL");
    if (n == 0) return FL_OK;
    const int64_t page_bytes = (int64_t)page_size * num_kv_heads * head_dim * elem;
    if (page_bytes % 16) return fl::set_error(FL_ERR_INVALID_ARG, "page bytes must be a multiple of 16");
    if (!k_pool) return fl::set_error(FL_ERR_INVALID_ARG, "k_pool is NULL");
    if (((uintptr_t)k_pool | (uintptr_t)v_pool) & 15)
        return fl::set_error(FL_ERR_INVALID_ARG, "pools must be 16-byte aligned");
    for (int32_t i = 0; i < n; ++i)
        if (page_ids[i] < 0 || page_ids[i] >= num_pages)
            return fl::set_error(FL_ERR_INVALID_ARG, "page id " + std::to_string(page_ids[i]) +
                                                         " outside [0, " + std::to_string(num_pages) + ")");
    fl::PoisonArgs a{page_ids, n, k_pool, v_pool, page_bytes, {word, word, word, word}};
    const int e = fl::launch_kv_poison(a, stream);
    if (e != (int)hipSuccess)
        return fl::set_error(FL_ERR_HIP, std::string("poison launch: ") + hipGetErrorName((hipError_t)e));
    return FL_OK;
}
