// KV append for gfx950: writes a step's new K and V rows into their tokens' page slots of
// the paged pools, before attention reads them (flashlet README, design bullets: the NHD
// pool is written in place by one indexed copy per step and layer).
//
// Query row r of the plan stands for one new token; the plan resolved that token's slot to
// the token row dst_rows[r] = page * P + slot. A token row of the pool is Hkv * D elements,
// contiguous, so the copy of one row is row_bytes contiguous bytes on both sides (a
// multiple of 128). Consecutive lanes take consecutive 16-byte chunks of a row, then of the
// next row, so every wavefront reads and writes whole 128-byte lines. The copy is the same
// for every element type: it moves bytes. The grid is sized for the handle's largest plan
// and the row count comes from the plan header, so one launch serves every plan.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fl_internal.h"

namespace fl {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

constexpr int kThreads = 256;
constexpr int64_t kMaxBlocks = 4096;  // grid-stride beyond this

__global__ __launch_bounds__(kThreads) void kv_append_kernel(
    const int32_t *__restrict__ hdr, int32_t *status, const int32_t *__restrict__ dst_rows,
    const u32x4 *__restrict__ k_new, const u32x4 *__restrict__ v_new, u32x4 *__restrict__ k_pool,
    u32x4 *__restrict__ v_pool, uint32_t row_chunks) {
    const int rows = hdr[HDR_APPEND_ROWS];
    if (rows < 0) {  // the plan has no valid append slots (only a replayed launch gets here)
        if (blockIdx.x == 0 && threadIdx.x == 0)
            __hip_atomic_fetch_add(status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const uint32_t total_chunks = (uint32_t)rows * row_chunks;  // below 2^31 (checked on the host)
    const uint32_t stride = gridDim.x * kThreads;
    for (uint32_t i = blockIdx.x * kThreads + threadIdx.x; i < total_chunks; i += stride) {
        const uint32_t row = i / row_chunks;
        const uint32_t c = i - row * row_chunks;
        const int64_t dst = (int64_t)dst_rows[row] * row_chunks + c;
        const u32x4 k = k_new[i];
        const u32x4 v = v_new[i];
        k_pool[dst] = k;
        v_pool[dst] = v;
    }
}

}  // namespace

int launch_kv_append(const AppendArgs &a, void *stream) {
    if (a.max_rows <= 0 || a.row_bytes <= 0 || a.row_bytes % 16) return (int)hipErrorInvalidValue;
    const uint32_t row_chunks = (uint32_t)(a.row_bytes / 16);
    const int64_t total = (int64_t)a.max_rows * row_chunks;
    if (total >= INT32_MAX) return (int)hipErrorInvalidValue;  // 32-bit chunk indices
    const int64_t blocks = std::min<int64_t>((total + kThreads - 1) / kThreads, kMaxBlocks);
    hipLaunchKernelGGL(kv_append_kernel, dim3((unsigned)blocks), dim3(kThreads), 0, (hipStream_t)stream,
                       a.hdr, a.status, a.dst_rows, (const u32x4 *)a.k_new, (const u32x4 *)a.v_new,
                       (u32x4 *)a.k_pool, (u32x4 *)a.v_pool, row_chunks);
    return (int)hipGetLastError();
}

}  // namespace fl
