// Plan metadata copy: pinned host staging -> the handle's device regions, one small kernel
// that reads the staging buffer over the bus (instead of one DMA transfer per region).
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <algorithm>

#include "fl_internal.h"

namespace fl {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

__global__ __launch_bounds__(256) void stage_copy_kernel(const StageCopy c) {
    const int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    const int64_t nthreads = (int64_t)gridDim.x * blockDim.x;
#pragma unroll
    for (int p = 0; p < kStageParts; ++p) {
        const char *src = c.src + c.off[p];
        char *dst = c.dst + c.off[p];
        const int64_t n16 = c.bytes[p] / 16;
        for (int64_t i = tid; i < n16; i += nthreads)
            *reinterpret_cast<u32x4 *>(dst + 16 * i) = *reinterpret_cast<const u32x4 *>(src + 16 * i);
        for (int64_t i = 16 * n16 + 4 * tid; i < c.bytes[p]; i += 4 * nthreads)
            *reinterpret_cast<uint32_t *>(dst + i) = *reinterpret_cast<const uint32_t *>(src + i);
    }
}

}  // namespace

int launch_stage_copy(const StageCopy &c, void *stream) {
    int64_t chunks = 0;
    for (int p = 0; p < kStageParts; ++p) chunks = std::max<int64_t>(chunks, (c.bytes[p] + 15) / 16);
    if (chunks == 0) return (int)hipSuccess;
    const int grid = (int)std::min<int64_t>((chunks + 255) / 256, 1024);
    hipLaunchKernelGGL(stage_copy_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream, c);
    return (int)hipGetLastError();
}

}  // namespace fl
