// Plan metadata copy: pinned host staging -> the handle's device regions, one small kernel
// that reads the staging buffer over the bus (instead of one DMA transfer per region).
// Offsets are 16-byte aligned; sizes are multiples of 4 bytes.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fl_internal.h"

namespace fl {
namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;

struct PartChunks {
    int64_t first[kStageParts + 1];  // first chunk index of each part; [kStageParts] = total
};

// Every thread copies one 16-byte chunk (or one 4-byte word of a part's tail) of one part:
// all reads of the bus go out at once, so the copy costs one round trip.
__global__ __launch_bounds__(256) void stage_copy_kernel(const StageCopy c, const PartChunks pc) {
    const int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;  // chunk index over all parts
    if (g >= pc.first[kStageParts]) return;
    int p = 0;
    while (g >= pc.first[p + 1]) ++p;
    const int64_t i = g - pc.first[p];
    const char *src = c.src + c.off[p];
    char *dst = c.dst + c.off[p];
    const int64_t n16 = c.bytes[p] / 16;
    if (i < n16) {
        *reinterpret_cast<u32x4 *>(dst + 16 * i) = *reinterpret_cast<const u32x4 *>(src + 16 * i);
    } else {  // the part's last 4, 8 or 12 bytes, one word per thread
        const int64_t b = 16 * n16 + 4 * (i - n16);
        if (b < c.bytes[p]) *reinterpret_cast<uint32_t *>(dst + b) = *reinterpret_cast<const uint32_t *>(src + b);
    }
}

}  // namespace

int launch_stage_copy(const StageCopy &c, void *stream) {
    PartChunks pc;  // 16-byte chunks of each part plus up to 3 tail words
    pc.first[0] = 0;
    for (int p = 0; p < kStageParts; ++p)
        pc.first[p + 1] = pc.first[p] + c.bytes[p] / 16 + (c.bytes[p] % 16) / 4;
    const int64_t total = pc.first[kStageParts];
    if (total == 0) return (int)hipSuccess;
    const int64_t grid = (total + 255) / 256;
    if (grid > INT32_MAX) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(stage_copy_kernel, dim3((unsigned)grid), dim3(256), 0, (hipStream_t)stream, c, pc);
    return (int)hipGetLastError();
}

}  // namespace fl
