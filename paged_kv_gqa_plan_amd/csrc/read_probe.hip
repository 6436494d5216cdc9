// Measurement kernels for the benchmark (libfl_read_probe.so, not part of the attention
// library): the read floor of a paged K/V access pattern and the cost of an empty launch.
//
// fl_probe_read_tiles reads exactly the bytes a decode attention launch must read -- for
// every 16-key tile of every (request, kv head), the kv head's slice of 16 token rows of
// the K pool and of the V pool -- and nothing else: no arithmetic beyond folding the loaded
// words into one value per wave (written to `sink`, so the loads cannot be dropped). Each
// workgroup takes an equal contiguous run of the tile list and tile j of the run goes to
// wave j % 4, as in the attention kernel; a wave issues the loads of NB tiles at once and
// waits once, so with NB at least its tile count every load of the launch is in flight at
// the start. Loads are 16 bytes per lane; one instruction covers whole 128-byte lines.
//
//   tile_rows   device int32[num_tiles]: pool row (page * P + slot) * Hkv + kv_head of the
//               tile's first key; its 16 keys are Hkv rows apart
//   k, v        the pools; a row is slice_bytes (head_dim * element size) long
//   slice_bytes 128 or 256 (or, to read whole token rows of every kv head at once, the
//               row's full width 256 or 512 with hkv = 1 and rows page * P + slot)
//   sink        device int32[grid * 4]
// fl_probe_empty launches `grid` workgroups of 256 threads that do nothing.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
constexpr int kWaves = 4;
constexpr int kKeys = 16;

template <int SLICE, int NB>
__global__ __launch_bounds__(256) void read_tiles_kernel(const int32_t *__restrict__ tile_rows, int64_t num_tiles,
                                                         const char *__restrict__ k, const char *__restrict__ v,
                                                         int hkv, int32_t *__restrict__ sink) {
    constexpr int kPieces = SLICE / 16;        // 16-byte pieces per key slice
    constexpr int kKeysPerLoad = 64 / kPieces;  // keys one instruction covers
    constexpr int kLoads = kKeys / kKeysPerLoad;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t t0 = num_tiles * blockIdx.x / gridDim.x;
    const int64_t t1 = num_tiles * (blockIdx.x + 1) / gridDim.x;
    const int key = lane / kPieces, piece = lane % kPieces;
    uint32_t acc = 0;
    for (int64_t base = t0 + wave; base < t1; base += (int64_t)NB * kWaves) {
        u32x4 kv[NB][2][kLoads];
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const int64_t t = base + (int64_t)j * kWaves;
            const int64_t row0 = t < t1 ? tile_rows[t] : tile_rows[t0];
#pragma unroll
            for (int c = 0; c < kLoads; ++c) {
                const int64_t off = (row0 + (int64_t)(c * kKeysPerLoad + key) * hkv) * SLICE + 16 * piece;
                kv[j][0][c] = *reinterpret_cast<const u32x4 *>(k + off);
                kv[j][1][c] = *reinterpret_cast<const u32x4 *>(v + off);
            }
        }
#pragma unroll
        for (int j = 0; j < NB; ++j) {
            const bool live = base + (int64_t)j * kWaves < t1;
#pragma unroll
            for (int c = 0; c < kLoads; ++c) {
                const u32x4 x = kv[j][0][c] ^ kv[j][1][c];
                acc += live ? (x[0] ^ x[1] ^ x[2] ^ x[3]) : 0u;
            }
        }
    }
    // one word per wave
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
    if (lane == 0) sink[blockIdx.x * kWaves + wave] = (int32_t)acc;
}

__global__ __launch_bounds__(256) void empty_kernel() {}

}  // namespace

extern "C" int fl_probe_read_tiles(const int32_t *tile_rows, int64_t num_tiles, const void *k, const void *v,
                                   int hkv, int slice_bytes, int tiles_in_flight, int32_t *sink, int grid,
                                   void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (num_tiles <= 0 || grid <= 0 || hkv <= 0) return (int)hipErrorInvalidValue;
    const char *kp = (const char *)k, *vp = (const char *)v;
    if (slice_bytes == 128 && tiles_in_flight == 8)
        hipLaunchKernelGGL((read_tiles_kernel<128, 8>), dim3(grid), dim3(256), 0, s, tile_rows, num_tiles, kp, vp,
                           hkv, sink);
    else if (slice_bytes == 128 && tiles_in_flight == 2)
        hipLaunchKernelGGL((read_tiles_kernel<128, 2>), dim3(grid), dim3(256), 0, s, tile_rows, num_tiles, kp, vp,
                           hkv, sink);
    else if (slice_bytes == 256 && tiles_in_flight == 4)
        hipLaunchKernelGGL((read_tiles_kernel<256, 4>), dim3(grid), dim3(256), 0, s, tile_rows, num_tiles, kp, vp,
                           hkv, sink);
    else if (slice_bytes == 256 && tiles_in_flight == 2)
        hipLaunchKernelGGL((read_tiles_kernel<256, 2>), dim3(grid), dim3(256), 0, s, tile_rows, num_tiles, kp, vp,
                           hkv, sink);
    else if (slice_bytes == 512 && tiles_in_flight == 2)
        hipLaunchKernelGGL((read_tiles_kernel<512, 2>), dim3(grid), dim3(256), 0, s, tile_rows, num_tiles, kp, vp,
                           hkv, sink);
    else
        return (int)hipErrorInvalidValue;
    return (int)hipGetLastError();
}

extern "C" int fl_probe_empty(int grid, void *stream) {
    if (grid <= 0) return (int)hipErrorInvalidValue;
    hipLaunchKernelGGL(empty_kernel, dim3(grid), dim3(256), 0, (hipStream_t)stream);
    return (int)hipGetLastError();
}
