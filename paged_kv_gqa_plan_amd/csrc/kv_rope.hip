// KV append fused with the rotary position embedding (RoPE) for gfx950.
//
// The decoder the pages run applies RoPE to the step's new query and key heads just before
// the new K/V rows go into the paged pool (Torchlet README: the running example's layers;
// flashlet README: the NHD pool written in place per step, and a RoPE fusion kernel on the
// roadmap). One launch does both: row r's key heads are rotated by the token's position
// and stored in its page slot, its value heads are copied there unchanged, and its query
// heads are rotated in place for the attention call that follows.
//
// Rotation (rotate-half pairs): element i of a head pairs with element i + D/2 and the pair
// turns by pos * f_i, with f_i = theta^(-2i/D) supplied by the host already rounded to
// fp32; the angle is the fp32 product of (float)pos and f_i, its sine and cosine come from
// the device library's sincosf, and the rotated pair is rounded once to the storage type.
// One workgroup per row (a grid sized for the handle's largest plan, striding over the
// plan header's row count): the work per row is a few hundred pairs, memory-light; the
// launch cost dominates, as for the plain append.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fl_internal.h"

namespace fl {
namespace {

constexpr int kThreads = 256;

template <int DT>
struct Store;
template <>
struct Store<FL_BF16> {
    using T = __bf16;
};
template <>
struct Store<FL_F16> {
    using T = _Float16;
};
template <>
struct Store<FL_F32> {
    using T = float;
};

// rotate `heads` head vectors of D values from src into dst (dst may equal src)
template <typename S, int D>
__device__ __forceinline__ void rotate_heads(const S *src, S *dst, int heads, float fpos,
                                             const float *inv_freq) {
    constexpr int H2 = D / 2;
    for (int j = threadIdx.x; j < heads * H2; j += kThreads) {
        const int h = j / H2, i = j - h * H2;
        float sn, cs;
        sincosf(fpos * inv_freq[i], &sn, &cs);
        const float x1 = (float)src[h * D + i], x2 = (float)src[h * D + i + H2];
        dst[h * D + i] = (S)(x1 * cs - x2 * sn);
        dst[h * D + i + H2] = (S)(x2 * cs + x1 * sn);
    }
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void kv_rope_kernel(const RopeArgs a) {
    using S = typename Store<DT>::T;
    const int rows = a.hdr[HDR_APPEND_ROWS];
    if (rows < 0) {  // the plan has no valid append slots (only a replayed launch gets here)
        if (blockIdx.x == 0 && threadIdx.x == 0)
            __hip_atomic_fetch_add(a.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    const int hkv = a.num_kv_heads;
    for (int r = blockIdx.x; r < rows; r += gridDim.x) {
        const float fpos = (float)a.pos[r];
        const int64_t src = (int64_t)r * hkv * D;
        const int64_t dst = (int64_t)a.dst_rows[r] * hkv * D;
        rotate_heads<S, D>((const S *)a.k_new + src, (S *)a.k_pool + dst, hkv, fpos, a.inv_freq);
        const S *vn = (const S *)a.v_new + src;
        S *vp = (S *)a.v_pool + dst;
        for (int j = threadIdx.x; j < hkv * D; j += kThreads) vp[j] = vn[j];
        if (a.q) {
            S *q = (S *)a.q + (int64_t)r * a.num_qo_heads * D;
            rotate_heads<S, D>(q, q, a.num_qo_heads, fpos, a.inv_freq);
        }
    }
}

constexpr int kMaxRopeBlocks = 1024;  // rows beyond this are strided

template <int DT>
hipError_t launch_d(const RopeArgs &a, hipStream_t s) {
    const unsigned grid = (unsigned)(a.max_rows < kMaxRopeBlocks ? a.max_rows : kMaxRopeBlocks);
    if (a.head_dim == 64)
        hipLaunchKernelGGL((kv_rope_kernel<DT, 64>), dim3(grid), dim3(kThreads), 0, s, a);
    else if (a.head_dim == 128)
        hipLaunchKernelGGL((kv_rope_kernel<DT, 128>), dim3(grid), dim3(kThreads), 0, s, a);
    else
        return hipErrorInvalidValue;
    return hipGetLastError();
}

}  // namespace

int launch_kv_append_rope(const RopeArgs &a, void *stream) {
    if (a.max_rows <= 0) return (int)hipErrorInvalidValue;
    hipStream_t s = (hipStream_t)stream;
    switch (a.dtype) {
    case FL_BF16: return (int)launch_d<FL_BF16>(a, s);
    case FL_F16: return (int)launch_d<FL_F16>(a, s);
    case FL_F32: return (int)launch_d<FL_F32>(a, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fl
