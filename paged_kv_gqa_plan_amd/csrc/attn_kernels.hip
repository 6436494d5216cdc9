// gfx950 kernels for paged grouped-query attention: split-KV partial attention over
// 16-key tiles and the log-sum-exp merge of partials.
//
// One workgroup runs one work item: a row block (up to 16 flattened query rows of one
// request and kv head, all sharing one K/V stream) over one key slice. Its waves take the
// slice's 16-key tiles round-robin, each keeping an online softmax state, and fold their
// states together in LDS at the end. A slice that covers its block's whole key range
// writes the final output; otherwise it writes an fp32 partial (o, lse) that the merge
// kernel combines ("A library kernel for decode", What changed: per-slice partial
// results merged into one).
//
// Per 16-key tile, a wave computes
//   S^T[16 keys x 16 rows]  = K_tile . Q^T      (MFMA 16x16x32, 16-bit; 16x16x4, fp32)
//   online softmax per row in the exp2 domain (scale * log2(e) folded into one factor)
//   O^T[d x 16 rows]       += V_tile^T . P^T     (MFMA 16x16x32, 16-bit; 16x16x4, fp32)
// The S^T accumulator layout (lane = row + 16 * (key / 4), 4 keys per lane) is exactly the
// B-operand layout the PV instruction wants for P^T, so P never leaves registers. V is
// stored token-major, so its tokens must move into each lane's registers: for 16-bit
// types one extra MFMA against the identity matrix turns the natural row load
// (4 consecutive d of one token per lane) into 4 tokens of one d per lane, exactly.
// Since the contraction over d can run in any order, each lane loads a contiguous
// 16-byte piece of a K row and the matching piece of the q row, and the output columns
// are permuted the same way, so every global load and store is a 16-byte vector access.
//
// Memory is read straight from the pool: token t of the slice lives in page
// kv_indices[page_base + t / P], slot t % P, at ((page * P + slot) * Hkv + kv_head) * D.
// Tiles start at multiples of 16 tokens and P is a multiple of 16, so one tile never
// crosses a page. Keys at or past the slice end are neither read nor scored; unused
// slots of a page may hold anything, NaN included.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "fl_internal.h"

namespace fl {
namespace {

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8;
typedef __attribute__((ext_vector_type(4))) short s16x4;
typedef __attribute__((ext_vector_type(4))) _Float16 f16x4;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(2))) _Float16 f16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ float shfl_xor(float v, int mask) { return __shfl_xor(v, mask, 64); }

// ---------------------------------------------------------------------------------------
// 16-bit element types
// ---------------------------------------------------------------------------------------
template <int DT>
struct Half;

template <>
struct Half<FL_BF16> {
    static constexpr uint32_t kOne = 0x3F80u;
    __device__ static __forceinline__ f32x4 mma_k32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                       __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma_k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, a),
                                                         __builtin_bit_cast(s16x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
        bf16x2 v = {(__bf16)lo, (__bf16)hi};  // round to nearest even
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ float lo_f(uint32_t v) { return __uint_as_float(v << 16); }
    __device__ static __forceinline__ float hi_f(uint32_t v) { return __uint_as_float(v & 0xFFFF0000u); }
};

template <>
struct Half<FL_F16> {
    static constexpr uint32_t kOne = 0x3C00u;
    __device__ static __forceinline__ f32x4 mma_k32(u32x4 a, u32x4 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                      __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ f32x4 mma_k16(u32x2 a, u32x2 b, f32x4 c) {
        return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, a),
                                                     __builtin_bit_cast(f16x4, b), c, 0, 0, 0);
    }
    __device__ static __forceinline__ uint32_t pack(float lo, float hi) {
        f16x2 v = {(_Float16)lo, (_Float16)hi};  // round to nearest even
        return __builtin_bit_cast(uint32_t, v);
    }
    __device__ static __forceinline__ float lo_f(uint32_t v) { return (float)__builtin_bit_cast(f16x2, v)[0]; }
    __device__ static __forceinline__ float hi_f(uint32_t v) { return (float)__builtin_bit_cast(f16x2, v)[1]; }
};

template <typename T>
__device__ __forceinline__ T ld_global(const void *p) {
    return *reinterpret_cast<const T *>(p);
}

// ---------------------------------------------------------------------------------------
// work item fields (scalar loads; every lane of the workgroup reads the same item)
// ---------------------------------------------------------------------------------------
struct Item {
    int q_start, qo_len, kv_len, page_base, kv_head, row_begin, num_rows, tok_begin, tok_end,
        part_row;
};

__device__ __forceinline__ Item load_item(const int32_t *items) {
    const int32_t *it = items + (size_t)blockIdx.x * FL_WORK_ITEM_INTS;
    Item w;
    w.q_start = it[FL_WI_Q_START];
    w.qo_len = it[FL_WI_QO_LEN];
    w.kv_len = it[FL_WI_KV_LEN];
    w.page_base = it[FL_WI_PAGE_BASE];
    w.kv_head = it[FL_WI_KV_HEAD];
    w.row_begin = it[FL_WI_ROW_BEGIN];
    w.num_rows = it[FL_WI_NUM_ROWS];
    w.tok_begin = it[FL_WI_TOK_BEGIN];
    w.tok_end = it[FL_WI_TOK_END];
    w.part_row = it[FL_WI_PART_ROW];
    return w;
}

// ---------------------------------------------------------------------------------------
// output stores: n fp32 results -> n elements of the output type at out + idx
// ---------------------------------------------------------------------------------------
template <int DT, int N>
__device__ __forceinline__ void store_out(void *out, int64_t idx, const float *res) {
    if constexpr (DT == FL_F32) {
        float *dst = (float *)out + idx;
        static_assert(N % 2 == 0, "even element count");
#pragma unroll
        for (int e = 0; e < N; e += 2)
            *reinterpret_cast<float2 *>(dst + e) = make_float2(res[e], res[e + 1]);
    } else {
        using H = Half<DT>;
        uint16_t *dst = (uint16_t *)out + idx;
        if constexpr (N % 8 == 0) {
#pragma unroll
            for (int e = 0; e < N; e += 8)
                *reinterpret_cast<u32x4 *>(dst + e) =
                    u32x4{H::pack(res[e], res[e + 1]), H::pack(res[e + 2], res[e + 3]),
                          H::pack(res[e + 4], res[e + 5]), H::pack(res[e + 6], res[e + 7])};
        } else if constexpr (N % 4 == 0) {
#pragma unroll
            for (int e = 0; e < N; e += 4)
                *reinterpret_cast<u32x2 *>(dst + e) =
                    u32x2{H::pack(res[e], res[e + 1]), H::pack(res[e + 2], res[e + 3])};
        } else {
#pragma unroll
            for (int e = 0; e < N; e += 2)
                *reinterpret_cast<uint32_t *>(dst + e) = H::pack(res[e], res[e + 1]);
        }
    }
}

// ---------------------------------------------------------------------------------------
// epilogue shared by all element types: fold the waves' softmax states in LDS and write
// either the final rows or the slice's partial rows.
//   o[w][row][d]  unnormalised accumulator of wave w; m / l its running max and sum
// ---------------------------------------------------------------------------------------
template <int D, int NW>
struct Smem {
    float o[NW][kBlockRows][D + 4];
    float m[NW][kBlockRows];
    float l[NW][kBlockRows];
};

template <int DT, int D, int NW>
__device__ __forceinline__ void fold_and_store(const Smem<D, NW> &sm, const Item &w,
                                               const AttnArgs &a) {
    constexpr int TPR = NW * 64 / kBlockRows;  // threads per row
    constexpr int EPT = D / TPR;               // elements per thread
    static_assert(D % TPR == 0 && EPT % 2 == 0, "bad epilogue split");
    const int r = threadIdx.x / TPR;
    const int c0 = (threadIdx.x % TPR) * EPT;
    if (r >= w.num_rows) return;
    float M = kNegInf;
#pragma unroll
    for (int v = 0; v < NW; ++v) M = fmaxf(M, sm.m[v][r]);
    float wt[NW];
    float L = 0.f;
#pragma unroll
    for (int v = 0; v < NW; ++v) {
        wt[v] = (M == kNegInf) ? 0.f : fast_exp2(sm.m[v][r] - M);
        L += sm.l[v][r] * wt[v];
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    float res[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        float acc = 0.f;
#pragma unroll
        for (int v = 0; v < NW; ++v) acc += sm.o[v][r][c0 + e] * wt[v];
        res[e] = acc * inv;
    }
    const float lse2 = L > 0.f ? M + fast_log2(L) : kNegInf;  // log2 domain
    if (w.part_row < 0) {
        const int f = w.row_begin + r;
        const int qi = f / a.group;
        const int qh = f - qi * a.group;
        const int64_t row = (int64_t)(w.q_start + qi) * a.num_qo_heads + w.kv_head * a.group + qh;
        store_out<DT, EPT>(a.out, row * D + c0, res);
        if (a.lse && c0 == 0) a.lse[row] = lse2 * kLn2;
    } else {
        store_out<FL_F32, EPT>(a.part_o, (int64_t)(w.part_row + r) * D + c0, res);
        if (c0 == 0) a.part_lse[w.part_row + r] = lse2;
    }
}

// Online softmax update for one 16-key tile. s holds S^T for keys t0 + 4*grp + e of the
// lane's row; returns P (against the new running max) and the rescale factor alpha.
__device__ __forceinline__ void softmax_tile(const f32x4 &s, int t0, int grp, int tok_end,
                                             int limit, float scale_log2, float &m_run,
                                             float &l_run, float p[4], float &alpha) {
    float sv[4];
    float mt = kNegInf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        const int t = t0 + 4 * grp + e;
        const bool ok = (t < tok_end) && (t <= limit);
        sv[e] = ok ? s[e] * scale_log2 : kNegInf;
        mt = fmaxf(mt, sv[e]);
    }
    mt = fmaxf(mt, shfl_xor(mt, 16));
    mt = fmaxf(mt, shfl_xor(mt, 32));
    const float m_new = fmaxf(m_run, mt);
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    alpha = fast_exp2(m_run - base);
    float ps = 0.f;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
        p[e] = fast_exp2(sv[e] - base);
        ps += p[e];
    }
    l_run = l_run * alpha + ps;
    m_run = m_new;
}

// Query row of column `col` in the block, and the last key it may see (-1: padding column).
struct RowInfo {
    int qi, qh, limit;
    bool ok;
};

__device__ __forceinline__ RowInfo row_info(const Item &w, const AttnArgs &a, int col) {
    RowInfo ri;
    const int f = w.row_begin + col;
    ri.ok = col < w.num_rows;
    ri.qi = f / a.group;
    ri.qh = f - ri.qi * a.group;
    ri.limit = !ri.ok ? -1 : (a.causal ? w.kv_len - w.qo_len + ri.qi : w.kv_len - 1);
    return ri;
}

// ---------------------------------------------------------------------------------------
// bf16 / fp16 kernel
// Lane l: col = l % 16 (row of the block for Q/P/O, key of the tile for K/V), grp = l / 16.
//   K and Q pieces: element d = 32c + 8grp + i (chunk c < D/32, i < 8).
//   PV block j (j < D/16) holds output d = 32(j/2) + 8grp + 4(j%2) + e in element e.
// ---------------------------------------------------------------------------------------
template <int DT, int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_half_kernel(const AttnArgs a) {
    using H = Half<DT>;
    constexpr int NC = D / 32;
    constexpr int NJ = D / 16;
    __shared__ Smem<D, NW> sm;

    const Item w = load_item(a.items);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int P = 1 << a.log2_page;
    const RowInfo ri = row_info(w, a, col);

    u32x4 qf[NC];
    {
        const uint16_t *qp =
            (const uint16_t *)a.q +
            ((int64_t)(w.q_start + ri.qi) * a.num_qo_heads + w.kv_head * a.group + ri.qh) * D +
            8 * grp;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            qf[c] = ri.ok ? ld_global<u32x4>(qp + 32 * c) : u32x4{0, 0, 0, 0};
    }
    // identity operand: element e of lane l is 1 where 4*grp + e == col
    u32x2 ident;
    {
        const uint32_t e0 = (4 * grp + 0 == col) ? H::kOne : 0u;
        const uint32_t e1 = (4 * grp + 1 == col) ? H::kOne : 0u;
        const uint32_t e2 = (4 * grp + 2 == col) ? H::kOne : 0u;
        const uint32_t e3 = (4 * grp + 3 == col) ? H::kOne : 0u;
        ident = u32x2{e0 | (e1 << 16), e2 | (e3 << 16)};
    }

    float m_run = kNegInf, l_run = 0.f;
    f32x4 o[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
    const uint16_t *kb = (const uint16_t *)a.k + (int64_t)w.kv_head * D + 8 * grp;
    const uint16_t *vb = (const uint16_t *)a.v + (int64_t)w.kv_head * D + 8 * grp;
    const int ntiles = (w.tok_end - w.tok_begin + kTileTokens - 1) / kTileTokens;

    for (int tile = wave; tile < ntiles; tile += NW) {
        const int t0 = w.tok_begin + tile * kTileTokens;
        const int page = a.kv_indices[w.page_base + (t0 >> a.log2_page)];
        const bool tv = t0 + col < w.tok_end;
        const int64_t off = ((int64_t)page * P + (t0 & (P - 1)) + col) * slot_stride;
        u32x4 kf[NC], vf[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            kf[c] = tv ? ld_global<u32x4>(kb + off + 32 * c) : u32x4{0, 0, 0, 0};
            vf[c] = tv ? ld_global<u32x4>(vb + off + 32 * c) : u32x4{0, 0, 0, 0};
        }
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) s = H::mma_k32(kf[c], qf[c], s);

        float p[4], alpha;
        softmax_tile(s, t0, grp, w.tok_end, ri.limit, a.scale_log2, m_run, l_run, p, alpha);
        // P = P_hi + P_lo, both in the 16-bit type: the pair carries p to ~16 bits more
        // than one rounding would, so the product with the exact 16-bit V loses nothing
        // measurable. One K=32 instruction contracts [V^T V^T] with [P_hi; P_lo].
        const uint32_t h01 = H::pack(p[0], p[1]), h23 = H::pack(p[2], p[3]);
        const uint32_t l01 = H::pack(p[0] - H::lo_f(h01), p[1] - H::hi_f(h01));
        const uint32_t l23 = H::pack(p[2] - H::lo_f(h23), p[3] - H::hi_f(h23));
        const u32x4 pk = {h01, h23, l01, l23};
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x4 ch = vf[j >> 1];
            const u32x2 va = (j & 1) ? u32x2{ch[2], ch[3]} : u32x2{ch[0], ch[1]};
            const f32x4 vt = H::mma_k16(va, ident, f32x4{0.f, 0.f, 0.f, 0.f});
            const uint32_t v01 = H::pack(vt[0], vt[1]), v23 = H::pack(vt[2], vt[3]);
            o[j] = H::mma_k32(u32x4{v01, v23, v01, v23}, pk, o[j] * alpha);
        }
    }
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);

#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int d0 = 32 * (j >> 1) + 8 * grp + 4 * (j & 1);
        *reinterpret_cast<f32x4 *>(&sm.o[wave][col][d0]) = o[j];
    }
    if (grp == 0) {
        sm.m[wave][col] = m_run;
        sm.l[wave][col] = l_run;
    }
    __syncthreads();
    fold_and_store<DT, D, NW>(sm, w, a);
}

// ---------------------------------------------------------------------------------------
// fp32 kernel (MFMA 16x16x4 f32: one element per lane per instruction)
//   K and Q: lane holds d = grp*(D/4) + s, s < D/4 (contiguous, 16-byte loads).
//   V for key 4grp+e of the tile: lane holds d = (D/16)*col + j, j < D/16.
//   PV block j holds output d = (D/16)*(4grp + e) + j in element e.
// ---------------------------------------------------------------------------------------
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) void attn_f32_kernel(const AttnArgs a) {
    constexpr int NS = D / 4;
    constexpr int NJ = D / 16;
    __shared__ Smem<D, NW> sm;

    const Item w = load_item(a.items);
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int P = 1 << a.log2_page;
    const RowInfo ri = row_info(w, a, col);

    float qf[NS];
    {
        const float *qp =
            (const float *)a.q +
            ((int64_t)(w.q_start + ri.qi) * a.num_qo_heads + w.kv_head * a.group + ri.qh) * D +
            grp * NS;
#pragma unroll
        for (int s4 = 0; s4 < NS; s4 += 4) {
            const float4 v = ri.ok ? ld_global<float4>(qp + s4) : make_float4(0.f, 0.f, 0.f, 0.f);
            qf[s4] = v.x;
            qf[s4 + 1] = v.y;
            qf[s4 + 2] = v.z;
            qf[s4 + 3] = v.w;
        }
    }
    float m_run = kNegInf, l_run = 0.f;
    f32x4 o[NJ];
#pragma unroll
    for (int j = 0; j < NJ; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t slot_stride = (int64_t)a.num_kv_heads * D;
    const float *kb = (const float *)a.k + (int64_t)w.kv_head * D + grp * NS;
    const float *vb = (const float *)a.v + (int64_t)w.kv_head * D + NJ * col;
    const int ntiles = (w.tok_end - w.tok_begin + kTileTokens - 1) / kTileTokens;

    for (int tile = wave; tile < ntiles; tile += NW) {
        const int t0 = w.tok_begin + tile * kTileTokens;
        const int page = a.kv_indices[w.page_base + (t0 >> a.log2_page)];
        const int64_t slot0 = (int64_t)page * P + (t0 & (P - 1));
        float kf[NS];
        {
            const bool tv = t0 + col < w.tok_end;
            const float *kp = kb + (slot0 + col) * slot_stride;
#pragma unroll
            for (int s4 = 0; s4 < NS; s4 += 4) {
                const float4 v = tv ? ld_global<float4>(kp + s4) : make_float4(0.f, 0.f, 0.f, 0.f);
                kf[s4] = v.x;
                kf[s4 + 1] = v.y;
                kf[s4 + 2] = v.z;
                kf[s4 + 3] = v.w;
            }
        }
        float vf[4][NJ];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const int key = 4 * grp + e;
            const bool tv = t0 + key < w.tok_end;
            const float *vp = vb + (slot0 + key) * slot_stride;
#pragma unroll
            for (int j4 = 0; j4 < NJ; j4 += 4) {
                const float4 v = tv ? ld_global<float4>(vp + j4) : make_float4(0.f, 0.f, 0.f, 0.f);
                vf[e][j4] = v.x;
                vf[e][j4 + 1] = v.y;
                vf[e][j4 + 2] = v.z;
                vf[e][j4 + 3] = v.w;
            }
        }
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < NS; ++st) s = __builtin_amdgcn_mfma_f32_16x16x4f32(kf[st], qf[st], s, 0, 0, 0);

        float p[4], alpha;
        softmax_tile(s, t0, grp, w.tok_end, ri.limit, a.scale_log2, m_run, l_run, p, alpha);
#pragma unroll
        for (int j = 0; j < NJ; ++j) o[j] = o[j] * alpha;
#pragma unroll
        for (int e = 0; e < 4; ++e)
#pragma unroll
            for (int j = 0; j < NJ; ++j)
                o[j] = __builtin_amdgcn_mfma_f32_16x16x4f32(vf[e][j], p[e], o[j], 0, 0, 0);
    }
    l_run += shfl_xor(l_run, 16);
    l_run += shfl_xor(l_run, 32);

#pragma unroll
    for (int j = 0; j < NJ; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) sm.o[wave][col][NJ * (4 * grp + e) + j] = o[j][e];
    if (grp == 0) {
        sm.m[wave][col] = m_run;
        sm.l[wave][col] = l_run;
    }
    __syncthreads();
    fold_and_store<FL_F32, D, NW>(sm, w, a);
}

// ---------------------------------------------------------------------------------------
// merge of a row block's slices:  M = max_s lse_s,  w_s = 2^(lse_s - M),
//   out = sum_s w_s o_s / sum_s w_s,  lse = M + log2(sum_s w_s)     (log2 domain)
// 256 threads: 16 per row, D/16 elements each.
// ---------------------------------------------------------------------------------------
template <int DT, int D>
__global__ __launch_bounds__(256) void merge_kernel(const MergeArgs a) {
    constexpr int EPT = D / 16;
    const int32_t *mi = a.merges + (size_t)blockIdx.x * kMergeInts;
    const int q_start = mi[MI_Q_START];
    const int kv_head = mi[MI_KV_HEAD];
    const int row_begin = mi[MI_ROW_BEGIN];
    const int nrows = mi[MI_NUM_ROWS];
    const int part_row = mi[MI_PART_ROW];
    const int ns = mi[MI_NUM_SPLITS];
    const int r = threadIdx.x >> 4;
    const int c0 = (threadIdx.x & 15) * EPT;
    if (r >= nrows) return;
    float M = kNegInf;
    for (int s = 0; s < ns; ++s) M = fmaxf(M, a.part_lse[part_row + s * nrows + r]);
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
    float L = 0.f;
    for (int s = 0; s < ns; ++s) {
        const int pr = part_row + s * nrows + r;
        const float wt = fast_exp2(a.part_lse[pr] - M);
        L += wt;
        const float *src = a.part_o + (int64_t)pr * D + c0;
#pragma unroll
        for (int e = 0; e < EPT; e += 4) {
            const float4 v = ld_global<float4>(src + e);
            acc[e] += wt * v.x;
            acc[e + 1] += wt * v.y;
            acc[e + 2] += wt * v.z;
            acc[e + 3] += wt * v.w;
        }
    }
    const float inv = 1.f / L;
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] *= inv;
    const int f = row_begin + r;
    const int qi = f / a.group;
    const int qh = f - qi * a.group;
    const int64_t row = (int64_t)(q_start + qi) * a.num_qo_heads + kv_head * a.group + qh;
    store_out<DT, EPT>(a.out, row * D + c0, acc);
    if (a.lse && c0 == 0) a.lse[row] = (M + fast_log2(L)) * kLn2;
}

constexpr int kWaves = 4;

template <int DT, int D>
hipError_t launch_attn_t(int n, const AttnArgs &a, hipStream_t s) {
    if constexpr (DT == FL_F32)
        hipLaunchKernelGGL((attn_f32_kernel<D, kWaves>), dim3(n), dim3(kWaves * 64), 0, s, a);
    else
        hipLaunchKernelGGL((attn_half_kernel<DT, D, kWaves>), dim3(n), dim3(kWaves * 64), 0, s, a);
    return hipGetLastError();
}

template <int DT, int D>
hipError_t launch_merge_t(int n, const MergeArgs &a, hipStream_t s) {
    hipLaunchKernelGGL((merge_kernel<DT, D>), dim3(n), dim3(256), 0, s, a);
    return hipGetLastError();
}

}  // namespace

int launch_attention(int dtype, int head_dim, int n, const AttnArgs &a, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (dtype * 1000 + head_dim) {
    case FL_BF16 * 1000 + 64: return (int)launch_attn_t<FL_BF16, 64>(n, a, s);
    case FL_BF16 * 1000 + 128: return (int)launch_attn_t<FL_BF16, 128>(n, a, s);
    case FL_F16 * 1000 + 64: return (int)launch_attn_t<FL_F16, 64>(n, a, s);
    case FL_F16 * 1000 + 128: return (int)launch_attn_t<FL_F16, 128>(n, a, s);
    case FL_F32 * 1000 + 64: return (int)launch_attn_t<FL_F32, 64>(n, a, s);
    case FL_F32 * 1000 + 128: return (int)launch_attn_t<FL_F32, 128>(n, a, s);
    default: return (int)hipErrorInvalidValue;
    }
}

int launch_merge(int dtype, int head_dim, int n, const MergeArgs &a, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    switch (dtype * 1000 + head_dim) {
    case FL_BF16 * 1000 + 64: return (int)launch_merge_t<FL_BF16, 64>(n, a, s);
    case FL_BF16 * 1000 + 128: return (int)launch_merge_t<FL_BF16, 128>(n, a, s);
    case FL_F16 * 1000 + 64: return (int)launch_merge_t<FL_F16, 64>(n, a, s);
    case FL_F16 * 1000 + 128: return (int)launch_merge_t<FL_F16, 128>(n, a, s);
    case FL_F32 * 1000 + 64: return (int)launch_merge_t<FL_F32, 64>(n, a, s);
    case FL_F32 * 1000 + 128: return (int)launch_merge_t<FL_F32, 128>(n, a, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fl
