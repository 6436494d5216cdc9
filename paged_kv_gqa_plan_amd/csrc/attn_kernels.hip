// gfx950 kernel for paged grouped-query attention: split-KV partial attention over
// 16-key tiles with the log-sum-exp merge of partials done in the same launch.
//
// A row block is up to 16 flattened query rows of one request and kv head, all sharing
// one K/V stream; its keys form 16-key tiles. Long histories are cut into pieces on
// several compute units and the partial results merged ("A library kernel for decode",
// What changed: per-slice partial results merged into one).
//
// Work layout. The plan gives each workgroup a contiguous share of all row blocks' tiles
// (shares of equal estimated time): a list of segments (pieces of row blocks) whose tiles
// the waves take round-robin across the whole share. Each tile's pool row was resolved by
// the plan, so the loads need no page table and no segment state. A workgroup starts from
// its record (one line: the first segment, the share's bounds, each wave's first pool
// rows). Each wave keeps PF tiles of K and V in flight in its own LDS ring, loaded
// straight into LDS with full-cache-line loads and refilled, across segment boundaries,
// as soon as a tile is in registers (memory-bound steps) or after its arithmetic (steps
// the arithmetic bounds). Segment headers, Q rows and windows of pool rows are staged into
// LDS the same way, ahead of use. At each segment's end the waves fold their softmax
// states in LDS and write the
// output rows, or, for a row block cut by a share boundary, fp32 partial rows. The piece
// of a cut block that finishes last merges the partials by log-sum-exp.
//
// Per 16-key tile, a wave computes
//   S^T[16 keys x 16 rows]  = K_tile . Q^T      (MFMA 16x16x32, 16-bit; 16x16x4, fp32)
//   online softmax per row in the exp2 domain (scale * log2(e) folded into one factor)
//   O^T[d x 16 rows]       += V_tile^T . P^T     (MFMA 16x16x16 twice, 16-bit; 16x16x4, fp32)
// The S^T accumulator layout (lane = row + 16 * (key / 4), 4 keys per lane) is exactly the
// B-operand layout the PV instruction wants for P^T, so P never leaves registers. V is
// stored token-major; for 16-bit types the transpose LDS read gives each lane 4 keys of
// one output column, which is the A operand of PV. Since the contraction over d can run
// in any order, each lane holds a contiguous 16-byte piece of a K row and the matching
// piece of the q row, and the output columns are permuted the same way.
//
// Memory is read straight from the pool: token t of a request lives in page
// kv_indices[page_base + t / P], slot t % P, at pool row (page * P + slot) * Hkv + kv_head.
// Tiles start at multiples of 16 tokens and P is a multiple of 16, so one tile never
// crosses a page and every slot a tile touches exists. Keys at or past a segment's end are
// loaded (in bounds) but never scored, and their V rows are replaced by zeros before
// use, so unused slots of a page may hold anything, NaN included.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

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
typedef __attribute__((address_space(3))) char lds_char;

constexpr float kNegInf = -__builtin_inff();
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// Reductions across the four 16-lane groups of a wave (lanes l, l^16, l^32, l^48) with the
// gfx950 lane-swap instructions: a swap of x with itself leaves, in the two results, x of
// lane l and of lane l^16 (or l^32) in some order, so max and + of the pair are the same in
// both lanes of it (bit-identical: both operations are commutative).
// max of the two values a lane holds after a 16- or 32-lane swap, never NaN (scores are
// finite or -inf): one instruction, with none of the quieting that fmaxf adds for operands
// of unknown origin. It takes the swap's result pair, so its operands always come from that
// ordinary VALU instruction, never straight from an MFMA accumulator (the compiler does not
// count inline asm among the readers of an MFMA result that must wait for it).
template <class SwapPair>
__device__ __forceinline__ float max_of_swap(const SwapPair &r) {
    float m;
    asm("v_max_f32 %0, %1, %2" : "=v"(m) : "v"(__uint_as_float(r[0])), "v"(__uint_as_float(r[1])));
    return m;
}
__device__ __forceinline__ float max_xor16(float x) {
    return max_of_swap(__builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false));
}
__device__ __forceinline__ float max_xor32(float x) {
    return max_of_swap(__builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false));
}
__device__ __forceinline__ float sum_xor16(float x) {
    const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
    const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
    return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

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

// Wait until at most N vector-memory loads of this wave are outstanding (loads complete in
// issue order). The memory clobber keeps the LDS reads that follow below the wait.
template <int N>
__device__ __forceinline__ void wait_vm() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// The same for a wave-uniform count n in [LO, HI] known only at run time (a binary search
// over the immediate forms).
template <int LO, int HI>
__device__ __forceinline__ void wait_vm_in(int n) {
    if constexpr (LO == HI) {
        wait_vm<LO>();
    } else {
        constexpr int MID = (LO + HI) / 2;
        if (n <= MID)
            wait_vm_in<LO, MID>(n);
        else
            wait_vm_in<MID + 1, HI>(n);
    }
}
// Wait until this wave's LDS reads have returned (before a slot is refilled).
__device__ __forceinline__ void wait_lds() { asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory"); }

// Loads straight into LDS: lane l's 16 (4) bytes at base + voff land at LDS byte
// lds + 16l (4l); base and lds are wave-uniform. They are issued from inline assembly, so
// the compiler neither counts nor waits for them: every read of their data follows an
// explicit wait_vm (loads complete in issue order), and the compiler's own waits for the
// loads it does see only grow stricter with loads it does not. The address is the
// instruction's scalar base plus the lane's 32-bit offset, so no lane forms a 64-bit
// address of its own.
__device__ __forceinline__ void dma_b128(const void *base, uint32_t voff, const lds_char *lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}
__device__ __forceinline__ void dma_b32(const void *base, uint32_t voff, const lds_char *lds) {
    asm volatile("s_mov_b32 m0, %2\n\tglobal_load_lds_dword %0, %1" ::"v"(voff), "s"(base),
                 "s"((uint32_t)(uintptr_t)lds)
                 : "memory", "m0");
}
__device__ __forceinline__ int lds_int(const lds_char *p) {
    return __builtin_amdgcn_readfirstlane(*(const __attribute__((address_space(3))) int *)p);
}

// compile-time loop: f(std::integral_constant<int, I>) for I = B .. E-1
template <int B, int E, class F>
__device__ __forceinline__ void static_for(F &&f) {
    if constexpr (B < E) {
        f(std::integral_constant<int, B>{});
        static_for<B + 1, E>(f);
    }
}

// ---------------------------------------------------------------------------------------
// segment headers (FL_WORK_ITEM_INTS fields): the first from the workgroup record, the
// next ones copied into a per-wave LDS slot of 256 bytes (lanes 16..63 repeat the fields)
// ---------------------------------------------------------------------------------------
constexpr int kHdrSlot = 256;
__device__ __forceinline__ void stage_header(const lds_char *slot, const int32_t *segs, int seg, int lane) {
    dma_b32(segs + (size_t)seg * FL_WORK_ITEM_INTS, 4u * (uint32_t)(lane & (FL_WORK_ITEM_INTS - 1)), slot);
}

struct Seg {  // wave-uniform fields of the segment being computed
    int q_start, qo_len, kv_len, kv_head, row_begin, num_rows, tok_begin, tok_end, part_row,
        split, num_splits, merge, pos_begin;
};
// Plan metadata is never written while a kernel runs: read through the constant address
// space, wave-uniform reads are scalar loads even after the kernel's own stores (which
// would otherwise make the compiler fall back to vector loads and full vmcnt drains).
typedef __attribute__((address_space(4))) const int32_t cint32;
__device__ __forceinline__ const cint32 *cptr(const int32_t *p) { return (const cint32 *)p; }

// the same fields read from memory with wave-uniform (scalar) loads
template <typename P>
__device__ __forceinline__ Seg seg_fields_mem(P h) {
    Seg s;
    s.q_start = h[FL_WI_Q_START];
    s.qo_len = h[FL_WI_QO_LEN];
    s.kv_len = h[FL_WI_KV_LEN];
    s.kv_head = h[FL_WI_KV_HEAD];
    s.row_begin = h[FL_WI_ROW_BEGIN];
    s.num_rows = h[FL_WI_NUM_ROWS];
    s.tok_begin = h[FL_WI_TOK_BEGIN];
    s.tok_end = h[FL_WI_TOK_END];
    s.part_row = h[FL_WI_PART_ROW];
    s.split = h[FL_WI_SPLIT];
    s.num_splits = h[FL_WI_NUM_SPLITS];
    s.merge = h[FL_WI_MERGE];
    s.pos_begin = h[FL_WI_POS_BEGIN];
    return s;
}
__device__ __forceinline__ Seg seg_fields_lds(const lds_char *h) {
    Seg s;
    s.q_start = lds_int(h + 4 * FL_WI_Q_START);
    s.qo_len = lds_int(h + 4 * FL_WI_QO_LEN);
    s.kv_len = lds_int(h + 4 * FL_WI_KV_LEN);
    s.kv_head = lds_int(h + 4 * FL_WI_KV_HEAD);
    s.row_begin = lds_int(h + 4 * FL_WI_ROW_BEGIN);
    s.num_rows = lds_int(h + 4 * FL_WI_NUM_ROWS);
    s.tok_begin = lds_int(h + 4 * FL_WI_TOK_BEGIN);
    s.tok_end = lds_int(h + 4 * FL_WI_TOK_END);
    s.part_row = lds_int(h + 4 * FL_WI_PART_ROW);
    s.split = lds_int(h + 4 * FL_WI_SPLIT);
    s.num_splits = lds_int(h + 4 * FL_WI_NUM_SPLITS);
    s.merge = lds_int(h + 4 * FL_WI_MERGE);
    s.pos_begin = lds_int(h + 4 * FL_WI_POS_BEGIN);
    return s;
}

// ---------------------------------------------------------------------------------------
// output stores: N fp32 results -> N elements of the output type at out + idx
// ---------------------------------------------------------------------------------------
template <int DT, int N>
__device__ __forceinline__ void store_out(void *out, int64_t idx, const float *res) {
    static_assert(N % 2 == 0, "even element count");
    if constexpr (DT == FL_F32) {
        float *dst = (float *)out + idx;
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int e = 0; e < N; e += 4)
                *reinterpret_cast<float4 *>(dst + e) = make_float4(res[e], res[e + 1], res[e + 2], res[e + 3]);
        } else {
#pragma unroll
            for (int e = 0; e < N; e += 2)
                *reinterpret_cast<float2 *>(dst + e) = make_float2(res[e], res[e + 1]);
        }
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

// Online softmax update for one 16-key tile. s holds S^T for keys t0 + 4*grp + e of the
// lane's row; returns P (against the running max) and the rescale factor alpha.
// The running max moves only when a tile's max exceeds it by more than kSlack (log2
// units): P then stays below 2^kSlack, harmless in fp32, and most tiles need no rescale
// of the accumulator (rescaled reports whether any row of the wave moved). Any reference
// value gives the same result once the final sum divides it out.
constexpr float kSlack = 8.f;

// full: every key of the tile is below tok_end and visible to every real row of the block
// (rows past the block's end see garbage-free zeros and are never stored), so no mask.
// The max is taken on the raw scores and scaled once (scale_log2 > 0 and rounding is
// monotonic, so it equals the max of the scaled scores). The rescale factor is computed
// only in the rare tiles where some row's running max moves (a wave-uniform branch).
// FMA: p = exp2(fma(s, scale, -m)) in one rounding (16-bit outputs, where the last bit of
// p vanishes in the output's rounding); otherwise exp2(s * scale - m), which is exactly 1
// for the key that sets the max (fp32 outputs keep single-key results exact).
// SUM: add the tile's p to l_run here (else the caller sums them itself).
template <bool FMA, bool SUM = true>
__device__ __forceinline__ void softmax_tile(const f32x4 &s, int t0, int grp, int tok_end,
                                             int limit, bool full, float scale_log2, float &m_run,
                                             float &l_run, float p[4], float &alpha,
                                             bool &rescaled) {
    f32x4 x = s;  // masked in place on tiles that need it
    if (!full) {
        // key t0 + 4grp + e, compared as 4grp against tile-relative bounds (nothing per key
        // is computed on the tiles that need no mask)
        const int g4 = 4 * grp, end_rel = tok_end - t0, over = g4 - (limit - t0);
#pragma unroll
        for (int e = 0; e < 4; ++e) x[e] = (g4 < end_rel - e) && (over <= -e) ? x[e] : kNegInf;
    }
    // fmaxf, not the inline-asm max: x may be the MFMA accumulator itself, and the compiler
    // inserts the wait states an MFMA result needs before a VALU read only for instructions
    // it can see (an asm max read stale accumulator values).
    float mt = fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3]));
    mt = max_xor32(max_xor16(mt)) * scale_log2;
    alpha = 1.f;
    const bool move = mt > m_run + kSlack;  // false while both are -inf
    rescaled = __builtin_amdgcn_ballot_w64(move) != 0;
    if (rescaled) {
        const float m_new = move ? mt : m_run;
        alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 while m_run is -inf
        l_run *= alpha;
        m_run = m_new;
    }
    // a full tile makes every row's running max finite
    const float base = (full || m_run != kNegInf) ? m_run : 0.f;
    if constexpr (FMA) {
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(__builtin_fmaf(x[e], scale_log2, -base));
    } else {
        // two roundings, kept apart (no contraction into an FMA): the key that sets the max
        // then gets exactly exp2(0) = 1
#pragma clang fp contract(off)
#pragma unroll
        for (int e = 0; e < 4; ++e) p[e] = fast_exp2(x[e] * scale_log2 - base);
    }
    if constexpr (SUM) l_run += (p[0] + p[1]) + (p[2] + p[3]);
}

// Query row of column `col` in the block, and the last key it may see (-1: padding column).
struct RowInfo {
    int qi, qh, limit;
    bool ok;
};

// f / G for 0 <= f < 2^32 / G. With m = ceil(2^32 / G) = 2^32 / G + e, 0 <= e < 1, the
// product f * m / 2^32 exceeds f / G by f * e / 2^32 < 1 / G, while f / G sits at least
// 1 / G below the next integer, so the high word of f * m is exactly floor(f / G). The
// create call bounds every flattened row so that this holds. G = 1 has m = 0 and adds f.
__device__ __forceinline__ int div_group(int f, const AttnArgs &a) {
    return (int)__umulhi((uint32_t)f, a.group_magic) + (a.group_magic ? 0 : f);
}

// End of the keys every real row of the segment's block may see (the first row has the
// tightest causal limit): tiles wholly below it need no mask.
__device__ __forceinline__ int seg_full_end(const Seg &w, const AttnArgs &a) {
    const int first_limit = a.causal ? w.kv_len - w.qo_len + div_group(w.row_begin, a) : w.kv_len - 1;
    return min(w.tok_end, first_limit + 1);
}

__device__ __forceinline__ RowInfo row_info(const Seg &w, const AttnArgs &a, int col) {
    RowInfo ri;
    const int f = w.row_begin + col;
    ri.ok = col < w.num_rows;
    ri.qi = div_group(f, a);
    ri.qh = f - ri.qi * a.group;
    ri.limit = !ri.ok ? -1 : (a.causal ? w.kv_len - w.qo_len + ri.qi : w.kv_len - 1);
    return ri;
}

// Q rows of a block. Flattened row f = row_begin + r is query row f / G, head
// kv_head * G + f % G. base: q row of the block's first query row and head kv_head * G;
// the returned offset (in rows) of block row r from it is small (rows past num_rows use
// row 0, whose data is never used).
__device__ __forceinline__ int64_t q_block_base(const Seg &w, const AttnArgs &a) {
    return ((int64_t)(w.q_start + div_group(w.row_begin, a)) * a.num_qo_heads + w.kv_head * a.group);
}
__device__ __forceinline__ int q_block_row(const Seg &w, const AttnArgs &a, int r) {
    const int f = w.row_begin + (r < w.num_rows ? r : 0);
    const int qi = div_group(f, a);
    return (qi - div_group(w.row_begin, a)) * a.num_qo_heads + (f - qi * a.group);
}

// ---------------------------------------------------------------------------------------
// tile policy, bf16 / fp16 (MFMA 16x16x32 for QK^T and PV, 16x16x16 for the transpose)
// Lane l: col = l % 16 (row of the block for Q/P/O, key of the tile for K/V), grp = l / 16.
//   K and Q pieces: element d = 32c + 8grp + i (chunk c < D/32, i < 8).
//   PV block j (j < D/16) holds output d = 32(j/2) + 8grp + 4(j%2) + e in element e.
// ---------------------------------------------------------------------------------------
template <int DT, int D>
struct HalfTile {
    using H = Half<DT>;
    static constexpr int NC = D / 32;
    static constexpr int NJ = D / 16;
    // accumulator blocks: the output's NJ, then one more whose every element holds the row's
    // running sum of p (the PV contraction against a block of ones: the sum costs two MFMAs
    // instead of a VALU add per score, and needs no reduction across lanes at the fold)
    static constexpr int NO = NJ + 1;
    static constexpr bool kSumInMma = true;
    struct Frag {
        u32x4 k[NC];   // K piece c of this lane's key
        u32x2 vt[NJ];  // V of keys 4grp .. 4grp+3 at this lane's output column of block j
    };
    struct QOp {
        u32x4 q[NC];
    };

    // ---- 16-byte pieces in LDS -------------------------------------------------------------
    // A row of K, V or Q is S = D/8 pieces of 16 bytes. One 1 KB load writes LDS bytes
    // [16l, 16l+16) from lane l, so lane l fetches whichever global piece belongs there:
    // instruction c covers rows KPL*c .. KPL*c + KPL-1 in full (whole cache lines); lane l
    // reads row KPL*c + l/S into position l % S, which holds piece (l % S) ^ swz(row). The
    // MFMA operand reads take, for lane (row t, group g), piece 4c + g of row t from
    // position (4c + g) ^ swz(t): over any 8 or 16 consecutive lanes (16 rows, one piece)
    // the positions and row parities differ, so the 16-byte LDS reads do not collide on
    // banks.
    static constexpr int S = D / 8;
    static constexpr int KPL = 64 / S;
    static constexpr int kOpBytes = kTileTokens * 2 * D;  // 16 rows of K, V or Q
    static constexpr int kSlotBytes = 2 * kOpBytes;        // K then V
    static constexpr int kQBytes = kOpBytes;
    static constexpr int kLoads = 2 * NC;                  // 1 KB loads per tile
    static_assert(kOpBytes == NC * 1024, "one 1 KB load per 32 d of 16 rows");
    template <int PF>
    static constexpr int ring_bytes() { return PF * kSlotBytes; }

    __device__ static __forceinline__ int swz(int row) {
        return S == 16 ? (row & 15) : ((row & 7) ^ ((row >> 3) & 1));
    }
    // LDS byte offset of lane (row t, group g)'s operand piece c within 16 rows
    __device__ static __forceinline__ uint32_t op_off(int c, int t, int g) {
        return (uint32_t)(t * 2 * D + 16 * ((4 * c + g) ^ swz(t)));
    }
    // V for PV block j through the 16-bit transpose read: lane (i, g) of a 16-lane group
    // receives element i % 4 of the 8 bytes read by lane 16g + 4e + i/4, for e = 0..3. So
    // lane 16g + 4e + q reads key 4g + e at columns 32(j/2) + 8q + 4(j%2) .. +3, and lane
    // (i, g) ends up with V[4g + e][32(j/2) + 8(i/4) + 4(j%2) + i%4], e = 0..3: the A operand
    // of PV (output column of block j for element i, keys of the lane's B-operand group).
    __device__ static __forceinline__ uint32_t vt_off(int j, int lane) {
        const int t = 4 * (lane >> 4) + ((lane >> 2) & 3);
        const int piece = 4 * (j >> 1) + (lane & 3);
        return (uint32_t)(t * 2 * D + 16 * (piece ^ swz(t)) + 8 * (j & 1));
    }

    // Q rows of block segment w into LDS (rows past num_rows repeat row 0).
    // Whole-row blocks (WR): block row h is query head h, whose D/2 values belong in the half
    // of the D-wide operand row that its kv head occupies in a token row (two kv heads of
    // D/2). Both halves of the LDS row receive the head's values; q_fetch zeroes the other
    // half, so the contraction over a whole token row only sees the head's own kv head.
    template <bool WR>
    __device__ static void q_stage(const lds_char *qb, const AttnArgs &a, const Seg &w, int lane) {
        constexpr int kRowB = WR ? D : 2 * D;           // bytes of one q row in memory
        constexpr int kPieces = WR ? S / 2 : S;         // 16-byte pieces of it
        const char *base = (const char *)a.q + q_block_base(w, a) * kRowB;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int r = KPL * c + lane / S;
            const int piece = ((lane % S) ^ swz(r)) & (kPieces - 1);
            dma_b128(base, (uint32_t)(q_block_row(w, a, r) * kRowB + 16 * piece), qb + 1024 * c);
        }
    }
    // kv_half: for whole-row blocks, the half (0 or 1) of the operand row this lane's block
    // row keeps; -1 keeps everything
    __device__ static QOp q_fetch(const lds_char *qb, const RowInfo &ri, int col, int grp, int kv_half = -1) {
        QOp op;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const u32x4 v = *(const __attribute__((address_space(3))) u32x4 *)(qb + op_off(c, col, grp));
            // piece 4c + grp of the row lies in half (4c + grp) / (S / 2) = c / (NC / 2)
            const bool keep = ri.ok && (kv_half < 0 || c / (NC / 2) == kv_half);
            op.q[c] = keep ? v : u32x4{0, 0, 0, 0};
        }
        return op;
    }

    // ---- K/V ring: PF slots of one wave in LDS ---------------------------------------------
    template <int PF>
    struct Ring {
        const lds_char *base;  // this wave's PF slots
        uint32_t goff[NC];     // lane's byte offset in load c from the tile's first key row
        uint32_t roff[NC];     // lane's LDS byte offset of operand piece c
        uint32_t toff[NJ];     // lane's LDS byte offset of its transpose read for PV block j
        Frag f;                // the tile being computed
    };
    template <int PF>
    __device__ static void ring_init(Ring<PF> &r, const lds_char *base, int lane, int hkv) {
        r.base = base;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            const int key = KPL * c + lane / S;
            const int piece = (lane % S) ^ swz(key);
            r.goff[c] = (uint32_t)(key * hkv * 2 * D + 16 * piece);
            r.roff[c] = op_off(c, lane & 15, lane >> 4);
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) r.toff[j] = kOpBytes + vt_off(j, lane);
    }
    // row0: pool row of the tile's first key; consecutive keys are hkv rows apart.
    template <int PF>
    __device__ static void ring_issue(Ring<PF> &r, int slot, const void *k, const void *v, int row0) {
        const int64_t rb = (int64_t)row0 * (2 * D);
        const char *kp = (const char *)k + rb;
        const char *vp = (const char *)v + rb;
        const lds_char *dst = r.base + slot * kSlotBytes;
#pragma unroll
        for (int c = 0; c < NC; ++c) {
            dma_b128(kp, r.goff[c], dst + 1024 * c);
            dma_b128(vp, r.goff[c], dst + kOpBytes + 1024 * c);
        }
    }
    // LATER: tiles issued after this slot's tile that may still be in flight
    template <int LATER, int PF>
    __device__ static void ring_arrive(Ring<PF> &r, int slot) {
        wait_vm<LATER * kLoads>();
        const lds_char *src = r.base + slot * kSlotBytes;
#pragma unroll
        for (int c = 0; c < NC; ++c)
            r.f.k[c] = *(const __attribute__((address_space(3))) u32x4 *)(src + r.roff[c]);
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            r.f.vt[j] = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                           (__attribute__((address_space(3))) s16x4 *)(src + r.toff[j])));
    }
    template <int PF>
    __device__ static const Frag &ring_frag(const Ring<PF> &r, int) { return r.f; }
    __device__ static void ring_release() { wait_lds(); }
    // A slot can be refilled before its tile's arithmetic (it is free once the tile is in
    // registers); the launch chooses: at head_dim 128 always (the arithmetic hides the wait
    // for the LDS reads), at 64 on memory-bound steps (saturated decode 6.92 -> 6.72 us) but
    // not where the arithmetic bounds the step (ragged step 20.1 vs 20.8 us).
    static constexpr bool kCanRefillEarly = true;
    // Issue the first tile ahead of the Q rows at the start: measured faster at head_dim
    // 128 (2-6%), slower at 64 (where the second tile then leaves later).
    static constexpr bool kTileFirst = D >= 128;

    // nrow, kt: with a fused append, the tile's key kt (0..15; -1: none) is the step's new
    // token, whose K and V rows sit in LDS at nrow and nrow + 256 (its pool slot may not hold
    // them yet): the lanes of that key take their operand pieces from there instead.
    __device__ static void compute(const Frag &f, const QOp &q, int t0, int col, int grp, int tok_end,
                                   int limit, bool full, float scale_log2, float &m_run, float &l_run,
                                   f32x4 *o, const lds_char *nrow = nullptr, int kt = -1) {
        u32x4 kk[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) kk[c] = f.k[c];
        u32x2 vt[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) vt[j] = f.vt[j];
        if (kt >= 0) {  // wave-uniform
            if (col == kt) {  // K piece 4c + grp of the key: d = 32c + 8grp .. +7
#pragma unroll
                for (int c = 0; c < NC; ++c)
                    kk[c] = *(const __attribute__((address_space(3))) u32x4 *)(nrow + 16 * (4 * c + grp));
            }
            if (grp == (kt >> 2)) {  // element kt % 4 of V block j: column 32(j/2) + 8(i/4) + 4(j%2) + i%4
                const int e = kt & 3;
#pragma unroll
                for (int j = 0; j < NJ; ++j) {
                    const int d = 32 * (j >> 1) + 8 * (col >> 2) + 4 * (j & 1) + (col & 3);
                    const uint32_t val = *(const __attribute__((address_space(3))) uint16_t *)(nrow + 256 + 2 * d);
                    const uint32_t w = vt[j][e >> 1];
                    vt[j][e >> 1] = (e & 1) ? ((w & 0xFFFFu) | (val << 16)) : ((w & 0xFFFF0000u) | val);
                }
            }
        }
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NC; ++c) s = H::mma_k32(kk[c], q.q[c], s);
        float p[4], alpha;
        bool rescaled;
        softmax_tile<true, false>(s, t0, grp, tok_end, limit, full, scale_log2, m_run, l_run, p, alpha,
                                  rescaled);
        if (rescaled) {
#pragma unroll
            for (int j = 0; j < NO; ++j) o[j] = o[j] * alpha;
        }
        // P = P_hi + P_lo, both in the 16-bit type: the pair carries p to ~16 bits more
        // than one rounding would, so the product with the exact 16-bit V loses nothing
        // measurable. Two K=16 instructions contract V^T with P_hi and with P_lo.
        uint32_t h01 = H::pack(p[0], p[1]), h23 = H::pack(p[2], p[3]);
        // opaque to the optimiser (no instruction): the lo parts then unpack these packed
        // values instead of converting every p a second time
        asm("" : "+v"(h01), "+v"(h23));
        const uint32_t l01 = H::pack(p[0] - H::lo_f(h01), p[1] - H::hi_f(h01));
        const uint32_t l23 = H::pack(p[2] - H::lo_f(h23), p[3] - H::hi_f(h23));
        // keys at or past tok_end may hold anything (NaN included): their V becomes 0
        if (t0 + kTileTokens > tok_end) {
            const int g4 = 4 * grp, r = tok_end - t0;  // key t0 + 4grp + j is below tok_end
            const u32x2 vmask = {(g4 < r ? 0xFFFFu : 0u) | (g4 < r - 1 ? 0xFFFF0000u : 0u),
                                 (g4 < r - 2 ? 0xFFFFu : 0u) | (g4 < r - 3 ? 0xFFFF0000u : 0u)};
#pragma unroll
            for (int j = 0; j < NJ; ++j) vt[j] &= vmask;
        }
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            o[j] = H::mma_k16(vt[j], u32x2{h01, h23}, o[j]);
            o[j] = H::mma_k16(vt[j], u32x2{l01, l23}, o[j]);
        }
        constexpr uint32_t kOnes = H::kOne | H::kOne << 16;
        o[NJ] = H::mma_k16(u32x2{kOnes, kOnes}, u32x2{h01, h23}, o[NJ]);
        o[NJ] = H::mma_k16(u32x2{kOnes, kOnes}, u32x2{l01, l23}, o[NJ]);
    }

    // accumulator element (block j, element e) of lane (col, grp) -> output column d
    __device__ static void to_smem(const f32x4 *o, float *row, int grp) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            *reinterpret_cast<f32x4 *>(row + 32 * (j >> 1) + 8 * grp + 4 * (j & 1)) = o[j];
    }
    __device__ static void from_smem(f32x4 *o, const float *row, int grp) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
            o[j] = *reinterpret_cast<const f32x4 *>(row + 32 * (j >> 1) + 8 * grp + 4 * (j & 1));
    }
};

// ---------------------------------------------------------------------------------------
// tile policy, fp32 (MFMA 16x16x4 f32: one element per lane per instruction)
//   K and Q: lane holds d = grp*(D/4) + s, s < D/4.
//   V for key 4grp+e of the tile: lane holds d = (D/16)*col + j, j < D/16.
//   PV block j holds output d = (D/16)*(4grp + e) + j in element e.
// ---------------------------------------------------------------------------------------
template <int D>
struct F32Tile {
    static constexpr int NS = D / 4;
    static constexpr int NJ = D / 16;
    static constexpr int NO = NJ;            // accumulator blocks: the output's only
    static constexpr bool kSumInMma = false;  // row sums kept per lane (l_run)
    struct Frag {
        float4 k[NS / 4];
        float4 v[4][NJ / 4];
    };
    struct QOp {
        float q[NS];
    };

    // ---- Q rows through LDS (16 rows of 4D bytes, row-major) ------------------------------
    static constexpr int P4 = D / 4;                      // 16-byte pieces per row
    static constexpr int RPL = 64 / P4;                   // rows per 1 KB load
    static constexpr int kQBytes = kBlockRows * 4 * D;
    static constexpr int kLoads = D / 8;                  // 16-byte loads per lane per tile
    template <bool WR>
    __device__ static void q_stage(const lds_char *qb, const AttnArgs &a, const Seg &w, int lane) {
        static_assert(!WR, "whole-row blocks are 16-bit only");
        const char *base = (const char *)a.q + q_block_base(w, a) * (4 * D);
#pragma unroll
        for (int c = 0; c < kQBytes / 1024; ++c) {
            const int r = RPL * c + lane / P4;
            dma_b128(base, (uint32_t)(q_block_row(w, a, r) * 4 * D + 16 * (lane % P4)), qb + 1024 * c);
        }
    }
    __device__ static QOp q_fetch(const lds_char *qb, const RowInfo &ri, int col, int grp, int = -1) {
        QOp op;
        const lds_char *row = qb + col * 4 * D + grp * NS * 4;
#pragma unroll
        for (int s4 = 0; s4 < NS; s4 += 4) {
            const f32x4 v = *(const __attribute__((address_space(3))) f32x4 *)(row + 4 * s4);
            op.q[s4] = ri.ok ? v[0] : 0.f;
            op.q[s4 + 1] = ri.ok ? v[1] : 0.f;
            op.q[s4 + 2] = ri.ok ? v[2] : 0.f;
            op.q[s4 + 3] = ri.ok ? v[3] : 0.f;
        }
        return op;
    }

    // ---- K/V ring: PF register slots per wave (the compiler tracks these loads) -----------
    template <int PF>
    static constexpr int ring_bytes() { return 0; }
    template <int PF>
    struct Ring {
        Frag buf[PF];
        int col, grp, hkv;
    };
    template <int PF>
    __device__ static void ring_init(Ring<PF> &r, const lds_char *, int lane, int hkv) {
        r.col = lane & 15;
        r.grp = lane >> 4;
        r.hkv = hkv;
    }
    template <int PF>
    __device__ static void ring_issue(Ring<PF> &r, int slot, const void *k, const void *v, int row0) {
        load(r.buf[slot], k, v, row0, r.hkv, r.col, r.grp);
    }
    template <int LATER, int PF>
    __device__ static void ring_arrive(Ring<PF> &, int) {
        wait_vm<LATER * kLoads>();
    }
    template <int PF>
    __device__ static const Frag &ring_frag(const Ring<PF> &r, int slot) { return r.buf[slot]; }
    __device__ static void ring_release() {}
    static constexpr bool kCanRefillEarly = false;  // a register slot is busy until the end
    static constexpr bool kTileFirst = false;

    __device__ static void load(Frag &f, const void *k, const void *v, int row0, int hkv, int col,
                                int grp) {
        const float *kp = (const float *)k + (int64_t)(row0 + col * hkv) * D + grp * NS;
#pragma unroll
        for (int c = 0; c < NS / 4; ++c) f.k[c] = ld_global<float4>(kp + 4 * c);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const float *vp = (const float *)v + (int64_t)(row0 + (4 * grp + e) * hkv) * D + NJ * col;
#pragma unroll
            for (int c = 0; c < NJ / 4; ++c) f.v[e][c] = ld_global<float4>(vp + 4 * c);
        }
    }

    __device__ static void compute(const Frag &f, const QOp &q, int t0, int, int grp, int tok_end,
                                   int limit, bool full, float scale_log2, float &m_run, float &l_run,
                                   f32x4 *o, const lds_char * = nullptr, int = -1) {
        f32x4 s = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int c = 0; c < NS / 4; ++c) {
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[c].x, q.q[4 * c], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[c].y, q.q[4 * c + 1], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[c].z, q.q[4 * c + 2], s, 0, 0, 0);
            s = __builtin_amdgcn_mfma_f32_16x16x4f32(f.k[c].w, q.q[4 * c + 3], s, 0, 0, 0);
        }
        float p[4], alpha;
        bool rescaled;
        softmax_tile<false>(s, t0, grp, tok_end, limit, full, scale_log2, m_run, l_run, p, alpha, rescaled);
        if (rescaled) {
#pragma unroll
            for (int j = 0; j < NJ; ++j) o[j] = o[j] * alpha;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            const bool ok = t0 + 4 * grp + e < tok_end;
#pragma unroll
            for (int c = 0; c < NJ / 4; ++c) {
                const float4 v = ok ? f.v[e][c] : make_float4(0.f, 0.f, 0.f, 0.f);
                o[4 * c] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.x, p[e], o[4 * c], 0, 0, 0);
                o[4 * c + 1] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.y, p[e], o[4 * c + 1], 0, 0, 0);
                o[4 * c + 2] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.z, p[e], o[4 * c + 2], 0, 0, 0);
                o[4 * c + 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(v.w, p[e], o[4 * c + 3], 0, 0, 0);
            }
        }
    }

    __device__ static void to_smem(const f32x4 *o, float *row, int grp) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) row[NJ * (4 * grp + e) + j] = o[j][e];
    }
    __device__ static void from_smem(f32x4 *o, const float *row, int grp) {
#pragma unroll
        for (int j = 0; j < NJ; ++j)
#pragma unroll
            for (int e = 0; e < 4; ++e) o[j][e] = row[NJ * (4 * grp + e) + j];
    }
};

// ---------------------------------------------------------------------------------------
// device-scope (cache policy SC1) accesses to the fp32 partial rows: stores write through
// to the point of coherence shared by all XCDs, loads read from it. Buffer instructions
// carry the policy bit on 8- and 16-byte accesses.
// ---------------------------------------------------------------------------------------
constexpr int kDeviceScope = 16;  // SC1
__device__ __forceinline__ __amdgpu_buffer_rsrc_t part_rsrc(const float *base) {
    return __builtin_amdgcn_make_buffer_rsrc((void *)base, 0, 0x7fffffff, 0x00020000);
}
template <int N>
__device__ __forceinline__ void part_store(__amdgpu_buffer_rsrc_t rs, int byte_off, const float *v) {
    static_assert(N % 2 == 0, "even");
#pragma unroll
    for (int e = 0; e < N; e += (N % 4 == 0 ? 4 : 2)) {
        if constexpr (N % 4 == 0)
            __builtin_amdgcn_raw_buffer_store_b128(
                u32x4{__float_as_uint(v[e]), __float_as_uint(v[e + 1]), __float_as_uint(v[e + 2]),
                      __float_as_uint(v[e + 3])},
                rs, byte_off + 4 * e, 0, kDeviceScope);
        else
            __builtin_amdgcn_raw_buffer_store_b64(u32x2{__float_as_uint(v[e]), __float_as_uint(v[e + 1])},
                                                  rs, byte_off + 4 * e, 0, kDeviceScope);
    }
}
template <int N>
__device__ __forceinline__ void part_load(__amdgpu_buffer_rsrc_t rs, int byte_off, float *v) {
    static_assert(N % 2 == 0, "even");
#pragma unroll
    for (int e = 0; e < N; e += (N % 4 == 0 ? 4 : 2)) {
        if constexpr (N % 4 == 0) {
            const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(rs, byte_off + 4 * e, 0, kDeviceScope);
            v[e] = __uint_as_float(x[0]);
            v[e + 1] = __uint_as_float(x[1]);
            v[e + 2] = __uint_as_float(x[2]);
            v[e + 3] = __uint_as_float(x[3]);
        } else {
            const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(rs, byte_off + 4 * e, 0, kDeviceScope);
            v[e] = __uint_as_float(x[0]);
            v[e + 1] = __uint_as_float(x[1]);
        }
    }
}
__device__ __forceinline__ float part_load1(__amdgpu_buffer_rsrc_t rs, int byte_off) {
    return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rs, byte_off, 0, kDeviceScope));
}
__device__ __forceinline__ void part_store1(__amdgpu_buffer_rsrc_t rs, int byte_off, float v) {
    __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), rs, byte_off, 0, kDeviceScope);
}

// ---------------------------------------------------------------------------------------
// LDS for the per-segment fold: the four wave states
// ---------------------------------------------------------------------------------------
// Fields of a piece whose merge ticket is still to be drawn, kept in LDS from its fold to
// the end of the kernel (no global reload of its header on the way to the merge).
enum { PD_MERGE, PD_NUM_SPLITS, PD_NUM_ROWS, PD_PART_ROW, PD_SPLIT, PD_ROW_BEGIN, PD_Q_START,
       PD_KV_HEAD, PD_INTS };
template <int D>
struct Smem {
    alignas(16) float o[4][kBlockRows][D + 4];  // rows of 16-byte multiples
    float m[4][kBlockRows];
    float l[4][kBlockRows];
    int pend[2][PD_INTS];
    int last[2];
};

// Columns of a row handled by thread t of the TPR threads on it: EPT = D / TPR values in
// chunks of up to four floats, chunk q at column CW * (q * TPR + t), so each load or store
// instruction covers whole contiguous stretches of the row across the threads.
template <int D, int TPR>
struct RowSplit {
    static constexpr int EPT = D / TPR;
    static constexpr int CW = EPT < 4 ? EPT : 4;
    static constexpr int NCH = EPT / CW;
    __device__ static __forceinline__ int col(int t, int q) { return CW * (q * TPR + t); }
};

// Merge of a row block's pieces by the piece that finished last:
//   M = max_s lse_s,  w_s = 2^(lse_s - M),  out = sum_s w_s o_s / sum_s w_s.
// The partial rows were written with device-scope stores and are read the same way, a batch
// of pieces at a time with every load of a batch issued before any is used (the running max
// carries across batches by rescaling, as in the online softmax). Partial-row byte
// offsets fit in 32 bits: the workspace is sized from the handle's capacities.
// Final row `row` (q row * Hq + head) from the D fp32 values a thread holds: every chunk,
// or for whole-row blocks only the chunks in the half of the row that the head's kv head
// owns, stored at their column within that half.
template <int DT, int D, int TPR, bool WR>
__device__ __forceinline__ void store_row(const AttnArgs &a, int64_t row, int head, int t, const float *res) {
    using RS = RowSplit<D, TPR>;
    constexpr int CW = RS::CW;
    if constexpr (WR) {
        constexpr int HD = D / 2;  // head_dim of the real kv heads
        static_assert(HD % CW == 0, "chunks do not straddle the halves");
        const int half = head / a.real_group;
#pragma unroll
        for (int q = 0; q < RS::NCH; ++q) {
            const int c0 = RS::col(t, q);
            if (c0 / HD == half) store_out<DT, CW>(a.out, row * HD + (c0 - half * HD), res + q * CW);
        }
    } else {
#pragma unroll
        for (int q = 0; q < RS::NCH; ++q) store_out<DT, CW>(a.out, row * D + RS::col(t, q), res + q * CW);
    }
}

template <int DT, int D, int TPR, int MB, bool WR>
__device__ __forceinline__ void merge_pieces(const Seg &w, const AttnArgs &a, int r, int t) {
    using RS = RowSplit<D, TPR>;
    constexpr int EPT = RS::EPT, CW = RS::CW;
    const int nr = w.num_rows;
    const int base = w.part_row - w.split * nr;
    const int ns = w.num_splits;
    float M = kNegInf, L = 0.f;
    float acc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] = 0.f;
    const __amdgpu_buffer_rsrc_t ro = part_rsrc(a.part_o), rl = part_rsrc(a.part_lse);
    for (int s0 = 0; s0 < ns; s0 += MB) {
        float ls[MB];
        float ov[MB][EPT];
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            if (s0 + i < ns) {  // the vector-memory path of one compute unit bounds the merge:
                                // no loads past the last piece
                const int pr = base + (s0 + i) * nr + r;
                ls[i] = part_load1(rl, pr * 4);
#pragma unroll
                for (int q = 0; q < RS::NCH; ++q) part_load<CW>(ro, (pr * D + RS::col(t, q)) * 4, ov[i] + q * CW);
            } else {
                ls[i] = kNegInf;
#pragma unroll
                for (int e = 0; e < EPT; ++e) ov[i][e] = 0.f;
            }
        }
        float bm = M;
#pragma unroll
        for (int i = 0; i < MB; ++i)
            if (s0 + i < ns) bm = fmaxf(bm, ls[i]);
        const float sc = M == kNegInf ? 0.f : fast_exp2(M - bm);
        L *= sc;
#pragma unroll
        for (int e = 0; e < EPT; ++e) acc[e] *= sc;
#pragma unroll
        for (int i = 0; i < MB; ++i) {
            const float wt = s0 + i < ns ? fast_exp2(ls[i] - bm) : 0.f;
            L += wt;
#pragma unroll
            for (int e = 0; e < EPT; ++e) acc[e] += wt * ov[i][e];
        }
        M = bm;
    }
    const float inv = __builtin_amdgcn_rcpf(L);  // L >= 1 (the largest piece weighs 1)
#pragma unroll
    for (int e = 0; e < EPT; ++e) acc[e] *= inv;
    const int f = w.row_begin + r;
    const int qi = div_group(f, a);
    const int qh = f - qi * a.group;
    const int64_t row = (int64_t)(w.q_start + qi) * a.num_qo_heads + w.kv_head * a.group + qh;
    store_row<DT, D, TPR, WR>(a, row, w.kv_head * a.group + qh, t, acc);
    if (a.lse && t == 0) a.lse[row] = (M + fast_log2(L)) * kLn2;
}

// Fold of one segment across the waves (all waves call it at the same step), then the
// output rows: final rows for a whole row block, device-scope fp32 partial rows for a piece.
// LAST: the workgroup's final fold: no segment follows, so the LDS slots need no release
// (the merge phase has a barrier of its own before it reads the pending pieces' fields).
template <class T, int DT, int D, int NW, bool WR, bool LAST = false, bool HOIST = true>
__device__ __forceinline__ void fold_segment(Smem<D> &sm, const AttnArgs &a, const Seg &cs, int k,
                                             float &m_run, float &l_run, f32x4 *o, int &npend,
                                             int wave, int col, int grp) {
    constexpr int NJ = D / 16;
    constexpr int TPR = NW * 64 / kBlockRows;
    constexpr int EPT = D / TPR;
    l_run = T::kSumInMma ? o[NJ][0] : sum_xor32(sum_xor16(l_run));
    T::to_smem(o, sm.o[wave][col], grp);
    if (grp == 0) {
        sm.m[wave][col] = m_run;
        sm.l[wave][col] = l_run;
    }
    __syncthreads();
    const int r = threadIdx.x / TPR;
    const int t = threadIdx.x % TPR;
    using RS = RowSplit<D, TPR>;
    constexpr int CW = RS::CW;
    if (r < cs.num_rows) {
        // every LDS read of the row first (one round trip), then the arithmetic
        static_assert(CW == 4, "the fold reads whole 16-byte chunks");
        float mv[4], lv[4];
        f32x4 ov[4][RS::NCH];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            mv[v] = sm.m[v][r];
            lv[v] = sm.l[v][r];
#pragma unroll
            for (int q = 0; q < RS::NCH; ++q) ov[v][q] = *reinterpret_cast<const f32x4 *>(&sm.o[v][r][RS::col(t, q)]);
        }
        // HOIST: every read above in flight before the first use below (no instruction: the
        // scheduler may not sink a read past its use here). Measured: 0.5% faster on
        // memory-bound decode, 2% slower where two workgroups share a compute unit.
        if constexpr (HOIST) {
#pragma unroll
            for (int v = 0; v < 4; ++v)
#pragma unroll
                for (int q = 0; q < RS::NCH; ++q) asm volatile("" : "+v"(ov[v][q]));
        }
        float M = kNegInf;
#pragma unroll
        for (int v = 0; v < 4; ++v) M = fmaxf(M, mv[v]);
        float wt[4];
        float L = 0.f;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            wt[v] = (M == kNegInf) ? 0.f : fast_exp2(mv[v] - M);
            L += lv[v] * wt[v];
        }
        const float inv = L > 0.f ? __builtin_amdgcn_rcpf(L) : 0.f;  // exact for powers of two
        float res[EPT];
#pragma unroll
        for (int q = 0; q < RS::NCH; ++q)
#pragma unroll
            for (int c = 0; c < 4; ++c) {
                float acc = 0.f;
#pragma unroll
                for (int v = 0; v < 4; ++v) acc += ov[v][q][c] * wt[v];
                res[q * 4 + c] = acc * inv;
            }
        const float lse2 = L > 0.f ? M + fast_log2(L) : kNegInf;  // log2 domain
        if (cs.part_row < 0) {
            const int f = cs.row_begin + r;
            const int qi = div_group(f, a);
            const int qh = f - qi * a.group;
            const int64_t row = (int64_t)(cs.q_start + qi) * a.num_qo_heads + cs.kv_head * a.group + qh;
            store_row<DT, D, TPR, WR>(a, row, cs.kv_head * a.group + qh, t, res);
            if (a.lse && t == 0) a.lse[row] = lse2 * kLn2;
        } else {
#pragma unroll
            for (int q = 0; q < RS::NCH; ++q)
                part_store<CW>(part_rsrc(a.part_o), ((cs.part_row + r) * D + RS::col(t, q)) * 4, res + q * CW);
            if (t == 0) part_store1(part_rsrc(a.part_lse), (cs.part_row + r) * 4, lse2);
        }
    }
    if (cs.part_row >= 0 && npend < 2) {  // the plan cuts only a share's first and last piece
        if (threadIdx.x == 0) {
            int *pd = sm.pend[npend];
            pd[PD_MERGE] = cs.merge;
            pd[PD_NUM_SPLITS] = cs.num_splits;
            pd[PD_NUM_ROWS] = cs.num_rows;
            pd[PD_PART_ROW] = cs.part_row;
            pd[PD_SPLIT] = cs.split;
            pd[PD_ROW_BEGIN] = cs.row_begin;
            pd[PD_Q_START] = cs.q_start;
            pd[PD_KV_HEAD] = cs.kv_head;
        }
        ++npend;
    }
    if constexpr (!LAST) {
        __syncthreads();  // the LDS slots are free again
        m_run = kNegInf;
        l_run = 0.f;
#pragma unroll
        for (int j = 0; j < T::NO; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
}

// Pool rows of 64 steps of this wave (win .. win+63; past the end: the last step's row)
// into an LDS window of 256 bytes.
__device__ __forceinline__ void stage_rows(const lds_char *dst, const int32_t *rows, int win, int nsteps,
                                           int lane) {
    dma_b32(rows, 4u * (uint32_t)min(win + lane, nsteps - 1), dst);
}

// ---------------------------------------------------------------------------------------
// prefill units (16-bit types): the rows of a prefill chunk in units of up to kQuadBlocks
// (four) 16-row blocks of one request and kv head, kWaveBlocks (one) per wave, over 64-key
// steps. The four waves load a step's four 16-key tiles (one each, the HalfTile ring
// format) into one LDS buffer and all read all four, so a unit streams its keys once for
// its 64 flattened rows; a ring of kQuadBufs buffers keeps the next two steps' loads in
// flight during a step's arithmetic.
// Per step and block: S^T = K Q^T over the four tiles (MFMA 16x16x32), one online-softmax
// update for all 64 keys, and O^T += V^T P^T as two 32-key contractions (16x16x32): the
// contraction runs over keys in any order, so 32-key operand k index 8g + j takes key
// 4g + j of the pair's first tile (j < 4) or 4g + j - 4 of its second, which is exactly how
// the S^T accumulators of the two tiles hold P and how the transpose reads return V.
// ---------------------------------------------------------------------------------------
constexpr int kQuadBufs = 3;
constexpr int kWaveBlocks = kQuadBlocks / kMaxWaves;  // row blocks each wave computes (1)

template <int D>
struct QuadLds {
    static constexpr int kSub = 2 * kTileTokens * 2 * D;  // one 16-key tile: K then V
    static constexpr int kStep = kQuadStepTiles * kSub;
    static constexpr int kQ = kTileTokens * 2 * D;        // one block's 16 Q rows
    // step buffers, then per wave two parities of its blocks' Q rows
    static constexpr int bytes = kQuadBufs * kStep + kMaxWaves * 2 * kWaveBlocks * kQ;
};

// One row block's state in a prefill wave.
template <int DT, int D>
struct UnitBlock {
    Seg w;
    RowInfo ri;
    typename HalfTile<DT, D>::QOp qc;
    int first_limit, last_limit;
    float m_run;
    f32x4 o[D / 16 + 1];  // the output blocks, then the row sums of p (PV against ones)
};

// One 64-key step for the wave's blocks that see some of its keys (act[b]); full[b]: no
// mask needed. K pieces and V columns are read from LDS once and serve every block.
template <int DT, int D>
__device__ __forceinline__ void unit_step(const lds_char *buf, const uint32_t *roff, const uint32_t *toff,
                                          UnitBlock<DT, D> *bs, const bool *act, const bool *full, int t0,
                                          int grp, int tok_end, float scale_log2) {
    using H = Half<DT>;
    constexpr int NC = D / 32, NJ = D / 16, NB = kWaveBlocks;
    f32x4 s[NB][kQuadStepTiles];
#pragma unroll
    for (int u = 0; u < kQuadStepTiles; ++u) {
        const lds_char *src = buf + u * QuadLds<D>::kSub;
        u32x4 kk[NC];
#pragma unroll
        for (int c = 0; c < NC; ++c) kk[c] = *(const __attribute__((address_space(3))) u32x4 *)(src + roff[c]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            s[b][u] = f32x4{0.f, 0.f, 0.f, 0.f};
            if (act[b]) {
#pragma unroll
                for (int c = 0; c < NC; ++c) s[b][u] = H::mma_k32(kk[c], bs[b].qc.q[c], s[b][u]);
            }
        }
    }
    float p[NB][kQuadStepTiles][4];
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (!act[b]) continue;
        if (!full[b]) {
            // key t = t0 + 16u + 4grp + e is visible when t < tok_end and t <= the row's
            // limit, compared as 4grp against step-relative bounds so that nothing per key
            // is computed on the steps that need no mask
            const int g4 = 4 * grp, end_rel = tok_end - t0, over = g4 - (bs[b].ri.limit - t0);
#pragma unroll
            for (int u = 0; u < kQuadStepTiles; ++u)
#pragma unroll
                for (int e = 0; e < 4; ++e) {
                    const int c = kTileTokens * u + e;
                    s[b][u][e] = (g4 < end_rel - c) && (over <= -c) ? s[b][u][e] : kNegInf;
                }
        }
        // one running-max update for the 64 keys (lazy: moves only by more than kSlack)
        float mt = kNegInf;
#pragma unroll
        for (int u = 0; u < kQuadStepTiles; ++u)
            mt = fmaxf(mt, fmaxf(fmaxf(s[b][u][0], s[b][u][1]), fmaxf(s[b][u][2], s[b][u][3])));
        mt = max_xor32(max_xor16(mt)) * scale_log2;
        float &m_run = bs[b].m_run;
        const bool move = mt > m_run + kSlack;  // false while both are -inf
        if (__builtin_amdgcn_ballot_w64(move) != 0) {
            const float m_new = move ? mt : m_run;
            const float alpha = move ? fast_exp2(m_run - m_new) : 1.f;  // 0 while m_run is -inf
            m_run = m_new;
#pragma unroll
            for (int j = 0; j <= NJ; ++j) bs[b].o[j] = bs[b].o[j] * alpha;
        }
        const float base = (full[b] || m_run != kNegInf) ? m_run : 0.f;
#pragma unroll
        for (int u = 0; u < kQuadStepTiles; ++u)
#pragma unroll
            for (int e = 0; e < 4; ++e) p[b][u][e] = fast_exp2(__builtin_fmaf(s[b][u][e], scale_log2, -base));
    }
    // keys at or past tok_end may hold anything (NaN included): their V becomes 0
    const bool tail = t0 + kQuadStepTokens > tok_end;
    constexpr uint32_t kOnes = H::kOne | H::kOne << 16;
    const u32x4 ones = {kOnes, kOnes, kOnes, kOnes};
#pragma unroll
    for (int v = 0; v < kQuadStepTiles / 2; ++v) {
        const int u0 = 2 * v, u1 = 2 * v + 1;
        const lds_char *b0 = buf + u0 * QuadLds<D>::kSub, *b1 = buf + u1 * QuadLds<D>::kSub;
        u32x4 vt[NJ];
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const u32x2 x0 = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(b0 + toff[j])));
            const u32x2 x1 = __builtin_bit_cast(
                u32x2, __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4 *)(b1 + toff[j])));
            vt[j] = u32x4{x0[0], x0[1], x1[0], x1[1]};
        }
        if (tail) {  // wave-uniform: only a piece's last step can reach past tok_end
            // key t0 + 16u + 4grp + j is below tok_end when 4grp < tok_end - t0 - 16u - j
            const int g4 = 4 * grp, r0 = tok_end - t0 - kTileTokens * u0, r1 = tok_end - t0 - kTileTokens * u1;
            const u32x4 m = {(g4 < r0 ? 0xFFFFu : 0u) | (g4 < r0 - 1 ? 0xFFFF0000u : 0u),
                             (g4 < r0 - 2 ? 0xFFFFu : 0u) | (g4 < r0 - 3 ? 0xFFFF0000u : 0u),
                             (g4 < r1 ? 0xFFFFu : 0u) | (g4 < r1 - 1 ? 0xFFFF0000u : 0u),
                             (g4 < r1 - 2 ? 0xFFFFu : 0u) | (g4 < r1 - 3 ? 0xFFFF0000u : 0u)};
#pragma unroll
            for (int j = 0; j < NJ; ++j) vt[j] &= m;
        }
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (!act[b]) continue;
            // P = P_hi + P_lo in the 16-bit type (as for the decode tiles); 32-key operand k
            // index 8g + j is key 4g + j of tile u0 (j < 4) or 4g + j - 4 of tile u1
            const float *p0 = p[b][u0], *p1 = p[b][u1];
            uint32_t h[4] = {H::pack(p0[0], p0[1]), H::pack(p0[2], p0[3]), H::pack(p1[0], p1[1]),
                             H::pack(p1[2], p1[3])};
            asm("" : "+v"(h[0]), "+v"(h[1]), "+v"(h[2]), "+v"(h[3]));
            const u32x4 ph = {h[0], h[1], h[2], h[3]};
            const u32x4 pl = {H::pack(p0[0] - H::lo_f(h[0]), p0[1] - H::hi_f(h[0])),
                              H::pack(p0[2] - H::lo_f(h[1]), p0[3] - H::hi_f(h[1])),
                              H::pack(p1[0] - H::lo_f(h[2]), p1[1] - H::hi_f(h[2])),
                              H::pack(p1[2] - H::lo_f(h[3]), p1[3] - H::hi_f(h[3]))};
#pragma unroll
            for (int j = 0; j < NJ; ++j) {
                bs[b].o[j] = H::mma_k32(vt[j], ph, bs[b].o[j]);
                bs[b].o[j] = H::mma_k32(vt[j], pl, bs[b].o[j]);
            }
            bs[b].o[NJ] = H::mma_k32(ones, ph, bs[b].o[NJ]);
            bs[b].o[NJ] = H::mma_k32(ones, pl, bs[b].o[NJ]);
        }
    }
}

// One wave's finish of one block of a unit piece: the final rows (or, for a piece of a
// block cut by a share boundary, device-scope fp32 partial rows and their log2-domain lse).
template <int DT, int D>
__device__ __forceinline__ void unit_finish(const AttnArgs &a, const UnitBlock<DT, D> &bl, int col, int grp) {
    constexpr int NJ = D / 16;
    const Seg &w = bl.w;
    const float l = bl.o[NJ][0];  // the row's sum of p, in every element of the sum block
    if (!bl.ri.ok) return;
    const float inv = l > 0.f ? __builtin_amdgcn_rcpf(l) : 0.f;  // exact for powers of two
    const float lse2 = l > 0.f ? bl.m_run + fast_log2(l) : kNegInf;
    if (w.part_row < 0) {
        const int64_t row = (int64_t)(w.q_start + bl.ri.qi) * a.num_qo_heads + w.kv_head * a.group + bl.ri.qh;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float res[4] = {bl.o[j][0] * inv, bl.o[j][1] * inv, bl.o[j][2] * inv, bl.o[j][3] * inv};
            store_out<DT, 4>(a.out, row * D + 32 * (j >> 1) + 8 * grp + 4 * (j & 1), res);
        }
        if (a.lse && grp == 0) a.lse[row] = lse2 * kLn2;
    } else {
        const __amdgpu_buffer_rsrc_t rs = part_rsrc(a.part_o);
        const int pr = w.part_row + col;
#pragma unroll
        for (int j = 0; j < NJ; ++j) {
            const float res[4] = {bl.o[j][0] * inv, bl.o[j][1] * inv, bl.o[j][2] * inv, bl.o[j][3] * inv};
            part_store<4>(rs, (pr * D + 32 * (j >> 1) + 8 * grp + 4 * (j & 1)) * 4, res);
        }
        if (grp == 0) part_store1(part_rsrc(a.part_lse), pr * 4, lse2);
    }
}

// A prefill workgroup: its share of unit pieces, step by step. Wave w computes blocks 2w
// and 2w + 1 of each unit; every wave loads tile w of each step.
template <int DT, int D>
__device__ __forceinline__ void quad_path(const int *rv, const AttnArgs &a, const void *k_pool, const void *v_pool,
                                          int hkv, const lds_char *lds, int wv, int lane) {
    using T = HalfTile<DT, D>;
    using UB = UnitBlock<DT, D>;
    constexpr int NJ = D / 16, NC = D / 32, NB = kWaveBlocks;
    constexpr int kL = T::kLoads;           // loads of one wave's tile of a step (K and V)
    constexpr int kQL = NB * NC;            // loads of one wave's Q rows (its blocks)
    static_assert(kQuadStepTiles == kMaxWaves, "one tile of a step per wave");
    const int col = lane & 15, grp = lane >> 4;
    const int seg_b = rv[REC_SEG_BEGIN];
    const int nsteps = rv[REC_STEPS];
    const cint32 *rows = cptr(a.step_rows) + rv[REC_POS];
    // Q rows of block b of this wave, parity par: NB * 2 buffers per wave
    auto qbuf = [&](int par, int b) {
        return lds + kQuadBufs * QuadLds<D>::kStep + ((wv * 2 + par) * NB + b) * QuadLds<D>::kQ;
    };
    typename T::template Ring<1> ring;      // lane offsets of the tile loads and operand reads
    T::ring_init(ring, lds, lane, hkv);
    auto unit_steps = [](const Seg &s) { return (s.tok_end - s.tok_begin + kQuadStepTokens - 1) / kQuadStepTokens; };
    auto seg_of = [&](int unit, int b) {
        return seg_fields_mem(cptr(a.segs) + (size_t)(seg_b + kQuadBlocks * unit + NB * wv + b) * FL_WORK_ITEM_INTS);
    };

    // issue cursor: the unit whose steps are being loaded, and its end step
    int iq = 0;
    Seg iw[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) iw[b] = seg_of(0, b);
    int i_end = unit_steps(iw[0]);
    auto stage_q = [&](int par) {
#pragma unroll
        for (int b = 0; b < NB; ++b) T::template q_stage<false>(qbuf(par, b), a, iw[b], lane);
    };
    // step g's tile of this wave into buffer g % kQuadBufs; at a unit's first step, its Q
    // rows go out first (into the wave's Q buffers of that unit's parity). The tile's pool
    // row was read at the end of the step before (next_row), so its scalar load is never
    // outstanding at the step's LDS waits.
    int next_row = 0;
    auto issue = [&](int g, auto buf) {  // buf: g % kQuadBufs, a compile-time constant
        constexpr int B = decltype(buf)::value;
        if (g == i_end) {
            ++iq;
#pragma unroll
            for (int b = 0; b < NB; ++b) iw[b] = seg_of(iq, b);
            i_end += unit_steps(iw[0]);
            stage_q(iq & 1);
        }
        T::ring_issue(ring, B * kQuadStepTiles + wv, k_pool, v_pool, next_row);
    };
    // compute cursor (taken before issue(1), which moves the issue cursor on when the
    // first piece has a single step)
    int k = 0, q_first = 0;
    UB bs[NB];
#pragma unroll
    for (int b = 0; b < NB; ++b) bs[b].w = iw[b];
    int q_end = unit_steps(bs[0].w);
    stage_q(0);
    T::ring_issue(ring, wv, k_pool, v_pool, rows[wv]);
    if (nsteps > 1) {
        next_row = rows[kQuadStepTiles + wv];
        issue(1, std::integral_constant<int, 1>{});
        if (nsteps > 2) next_row = rows[2 * kQuadStepTiles + wv];
    }

    int npend = 0;
    Seg pend[2][NB];  // the wave's cut blocks (first and last piece of the share)
    // one step; B = g % kQuadBufs is a compile-time constant, so every LDS address of the
    // step is a lane's fixed offset plus an immediate
    auto step = [&](int g, auto buf) {
        constexpr int B = decltype(buf)::value;
        // this wave's tile of step g (and the Q rows of a unit starting there) have landed
        // when at most the next step's loads are outstanding
        if (g + 1 < nsteps) {
            if (g + 1 == q_end)  // step g + 1 starts the next unit: its Q rows went out first
                wait_vm<kL + kQL>();
            else
                wait_vm<kL>();
        } else {
            wait_vm<0>();
        }
        __syncthreads();  // every wave's tile of step g is in LDS; step g - 1's buffer is free
        if (g == q_first) {
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                UB &x = bs[b];
                x.ri = row_info(x.w, a, col);
                x.qc = T::q_fetch(qbuf(k & 1, b), x.ri, col, grp);
                const int f_last = x.w.row_begin + max(x.w.num_rows, 1) - 1;
                x.first_limit = a.causal ? x.w.kv_len - x.w.qo_len + div_group(x.w.row_begin, a) : x.w.kv_len - 1;
                x.last_limit = a.causal ? x.w.kv_len - x.w.qo_len + div_group(f_last, a) : x.w.kv_len - 1;
                x.m_run = kNegInf;
#pragma unroll
                for (int j = 0; j <= NJ; ++j) x.o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
            }
            wait_lds();  // the Q buffers may be refilled from here on
        }
        if (g + 2 < nsteps) issue(g + 2, std::integral_constant<int, (B + 2) % kQuadBufs>{});
        const int t0 = bs[0].w.tok_begin + kQuadStepTokens * (g - q_first);
        const int tok_end = bs[0].w.tok_end;
        bool act[NB], full[NB];
        bool any = false;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            act[b] = bs[b].w.num_rows > 0 && t0 <= bs[b].last_limit;
            full[b] = t0 + kQuadStepTokens <= tok_end && t0 + kQuadStepTokens - 1 <= bs[b].first_limit;
            any = any || act[b];
        }
        if (any)
            unit_step<DT, D>(lds + B * QuadLds<D>::kStep, ring.roff, ring.toff, bs, act, full, t0, grp, tok_end,
                             a.scale_log2);
        if (g + 1 == q_end) {
#pragma unroll
            for (int b = 0; b < NB; ++b)
                if (bs[b].w.num_rows > 0) unit_finish<DT, D>(a, bs[b], col, grp);
            if (bs[0].w.part_row >= 0 && npend < 2) {  // a cut unit: first and last piece only
#pragma unroll
                for (int b = 0; b < NB; ++b) {
                    if (npend == 0)
                        pend[0][b] = bs[b].w;
                    else
                        pend[1][b] = bs[b].w;
                }
                ++npend;
            }
            if (g + 1 < nsteps) {
                ++k;
                q_first = q_end;
#pragma unroll
                for (int b = 0; b < NB; ++b) bs[b].w = seg_of(k, b);
                q_end += unit_steps(bs[0].w);
            }
        }
        // the pool row of step g + 3's tile, for the next step's issue: read at the step's
        // end, after its last LDS wait (a scalar load outstanding at an LDS wait makes that
        // wait cover the scalar load too)
        __builtin_amdgcn_sched_barrier(0);
        if (g + 3 < nsteps) next_row = rows[kQuadStepTiles * (g + 3) + wv];
    };
    static_assert(kQuadBufs == 3, "the step loop is unrolled by the three buffers");
    for (int g = 0; g < nsteps; g += kQuadBufs) {
        step(g, std::integral_constant<int, 0>{});
        if (g + 1 < nsteps) step(g + 1, std::integral_constant<int, 1>{});
        if (g + 2 < nsteps) step(g + 2, std::integral_constant<int, 2>{});
    }
    // merge tickets of this wave's cut blocks: each wave draws its own blocks' tickets once
    // its partial rows are acknowledged; the piece that draws a block's last ticket merges it
    // (the same ordering as the decode path's tickets; a wave writes and merges only its
    // own blocks' rows, so its own wait suffices and no barrier is needed)
    if (npend > 0) {
        __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
        for (int i = 0; i < 2; ++i) {
            if (i >= npend) break;
#pragma unroll
            for (int b = 0; b < NB; ++b) {
                const Seg &ps = i == 0 ? pend[0][b] : pend[1][b];
                if (ps.num_rows == 0) continue;  // an empty slot of the unit
                int last = 0;
                if (lane == 0) {
                    const int done = __hip_atomic_fetch_add(a.tickets + ps.merge, 1, __ATOMIC_RELAXED,
                                                            __HIP_MEMORY_SCOPE_AGENT);
                    if (done == ps.num_splits - 1) {
                        __hip_atomic_store(a.tickets + ps.merge, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                        last = 1;
                    }
                }
                last = __builtin_amdgcn_readfirstlane(last);
                if (last) {
                    const int r = lane >> 2;
                    if (r < ps.num_rows) merge_pieces<DT, D, 4, (D > 64 ? 4 : 8), false>(ps, a, r, lane & 3);
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------------------
// the kernel: one workgroup per equal share of the plan's tiles
// ---------------------------------------------------------------------------------------
// The record and the pools come as separate leading arguments as well: those arrive in
// SGPRs with the dispatch (kernel-argument preloading), so the record's loads go out at
// once, beside the loads of the other arguments instead of after them.
// The new K/V rows of a decode segment (fused append) into a per-wave LDS slot: K at
// [0, 2D), V at [256, 256 + 2D) (4 bytes per lane, the row repeated where 2D < 256).
template <int D>
__device__ __forceinline__ void stage_new_rows(const lds_char *slot, const AttnArgs &a, const Seg &w,
                                               int hkv, int lane) {
    constexpr int kRowB = 2 * D;
    const int64_t off = ((int64_t)w.q_start * hkv + w.kv_head) * kRowB;
    const uint32_t lo = 4u * (uint32_t)(lane % (kRowB / 4));
    dma_b32((const char *)a.k_new + off, lo, slot);
    dma_b32((const char *)a.v_new + off, lo, slot + 256);
}
// ... and from there to the new token's pool slot (token row app_row of the pools), by the
// workgroup that runs the block's last piece (the one whose tiles include the new token).
// The token row is loaded when the segment starts and the rows are written when it ends, so
// the load's latency never sits in front of the loop.
template <int D>
__device__ __forceinline__ void write_new_rows(const lds_char *slot, const AttnArgs &a, const Seg &w,
                                               int app_row, int hkv, int lane) {
    constexpr int kRowB = 2 * D;
    if (lane < kRowB / 16) {
        const int64_t off = ((int64_t)app_row * hkv + w.kv_head) * kRowB + 16 * lane;
        const u32x4 kv = *(const __attribute__((address_space(3))) u32x4 *)(slot + 16 * lane);
        const u32x4 vv = *(const __attribute__((address_space(3))) u32x4 *)(slot + 256 + 16 * lane);
        *reinterpret_cast<u32x4 *>((char *)a.k + off) = kv;
        *reinterpret_cast<u32x4 *>((char *)a.v + off) = vv;
    }
}

// Launch-shape independence: the grid is fixed per launch class, and everything a plan
// changes (how many workgroups have work, causal flag, scale, head grouping) comes from the
// plan header in front of the records, read in the same batch of scalar loads as the
// workgroup's record. A launch whose class stamp is not the plan's touches nothing.
template <class T, int DT, int D, int NW, bool EARLY, bool WR, bool FUSE>
__global__ __launch_bounds__(NW * 64) void attn_kernel(const int32_t *wg_rec, const void *k_pool,
                                                      const void *v_pool, int launch_class,
                                                      const AttnArgs a_in) {
    static_assert(NW == 4 && NW <= kMaxWaves, "four waves per workgroup");
    static_assert(REC_HEAD + FL_WORK_ITEM_INTS <= REC_SEG_BEGIN &&
                  REC_ROWS + kMaxWaves * kRingDepth <= kRecInts, "record layout");
    constexpr int PF = kRingDepth;
    constexpr int NJ = D / 16;
    constexpr int TPR = NW * 64 / kBlockRows;  // fold: threads per row
    constexpr int EPT = D / TPR;               // fold: elements per thread
    static_assert(D % TPR == 0 && EPT % 2 == 0, "bad fold split");
    constexpr int kLoads = T::kLoads;
    static_assert(PF * kLoads < 64, "vmcnt range");
    // Per-wave LDS: the K/V ring (16-bit types), the Q rows of the block being computed,
    // a ring of four segment headers and two 64-step windows of pool rows.
    constexpr int kRingB = T::template ring_bytes<PF>();
    constexpr int kQB = T::kQBytes;
    static_assert(!FUSE || DT != FL_F32, "the fused append runs with 16-bit types");
    constexpr int kNewB = FUSE ? 2 * 512 : 0;  // two slots of new K and V rows
    constexpr int kWaveB = kRingB + kQB + 4 * kHdrSlot + 2 * 256 + kNewB;
    // one LDS area: the decode path's fold state and per-wave rings, or the prefill path's
    // step buffers and Q rows
    constexpr bool kQuads = !WR && !FUSE && DT != FL_F32;
    constexpr int kSmemB = (int)((sizeof(Smem<D>) + 15) / 16 * 16);
    constexpr int kDecodeB = kSmemB + NW * kWaveB;
    constexpr int kQuadB = kQuads ? QuadLds<D>::bytes : 0;
    __shared__ __attribute__((aligned(16))) char lds_raw[kDecodeB > kQuadB ? kDecodeB : kQuadB];
    Smem<D> &sm = *reinterpret_cast<Smem<D> *>(lds_raw);
    char *const wave_lds = lds_raw + kSmemB;

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int col = lane & 15;
    const int grp = lane >> 4;
    const int wv = __builtin_amdgcn_readfirstlane(wave);
    // The plan header and the workgroup record (the share, the first segment and every
    // wave's first pool rows): one batch of scalar loads, issued before anything else.
    // Every launch's grid lies within the record region, whatever the plan.
    const int32_t *rec = wg_rec + kHdrInts + (size_t)blockIdx.x * kRecInts;
    int hv[HDR_USED];
#pragma unroll
    for (int i = 0; i < HDR_USED; ++i) hv[i] = wg_rec[i];
    int rv[REC_ROWS + kMaxWaves * PF];
#pragma unroll
    for (int i = 0; i < REC_ROWS + kMaxWaves * PF; ++i) rv[i] = rec[i];
    // the arguments the first loads need, read in the same batch (consumed here, so they
    // are not sunk below the branch into a second round trip)
    AttnArgs a = a_in;
    asm volatile("" ::"s"(a.segs), "s"(a.step_rows), "s"(a.q), "s"(a.num_qo_heads));
    __builtin_amdgcn_sched_barrier(0);
    if (hv[FUSE ? HDR_FCLASS : HDR_CLASS] != launch_class) {
        // launched for a plan of another class (a stale captured graph): refuse
        if (blockIdx.x == 0 && threadIdx.x == 0)
            __hip_atomic_fetch_add(a_in.status, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        return;
    }
    if ((int)blockIdx.x >= hv[HDR_NUM_GROUPS]) return;  // idle: this plan needs fewer workgroups
    a.causal = hv[HDR_CAUSAL];
    a.scale_log2 = __int_as_float(hv[HDR_SCALE_LOG2]);
    a.num_kv_heads = hv[HDR_HKV];
    a.group = hv[HDR_GROUP];
    a.group_magic = (uint32_t)hv[HDR_GROUP_MAGIC];
    a.real_group = hv[HDR_REAL_GROUP];
    const int hkv = a.num_kv_heads;
    if constexpr (kQuads) {
        if (rv[REC_KIND] == 1) {  // a prefill workgroup
            quad_path<DT, D>(rv, a, k_pool, v_pool, hkv, (const lds_char *)lds_raw, wv, lane);
            return;
        }
    }
    const int seg_b = rv[REC_SEG_BEGIN], seg_e = rv[REC_SEG_END];
    const int pos0 = rv[REC_POS];
    const int nsteps = rv[REC_STEPS];  // steps per wave (at least PF)
    int seg_end = rv[REC_FIRST_END];
    int row_first[PF];  // this wave's (a select over the waves' entries, all in SGPRs)
#pragma unroll
    for (int s = 0; s < PF; ++s) {
        int r = rv[REC_ROWS + s];
#pragma unroll
        for (int w = 1; w < NW; ++w) r = wv == w ? rv[REC_ROWS + w * PF + s] : r;
        row_first[s] = r;
    }
    Seg cs = seg_fields_mem(rv + REC_HEAD);
    int k = seg_b;
    const int32_t *rows = a.step_rows + pos0 + wv * nsteps;
    const lds_char *ring_b = (const lds_char *)wave_lds + wv * kWaveB;
    const lds_char *q_b = ring_b + kRingB;
    const lds_char *hdr_b = q_b + kQB;
    const lds_char *rows_b = hdr_b + 4 * kHdrSlot;
    auto hdr_slot = [&](int seg) { return hdr_b + kHdrSlot * ((seg - seg_b) & 3); };
    const lds_char *new_b = rows_b + 2 * 256;
    auto new_slot = [&](int seg) { return new_b + 512 * ((seg - seg_b) & 1); };

    // Q, the next two headers and the first row windows go out ahead of the ring, or just
    // behind its first tile (whose addresses need the least arithmetic); the first
    // arrival waits for all but the ring slots behind them.
    typename T::template Ring<PF> ring;
    T::ring_init(ring, ring_b, lane, hkv);
    constexpr int kAhead = T::kTileFirst ? 1 : 0;  // ring slots issued before Q
    static_for<0, kAhead>([&](auto si) { T::ring_issue(ring, si, k_pool, v_pool, row_first[si]); });
    T::template q_stage<WR>(q_b, a, cs, lane);
    if constexpr (FUSE) stage_new_rows<D>(new_slot(seg_b), a, cs, hkv, lane);
    stage_header(hdr_slot(seg_b + 1), a.segs, min(seg_b + 1, seg_e - 1), lane);
    stage_header(hdr_slot(seg_b + 2), a.segs, min(seg_b + 2, seg_e - 1), lane);
    stage_rows(rows_b, rows, 0, nsteps, lane);
    stage_rows(rows_b + 256, rows, 64, nsteps, lane);
    static_for<kAhead, PF>([&](auto si) { T::ring_issue(ring, si, k_pool, v_pool, row_first[si]); });
    wait_vm<(PF - kAhead) * kLoads>();
    // whole-row blocks: block row h keeps the half of the operand row of its kv head
    auto kv_half = [&](const RowInfo &x) { return WR ? x.qh / a.real_group : -1; };
    RowInfo ri = row_info(cs, a, col);
    typename T::QOp qc = T::q_fetch(q_b, ri, col, grp, kv_half(ri));
    // the piece that holds the block's newest key writes the new rows to the pools (at its end)
    auto new_token_row = [&](const Seg &w) {
        return FUSE && wv == 0 && w.tok_end == w.kv_len ? a.append_rows[w.q_start] : -1;
    };
    int app_row = new_token_row(cs);
    int ntile = (cs.tok_end - cs.tok_begin + kTileTokens - 1) / kTileTokens;
    int full_end = seg_full_end(cs, a);

    float m_run = kNegInf, l_run = 0.f;
    f32x4 o[T::NO];
#pragma unroll
    for (int j = 0; j < T::NO; ++j) o[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    int npend = 0;  // pieces whose merge ticket is still to be drawn (fields in sm.pend)

    // ---- the step stream: PF tiles of K and V in flight per wave -------------------------
    // Every slot of the ring is in flight until its step (padding steps re-read a real tile
    // and are never scored). Segments start on multiples of PF steps; only the last one may
    // end between them, so the last group holds e = nsteps - p0 <= PF steps and the one
    // before it refills only those e slots. Loads complete in issue order, so at slot s of a
    // group at most PF - 1 later tiles are outstanding behind it (fewer in those two groups:
    // PF - 1 - s + min(s, e) in the one before the last, e - 1 - s in the last), and at a
    // group's top everything issued before the previous group's refills has landed
    // (headers, Q, row windows included).
    int win = 0;  // window of the last refill
    // One group of PF steps (e of them real in the last group, e refills in the one before
    // it, PF elsewhere). The last group issues no refills, so nothing is in flight when the
    // final fold starts.
    auto group = [&](int p0, auto refill, int e) {
        constexpr bool kRefill = decltype(refill)::value;
        if (kRefill || e == PF)
            wait_vm<PF * kLoads>();
        else
            wait_vm_in<kLoads, PF * kLoads>(e * kLoads);
        if (p0 == seg_end) {  // the same step in every wave: segment k is done
            if constexpr (FUSE)
                if (app_row >= 0) write_new_rows<D>(new_slot(k), a, cs, app_row, hkv, lane);
            fold_segment<T, DT, D, NW, WR, false, EARLY>(sm, a, cs, k, m_run, l_run, o, npend, wave, col, grp);
            ++k;
            cs = seg_fields_lds(hdr_slot(k));
            seg_end = k + 1 < seg_e ? lds_int(hdr_slot(k + 1) + 4 * FL_WI_POS_BEGIN) : nsteps;
            ri = row_info(cs, a, col);
            qc = T::q_fetch(q_b, ri, col, grp, kv_half(ri));
            app_row = new_token_row(cs);
            ntile = (cs.tok_end - cs.tok_begin + kTileTokens - 1) / kTileTokens;
            full_end = seg_full_end(cs, a);
            wait_lds();  // the slot of header k - 2 is free
            stage_header(hdr_slot(k + 2), a.segs, min(k + 2, seg_e - 1), lane);
        }
        if (p0 + PF == seg_end && k + 1 < seg_e) {
            // the last group of segment k: the Q rows of segment k + 1 go out before this
            // group's refills, so they have landed at the next group's top
            const Seg ns = seg_fields_lds(hdr_slot(k + 1));
            wait_lds();  // this wave's reads of the Q rows are done
            T::template q_stage<WR>(q_b, a, ns, lane);
            if constexpr (FUSE) stage_new_rows<D>(new_slot(k + 1), a, ns, hkv, lane);
        }
        int nrow[PF];  // pool rows of this group's refills (entries past nsteps unused)
        if constexpr (kRefill) {
#pragma unroll
            for (int s = 0; s < PF; ++s) {
                const int q = p0 + PF + s;
                nrow[s] = lds_int(rows_b + 256 * ((q >> 6) & 1) + 4 * (q & 63));
            }
        }
        static_for<0, PF>([&](auto si) {
            constexpr int s = decltype(si)::value;
            if (!kRefill && s > 0 && s >= e) return;  // past the share's last step
            const int p = p0 + s;
            const int j = (p - cs.pos_begin) * NW + wv;  // tile of the segment (wave-uniform)
            constexpr int kLater = kRefill ? PF - 1 : PF - 1 - s;
            if ((!kRefill || s > 0) && e != PF) {  // fewer tiles behind: wait for the exact count
                const int later = kRefill ? PF - 1 - s + min(s, e) : e - 1 - s;
                wait_vm_in<0, kLater * kLoads>(later * kLoads);
            }
            T::template ring_arrive<kLater>(ring, s);
            auto refill = [&] {
                if constexpr (kRefill) {
                    const int q = p + PF;
                    if (s > 0 && s >= e) return;  // past the share's last step
                    T::ring_release();
                    if ((q >> 6) != win) {  // first refill in window q/64: fetch the next window
                        win = q >> 6;
                        stage_rows(rows_b + 256 * ((win + 1) & 1), rows, 64 * (win + 1), nsteps, lane);
                    }
                    T::ring_issue(ring, s, k_pool, v_pool, nrow[s]);
                }
            };
            // An LDS slot is free once its tile is in registers: refill it before computing,
            // so the load's latency runs under the arithmetic. A register slot is free only
            // after the arithmetic.
            constexpr bool kEarly = T::kCanRefillEarly && EARLY;
            if constexpr (kEarly) refill();
            if (j < ntile) {
                const int t0 = cs.tok_begin + j * kTileTokens;
                // fused append: the newest key (kv_len - 1) comes from the staged new rows
                const int kt = FUSE && cs.kv_len - 1 - t0 < kTileTokens ? cs.kv_len - 1 - t0 : -1;
                T::compute(T::ring_frag(ring, s), qc, t0, col, grp, cs.tok_end, ri.limit,
                           t0 + kTileTokens <= full_end, a.scale_log2, m_run, l_run, o,
                           new_slot(k), kt);
            }
            if constexpr (!kEarly) refill();
            __builtin_amdgcn_sched_barrier(0);
        });
    };
    int p0 = 0;
    for (; p0 + PF < nsteps; p0 += PF) group(p0, std::true_type{}, min(PF, nsteps - p0 - PF));
    group(p0, std::false_type{}, nsteps - p0);
    if constexpr (FUSE)
        if (app_row >= 0) write_new_rows<D>(new_slot(k), a, cs, app_row, hkv, lane);
    fold_segment<T, DT, D, NW, WR, true, EARLY>(sm, a, cs, k, m_run, l_run, o, npend, wave, col, grp);

    // ---- merge tickets of the partial pieces (at most the first and the last) -----------
    // The partial rows went out as device-scope stores; each wave waits for their
    // acknowledgement before the workgroup draws its tickets with device-scope atomics (one
    // lane per piece, both in one instruction), so the piece that draws a row block's last
    // ticket finds every other piece complete.
    // Ordering, in the terms of the CDNA3/CDNA4 ISA's scope bits (SC1 set, SC0 clear:
    // device scope) and of LLVM's AMDGPU memory model for gfx942/gfx950:
    //   1. a device-scope store writes through this XCD's L2 to the coherence point all
    //      XCDs share, and is acknowledged (vmcnt, which counts stores on this target) only
    //      once it is there; s_waitcnt(0) then the barrier: every wave's rows are there;
    //   2. the ticket is an agent-scope atomic, performed at that same point; atomics on one
    //      address are totally ordered, so the last ticket is drawn after every other
    //      piece's increment, each made after that piece's acknowledged stores;
    //   3. the merging piece reads the partial rows with device-scope loads, which do not
    //      take lines from its own L2, and issues them only after its atomic returned (the
    //      loads depend on the returned value).
    // This is the agent-scope release/acquire code sequence of that memory model without
    // its L2 write-back and invalidate steps, which only order non-device-scope accesses:
    // every access another workgroup reads here is device scope. A whole-cache write-back
    // and invalidate (the fence form) measured 5-7x slower on split workloads.
    if (npend > 0) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x < 2) {
            int last = 0;
            if ((int)threadIdx.x < npend) {
                const int *pd = sm.pend[threadIdx.x];
                const int tk = pd[PD_MERGE];
                const int done = __hip_atomic_fetch_add(a.tickets + tk, 1, __ATOMIC_RELAXED,
                                                        __HIP_MEMORY_SCOPE_AGENT);
                if (done == pd[PD_NUM_SPLITS] - 1) {
                    __hip_atomic_store(a.tickets + tk, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    last = 1;
                }
            }
            sm.last[threadIdx.x] = last;
        }
        __syncthreads();
        auto pend_seg = [&](int i) {
            const lds_char *pd = (const lds_char *)sm.pend[i];
            Seg ps{};
            ps.merge = lds_int(pd + 4 * PD_MERGE);
            ps.num_splits = lds_int(pd + 4 * PD_NUM_SPLITS);
            ps.num_rows = lds_int(pd + 4 * PD_NUM_ROWS);
            ps.part_row = lds_int(pd + 4 * PD_PART_ROW);
            ps.split = lds_int(pd + 4 * PD_SPLIT);
            ps.row_begin = lds_int(pd + 4 * PD_ROW_BEGIN);
            ps.q_start = lds_int(pd + 4 * PD_Q_START);
            ps.kv_head = lds_int(pd + 4 * PD_KV_HEAD);
            return ps;
        };
        const bool both = npend == 2 && lds_int((const lds_char *)&sm.last[0]) &&
                          lds_int((const lds_char *)&sm.last[1]);
        // A block's merge takes its pieces kMbWide (more than eight rows) or kMbNarrow (up to
        // eight) at a time whichever way the workgroup's threads are split over its rows: the
        // batches fix the order of the arithmetic, so a block's rows come out bit for bit
        // the same whichever workgroup merges it. (fp32 rows take half as many per batch:
        // twice the registers per piece.)
        constexpr int kMbWide = DT == FL_F32 ? 4 : 8, kMbNarrow = 2 * kMbWide;
        if (both) {
            // both pieces merge here: each half of the workgroup (two waves) takes one, so
            // the two merges' loads are in flight together instead of one after the other
            constexpr int kHalf = NW * 64 / 2;
            const int i = threadIdx.x / kHalf;
            const int u = threadIdx.x % kHalf;
            const Seg ps = pend_seg(i);
            if (ps.num_rows > kBlockRows / 2) {
                constexpr int TPRH = TPR / 2;
                const int r = u / TPRH;
                if (r < ps.num_rows) merge_pieces<DT, D, TPRH, kMbWide, WR>(ps, a, r, u % TPRH);
            } else {
                const int r = u / TPR;
                if (r < ps.num_rows) merge_pieces<DT, D, TPR, kMbNarrow, WR>(ps, a, r, u % TPR);
            }
        } else {
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                if (i >= npend || !lds_int((const lds_char *)&sm.last[i])) continue;
                const Seg ps = pend_seg(i);
                if (ps.num_rows > kBlockRows / 2) {
                    const int r = threadIdx.x / TPR;
                    if (r < ps.num_rows) merge_pieces<DT, D, TPR, kMbWide, WR>(ps, a, r, threadIdx.x % TPR);
                } else {  // up to 8 rows: twice the threads per row, twice the pieces per batch
                    constexpr int TPR2 = 2 * TPR;
                    const int r2 = threadIdx.x / TPR2;
                    if (r2 < ps.num_rows)
                        merge_pieces<DT, D, TPR2, kMbNarrow, WR>(ps, a, r2, threadIdx.x % TPR2);
                }
            }
        }
    }
}

template <int DT, int D>
struct TileFor {
    using type = HalfTile<DT, D>;
};
template <int D>
struct TileFor<FL_F32, D> {
    using type = F32Tile<D>;
};

template <int DT, int D, int NW, bool EARLY, bool WR = false, bool FUSE = false>
hipError_t launch_t(int n, const AttnArgs &a, hipStream_t s) {  // n: workgroups
    using T = typename TileFor<DT, D>::type;
    hipLaunchKernelGGL((attn_kernel<T, DT, D, NW, EARLY, WR, FUSE>), dim3(n), dim3(NW * 64), 0, s, a.wg_rec,
                       a.k, a.v, a.launch_class, a);
    return hipGetLastError();
}

// Fused append: decode-only plans (one workgroup per compute unit, early refill), 16-bit.
template <int DT>
hipError_t launch_fused(int head_dim, bool whole_rows, int n, const AttnArgs &a, hipStream_t s) {
    if (whole_rows) return head_dim == 128 ? launch_t<DT, 128, 4, true, true, true>(n, a, s) : hipErrorInvalidValue;
    if (head_dim == 64) return launch_t<DT, 64, 4, true, false, true>(n, a, s);
    if (head_dim == 128) return launch_t<DT, 128, 4, true, false, true>(n, a, s);
    return hipErrorInvalidValue;
}

// One instantiation where the refill point cannot vary: always early at head_dim 128,
// never for fp32 (register ring).
template <int DT, int D>
hipError_t launch_w(int waves, bool early, int n, const AttnArgs &a, hipStream_t s) {
    if (waves != 4) return hipErrorInvalidValue;
    if constexpr (DT == FL_F32) return launch_t<DT, D, 4, false>(n, a, s);
    else if constexpr (D >= 128) return launch_t<DT, D, 4, true>(n, a, s);
    else return early ? launch_t<DT, D, 4, true>(n, a, s) : launch_t<DT, D, 4, false>(n, a, s);
}

}  // namespace

int launch_attention(int dtype, int head_dim, int waves, bool early, bool whole_rows, bool fuse_append,
                     int n, const AttnArgs &a, void *stream) {
    hipStream_t s = (hipStream_t)stream;
    if (fuse_append) {
        if (waves != 4) return (int)hipErrorInvalidValue;
        if (dtype == FL_BF16) return (int)launch_fused<FL_BF16>(head_dim, whole_rows, n, a, s);
        if (dtype == FL_F16) return (int)launch_fused<FL_F16>(head_dim, whole_rows, n, a, s);
        return (int)hipErrorInvalidValue;
    }
    if (whole_rows) {  // two kv heads of 64 as one row of 128 (refilled early, as at 128)
        if (waves != 4 || head_dim != 128) return (int)hipErrorInvalidValue;
        if (dtype == FL_BF16) return (int)launch_t<FL_BF16, 128, 4, true, true>(n, a, s);
        if (dtype == FL_F16) return (int)launch_t<FL_F16, 128, 4, true, true>(n, a, s);
        return (int)hipErrorInvalidValue;
    }
    switch (dtype * 1000 + head_dim) {
    case FL_BF16 * 1000 + 64: return (int)launch_w<FL_BF16, 64>(waves, early, n, a, s);
    case FL_BF16 * 1000 + 128: return (int)launch_w<FL_BF16, 128>(waves, early, n, a, s);
    case FL_F16 * 1000 + 64: return (int)launch_w<FL_F16, 64>(waves, early, n, a, s);
    case FL_F16 * 1000 + 128: return (int)launch_w<FL_F16, 128>(waves, early, n, a, s);
    case FL_F32 * 1000 + 64: return (int)launch_w<FL_F32, 64>(waves, early, n, a, s);
    case FL_F32 * 1000 + 128: return (int)launch_w<FL_F32, 128>(waves, early, n, a, s);
    default: return (int)hipErrorInvalidValue;
    }
}

}  // namespace fl
