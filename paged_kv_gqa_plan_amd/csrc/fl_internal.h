// Internal types shared by the planner (plan.cpp), the C-ABI layer (api.cpp) and the
// gfx950 kernels (attn_kernels.hip). Not part of the public interface.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "fl_paged_attn.h"

namespace fl {

// The thread's last error message (fl_last_error): set it and return st; clear it.
fl_status set_error(fl_status st, const std::string &msg);
void clear_error();

// Keys per MFMA tile: the 16-row M dimension of the 16x16xK matrix instructions.
constexpr int kTileTokens = 16;
// Flattened query rows (query row * G + head in group) per row block: the 16-column N
// dimension of the same instructions.
constexpr int kBlockRows = 16;
// Tiles of K and V each wave keeps in flight. Every segment's per-wave step count but a
// share's last is a multiple of it, so segment boundaries fall on the same loop step in
// every wave, the first of a ring group; every share has at least that many steps.
#ifndef FL_RING_DEPTH
#define FL_RING_DEPTH 2
#endif
constexpr int kRingDepth = FL_RING_DEPTH;
// Planner's time estimate, in hundredths of a streamed tile. A tile whose keys only its
// own row block reads is streamed from memory (100); the tiles of a request with several
// row blocks per kv head (a prefill chunk) are shared through the L2 cache (80: measured
// 0.098 vs 0.121 us per tile on a ragged mixed step). Where every token row of the pool
// spans whole 512-byte units, a kv head whose slice of the row lies in the odd 256-byte
// half of a unit streams slower than one in the even half (long-context skew at head_dim
// 128: 49.5 vs 43.4 us per workgroup for equal tiles; shifting the pools by 256 bytes
// swaps which head is slow), so its tiles cost kOddHalfPercent more (chosen by A/B:
// long-context skew 56.5 -> 55.4 us, mixed-length decode 13.6 -> 13.5 us). Each segment adds a fold (the cross-wave
// merge of the softmax states at its end, with the padding of its last step group), and a
// piece of a block cut by a share boundary adds its end-of-kernel merge ticket (and the
// merge itself when it finishes last). Measured best: decode-only steps 6 and 4 tiles
// (mixed-length decode 13.6 vs 14.5 us with 6 and 0), steps with a prefill chunk, whose
// short decode blocks pack many segments into a share, 12 and 0 (ragged step 19.1 vs 19.7).
constexpr int kStreamTileCost = 100;
constexpr int kSharedTileCost = 80;
constexpr int kOddHalfPercent = 20;
#ifndef FL_FOLD_TILES_DECODE
#define FL_FOLD_TILES_DECODE 6
#endif
#ifndef FL_CUT_TILES_DECODE
#define FL_CUT_TILES_DECODE 4
#endif
#ifndef FL_FOLD_TILES_MIXED
#define FL_FOLD_TILES_MIXED 12
#endif
#ifndef FL_CUT_TILES_MIXED
#define FL_CUT_TILES_MIXED 0
#endif
// Whole-row tiles move twice the bytes of a per-kv-head tile, so the same fold and cut
// costs are half as many of them.
#ifndef FL_FOLD_TILES_WHOLE
#define FL_FOLD_TILES_WHOLE 3
#endif
#ifndef FL_CUT_TILES_WHOLE
#define FL_CUT_TILES_WHOLE 2
#endif
constexpr int kFoldCostWhole = kStreamTileCost * FL_FOLD_TILES_WHOLE;
constexpr int kCutCostWhole = kStreamTileCost * FL_CUT_TILES_WHOLE;
constexpr int kFoldCostDecode = kStreamTileCost * FL_FOLD_TILES_DECODE;
constexpr int kCutCostDecode = kStreamTileCost * FL_CUT_TILES_DECODE;
constexpr int kFoldCostMixed = kStreamTileCost * FL_FOLD_TILES_MIXED;
constexpr int kCutCostMixed = kStreamTileCost * FL_CUT_TILES_MIXED;
// Prefill units: up to kQuadBlocks consecutive row blocks of one request and kv head (one
// per wave: 64 flattened rows) over 64-key steps of four 16-key tiles (one loaded by each
// wave). Two blocks per wave (128 rows) measured slower on the ragged mixed step (29.6 vs
// 16.8 us for the chunk alone): half the units to spread, as many merges, and the two
// blocks' arithmetic did not overlap. Planner's estimate of a unit step and of a unit
// piece's fixed costs, in the same hundredths of a streamed decode tile as above.
#ifndef FL_QUAD_BLOCKS
#define FL_QUAD_BLOCKS 4
#endif
constexpr int kQuadBlocks = FL_QUAD_BLOCKS;
constexpr int kQuadStepTiles = 4;
constexpr int kQuadStepTokens = kQuadStepTiles * 16;
#ifndef FL_QUAD_STEP_COST
#define FL_QUAD_STEP_COST 450
#endif
#ifndef FL_QUAD_SEG_COST
#define FL_QUAD_SEG_COST 400
#endif
// A unit cut by a share boundary costs its pieces a round trip each for the partial rows
// and the ticket, and one more for the merge. Step 450 and cut 1100, chosen by a sweep of
// both (four runs on two boxes): ragged mixed step 17.3-17.6 us and four-chunk step
// 16.4-16.6 us, against 17.6-19.0 and 16.7-16.9 at 500 and 1500; cuts of 200-600 or
// 2500-4000 measured 19.4-22 us.
#ifndef FL_QUAD_CUT_COST
#define FL_QUAD_CUT_COST 1100
#endif
constexpr int64_t kQuadStepCost = FL_QUAD_STEP_COST;
constexpr int64_t kQuadSegCost = FL_QUAD_SEG_COST;
constexpr int64_t kQuadCutCost = FL_QUAD_CUT_COST;
// XCDs of the GPU (MI355X: 8 of 32 compute units), which take a launch's workgroups in
// turn; the plan places runs of neighbouring shares on one XCD (one L2).
constexpr int kXcds = 8;
#ifndef FL_XCD_AWARE
#define FL_XCD_AWARE 1
#endif
constexpr bool kXcdAwareLayout = FL_XCD_AWARE != 0;
// Per-workgroup record (int32): the first segment's header, the segment range, the step
// range, the first segment's end step and the pool rows of every wave's first kRingDepth
// steps, so every load a workgroup issues first (Q, K/V, step rows) depends on this record
// alone. With two ring slots it is one 128-byte line, read by one batch of scalar loads.
constexpr int kMaxWaves = 4;
// A prefill workgroup's record (REC_KIND 1) uses the segment range (kQuadBlocks slots per
// quad piece), REC_POS (its first step row: kQuadBlocks per 64-key step) and REC_STEPS
// (its 64-key steps).
enum {
    REC_HEAD = 0,    // FL_WORK_ITEM_INTS entries
    REC_SEG_BEGIN = 16, REC_SEG_END = 17, REC_POS = 18, REC_STEPS = 19, REC_FIRST_END = 20,
    REC_KIND = 21,   // 0: decode blocks, 1: prefill quads
    REC_ROWS = 24,   // kMaxWaves * kRingDepth entries
};
constexpr int kRecInts = (REC_ROWS + kMaxWaves * kRingDepth + 31) / 32 * 32;
// Plan header (int32): one 128-byte line in front of the workgroup records, written by
// every plan. It carries everything about the step that a launch needs besides the
// buffers, so one launch (grid, kernel, arguments) serves every plan of its launch class
// and a captured HIP graph replays correctly after any later plan of that class.
// Workgroups at or past HDR_NUM_GROUPS exit at once; a launch whose class stamp differs
// from the plan's (a graph captured on a plan of another class) touches nothing, and its
// first workgroup counts the refusal in the handle's status word.
enum {
    HDR_NUM_GROUPS = 0,  // workgroups with work (the rest of the grid is idle)
    HDR_CLASS = 1,       // launch class of run() (attention alone)
    HDR_FCLASS = 2,      // launch class of the one-launch run_append (0: none)
    HDR_CAUSAL = 3,
    HDR_SCALE_LOG2 = 4,  // float bits: sm_scale * log2(e)
    HDR_HKV = 5,         // kv heads as the kernel sees them (1 for whole-row blocks)
    HDR_GROUP = 6,       // query heads per (virtual) kv head
    HDR_GROUP_MAGIC = 7, // ceil(2^32 / group), 0 when group == 1
    HDR_REAL_GROUP = 8,  // query heads per real kv head
    HDR_APPEND_ROWS = 9, // query rows the append kernels write; -1: the plan has no valid
                         // append slots (the kernels refuse and count it)
    HDR_USED = 10,
    kHdrInts = 32,
};

struct PlanLimits {
    int32_t num_qo_heads, num_kv_heads, head_dim, page_size;
    int32_t dtype;
    int32_t max_batch, max_qo_rows;
    int64_t max_kv_pages;
    int32_t num_cus;
    int32_t groups_per_cu;        // > 0, or 0: per step (see build_plan)
    int32_t waves;                // wavefronts per workgroup
    int32_t min_group_tiles;      // resolved (> 0)
    int64_t max_tiles;            // per-wave steps (x waves) one plan may hold
    int64_t seg_cap;              // segments one plan may hold
    int64_t group_cap;            // workgroups one plan may launch
    int64_t part_rows_cap;        // fp32 partial rows one plan may use
    bool whole_rows_ok;           // decode-only steps may use whole-row blocks (Hkv * D = 128,
                                  // Hq <= 16, 16-bit type, not switched off)
    bool whole_rows_always;       // ... on every decode-only step, not only those with at
                                  // least one query row per compute unit
};

struct PlanInput {
    int32_t batch;
    const int32_t *qo_indptr;     // may be NULL
    const int32_t *kv_indptr;
    const int32_t *kv_indices;
    const int32_t *last_page_len;
    int64_t num_pages;
    int32_t causal;
    int32_t num_splits;           // 0 = spread evenly over the compute units
};

struct Plan {
    std::vector<int32_t> segs;      // FL_WORK_ITEM_INTS per segment, grouped by workgroup
    std::vector<int32_t> wg_rec;    // kRecInts per workgroup (the plan header in front of
                                    // them is written by the C-ABI layer)
    std::vector<int32_t> step_rows; // per workgroup, per wave, per step: pool row
                                    // (page * P + slot) * Hkv + kv_head of the step's tile's
                                    // first key (padding steps repeat a real tile's row)
    int32_t num_groups = 0;
    int32_t num_prefill_groups = 0; // workgroups 0 .. this - 1 run prefill quads
    int32_t groups_per_cu = 1;      // workgroups per compute unit the shares were cut for
    int32_t num_segs = 0;           // work items (empty quad slots not counted)
    int32_t num_seg_slots = 0;      // segment slots in segs
    int32_t num_merges = 0;
    bool whole_rows = false;        // blocks hold every query head of a request and read whole
                                    // token rows (one virtual kv head of Hkv * D values)
    bool decode_only = false;       // every request has at most one query row
    bool units = false;             // the plan holds prefill units (16-bit, > 16 flattened rows)
    bool forced = false;            // num_splits > 0: one workgroup per piece, grid = num_groups
    int32_t max_splits = 0;
    int64_t part_rows = 0;
    std::vector<int32_t> append_rows;  // per query row: token row page * P + slot of the
                                       // token it stands for (the KV append's destination)
    std::vector<int32_t> append_pos;   // per query row: that token's position in its request
    bool append_ok = false;            // every row has a slot, no two rows share one
    std::string append_err;            // why not, when !append_ok
};

// Validate the step's metadata and build the work list. Host only, integer only.
// Returns FL_OK or an error status with a message in *err.
fl_status build_plan(const PlanLimits &lim, const PlanInput &in, Plan &out, std::string *err);

// Upper bound on the row blocks of one plan, used to size the handle's buffers.
int64_t row_block_bound(const PlanLimits &lim);

// ---------------------------------------------------------------------------------------
// kernel launch interface (attn_kernels.hip)
// ---------------------------------------------------------------------------------------
struct AttnArgs {
    const int32_t *segs;       // FL_WORK_ITEM_INTS per segment
    const int32_t *wg_rec;     // plan header (kHdrInts), then kRecInts per workgroup
    const int32_t *step_rows;  // per workgroup, wave and step
    int32_t *tickets;          // one per merged row block, zero between runs
    int32_t *status;           // refused launches are counted here
    const void *q;
    const void *k;
    const void *v;
    void *out;
    float *lse;                // may be NULL
    float *part_o;             // [part_rows, head_dim]
    float *part_lse;           // [part_rows], log2 domain
    int32_t num_qo_heads;
    int32_t launch_class;      // must equal the plan header's class (HDR_CLASS, or
                               // HDR_FCLASS for the fused append) or the launch is refused
    // Per-plan values: the host leaves them zero; the kernel fills them from the plan header
    // (so a captured launch sees the plan current at replay time).
    int32_t num_kv_heads;
    int32_t group;
    uint32_t group_magic;      // ceil(2^32 / group) (unused when group == 1)
    int32_t causal;
    float scale_log2;          // sm_scale * log2(e)
    int32_t real_group;        // whole-row blocks: query heads per real kv head (the kv head
                               // of block row h is h / real_group); otherwise unused
    // fused KV append (decode-only steps): the step's new K/V rows [rows, Hkv, D], and per
    // query row the token row (page * P + slot) they go to; NULL when not fused
    const void *k_new;
    const void *v_new;
    const int32_t *append_rows;
};

// Return hipSuccess or the launch error (as int to keep HIP headers out of this file).
// early_refill: refill a K/V slot as soon as its tile is in registers (memory-bound steps)
// rather than after the tile's arithmetic (steps bound by the arithmetic).
// whole_rows: head_dim is the virtual row width Hkv * D (128) of whole-row blocks.
// fuse_append: the launch also appends the new K/V rows (a.k_new, a.v_new; decode-only
// plans, 16-bit types): it writes them to the pools and uses them for the newest key.
// grid: workgroups of the launch (the launch class's fixed grid).
int launch_attention(int dtype, int head_dim, int waves, bool early_refill, bool whole_rows,
                     bool fuse_append, int grid, const AttnArgs &a, void *stream);

// KV append: copy row r of k_new / v_new (row_bytes each, a multiple of 16) to token row
// dst_rows[r] of k_pool / v_pool (kv_append.hip), for r below the plan header's
// HDR_APPEND_ROWS. The grid is sized for max_rows rows, so one launch serves every plan.
struct AppendArgs {
    const int32_t *hdr;        // plan header
    int32_t *status;           // refused launches are counted here
    const int32_t *dst_rows;
    const void *k_new;
    const void *v_new;
    void *k_pool;
    void *v_pool;
    int32_t max_rows;
    int32_t row_bytes;
};
int launch_kv_append(const AppendArgs &a, void *stream);

// KV append fused with the rotary position embedding (kv_rope.hip): row r's K heads are
// rotated by position pos[r] and written to token row dst_rows[r] of k_pool, its V heads
// copied to v_pool, and (when q is not NULL) its query heads rotated in place. inv_freq[i]
// (i < head_dim / 2) are the pair frequencies, already rounded to fp32 on the host.
constexpr int kMaxRopePairs = 64;  // head_dim <= 128
struct RopeArgs {
    const int32_t *hdr;        // plan header: HDR_APPEND_ROWS rows (-1: refused)
    int32_t *status;
    const int32_t *dst_rows;
    const int32_t *pos;
    const void *k_new;
    const void *v_new;
    void *k_pool;
    void *v_pool;
    void *q;
    int32_t max_rows, num_kv_heads, num_qo_heads, head_dim, dtype;
    float inv_freq[kMaxRopePairs];
};
int launch_kv_append_rope(const RopeArgs &a, void *stream);

// Poison: fill whole pages of one or two pools with a 16-byte pattern (kv_poison.hip).
constexpr int kPoisonIdsPerLaunch = 256;
struct PoisonArgs {
    const int32_t *page_ids;   // host
    int32_t n;
    void *k_pool;
    void *v_pool;              // may be NULL
    int64_t page_bytes;        // a multiple of 16
    uint32_t pattern[4];
};
int launch_kv_poison(const PoisonArgs &a, void *stream);

// What the allocation-free run (noalloc.hip) needs from a planned handle: the host copy of
// the plan's device metadata, its partial-row needs and its launch (api.cpp).
struct NoallocView {
    int device;                    // the handle's device, -1 for a host-only handle
    const int32_t *hdr;            // kHdrInts
    const int32_t *recs;           // kRecInts per busy workgroup
    int64_t rec_bytes;
    const int32_t *segs;
    int64_t seg_bytes;
    const int32_t *steps;
    int64_t step_bytes;
    int32_t num_merges;            // merge tickets the plan uses (must start at zero)
    int64_t part_rows;             // fp32 partial rows of part_width floats (+ one lse each)
    int32_t part_width;
    int32_t dtype, head_dim, waves, grid, launch_class, num_qo_heads;
    bool early, whole_rows;
};
fl_status noalloc_view(fl_handle h, NoallocView *v);

// Copy byte ranges [off, off + bytes) from pinned host memory to the same offsets of a
// device buffer with one kernel (offsets 16-byte aligned, sizes multiples of 4).
constexpr int kStageParts = 5;
struct StageCopy {
    const char *src;   // pinned host memory, device-accessible
    char *dst;         // device memory
    int64_t off[kStageParts], bytes[kStageParts];
};
int launch_stage_copy(const StageCopy &c, void *stream);

}  // namespace fl
