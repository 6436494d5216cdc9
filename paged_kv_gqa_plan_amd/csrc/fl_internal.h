// Internal types shared by the planner (plan.cpp), the C-ABI layer (api.cpp) and the
// gfx950 kernels (attn_kernels.hip). Not part of the public interface.
#pragma once

#include <stdint.h>

#include <string>
#include <vector>

#include "fl_paged_attn.h"

namespace fl {

// Keys per MFMA tile: the 16-row M dimension of the 16x16xK matrix instructions.
constexpr int kTileTokens = 16;
// Flattened query rows (query row * G + head in group) per row block: the 16-column N
// dimension of the same instructions.
constexpr int kBlockRows = 16;
// int32 fields per merge item.
constexpr int kMergeInts = 8;
enum { MI_Q_START = 0, MI_KV_HEAD, MI_ROW_BEGIN, MI_NUM_ROWS, MI_PART_ROW, MI_NUM_SPLITS };

struct PlanLimits {
    int32_t num_qo_heads, num_kv_heads, head_dim, page_size;
    int32_t max_batch, max_qo_rows;
    int64_t max_kv_pages;
    int32_t num_cus;
    int32_t split_items_per_cu;   // resolved (> 0)
    int32_t min_split_tokens;     // resolved (> 0, multiple of 16)
    int64_t item_cap;             // work items one plan may emit
    int64_t part_rows_cap;        // fp32 partial rows one plan may use
};

struct PlanInput {
    int32_t batch;
    const int32_t *qo_indptr;     // may be NULL
    const int32_t *kv_indptr;
    const int32_t *kv_indices;
    const int32_t *last_page_len;
    int64_t num_pages;
    int32_t causal;
    int32_t num_splits;           // 0 = automatic
};

struct Plan {
    std::vector<int32_t> items;   // FL_WORK_ITEM_INTS per item, launch order
    std::vector<int32_t> merges;  // kMergeInts per merged row block
    int32_t num_items = 0;
    int32_t num_merges = 0;
    int32_t max_splits = 0;
    int64_t part_rows = 0;
    int64_t nnz = 0;
};

// Validate the step's metadata and build the work list. Host only, integer only.
// Returns FL_OK or an error status with a message in *err.
fl_status build_plan(const PlanLimits &lim, const PlanInput &in, Plan &out, std::string *err);

// Upper bounds used to size the handle's buffers.
int64_t row_block_bound(const PlanLimits &lim);

// ---------------------------------------------------------------------------------------
// kernel launch interface (attn_kernels.hip)
// ---------------------------------------------------------------------------------------
struct AttnArgs {
    const int32_t *items;
    const int32_t *kv_indices;
    const void *q;
    const void *k;
    const void *v;
    void *out;
    float *lse;          // may be NULL
    float *part_o;       // [part_rows, head_dim]
    float *part_lse;     // [part_rows], log2 domain
    int32_t num_qo_heads;
    int32_t num_kv_heads;
    int32_t group;
    int32_t log2_page;
    int32_t causal;
    float scale_log2;    // sm_scale * log2(e)
};

struct MergeArgs {
    const int32_t *merges;
    const float *part_o;
    const float *part_lse;
    void *out;
    float *lse;          // may be NULL
    int32_t num_qo_heads;
    int32_t group;
};

// Return hipSuccess or the launch error (as int to keep HIP headers out of this file).
int launch_attention(int dtype, int head_dim, int num_items, const AttnArgs &a, void *stream);
int launch_merge(int dtype, int head_dim, int num_merges, const MergeArgs &a, void *stream);

}  // namespace fl
