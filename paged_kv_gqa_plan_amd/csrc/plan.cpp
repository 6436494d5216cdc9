// Host planner: validates one step's page-table metadata and cuts the attention work into
// items for the gfx950 kernels. Integer arithmetic only; no HIP calls.
//
// Work decomposition.
//   * A row block is up to 16 flattened query rows of one request and one kv head, the
//     flattened row being (query row i) * G + (head within the group). Decode rows give
//     one block of G rows per kv head; a prefill chunk of qo_len rows gives
//     ceil(qo_len * G / 16) blocks. All rows of a block share the block's K/V stream.
//   * A block's keys are [0, kv_end): kv_end = kv_len, or with the causal mask the last
//     key its final row may see plus one (kv_len - qo_len + i_last + 1).
//   * Long key ranges are cut into slices that run as separate workgroups, and their
//     partial results are merged by log-sum-exp afterwards ("A library kernel for decode",
//     What changed: slices of one history spread over many processor groups). The slice
//     length is chosen from the total work and the compute-unit count so that the
//     longest histories, which set the step's cost (same write-up, What I expected), are
//     spread over the whole chip, while short histories stay in one slice.
//   * The plan depends on the lengths only, never on page ids.
#include <algorithm>
#include <cstdio>
#include <numeric>

#include "fl_internal.h"

namespace fl {

namespace {

struct Block {
    int32_t req, kvh, row_begin, nrows, kv_end;
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

fl_status fail(std::string *err, fl_status st, const char *fmt, long long a = 0,
               long long b = 0, long long c = 0) {
    char buf[256];
    std::snprintf(buf, sizeof buf, fmt, a, b, c);
    if (err) *err = buf;
    return st;
}

}  // namespace

int64_t row_block_bound(const PlanLimits &lim) {
    const int64_t G = lim.num_qo_heads / lim.num_kv_heads;
    // sum_r ceil(qo_len_r * G / 16) <= rows * G / 16 + batch
    return (int64_t)lim.num_kv_heads *
           (ceil_div((int64_t)lim.max_qo_rows * G, kBlockRows) + lim.max_batch);
}

fl_status build_plan(const PlanLimits &lim, const PlanInput &in, Plan &out, std::string *err) {
    out = Plan();
    const int32_t B = in.batch;
    const int32_t P = lim.page_size;
    const int32_t Hkv = lim.num_kv_heads;
    const int32_t G = lim.num_qo_heads / lim.num_kv_heads;
    if (B < 0) return fail(err, FL_ERR_INVALID_ARG, "batch %lld < 0", B);
    if (B > lim.max_batch)
        return fail(err, FL_ERR_CAPACITY, "batch %lld exceeds max_batch %lld", B, lim.max_batch);
    if (in.num_splits < 0)
        return fail(err, FL_ERR_INVALID_ARG, "num_splits %lld < 0", in.num_splits);
    if (B == 0) return FL_OK;
    if (!in.kv_indptr || !in.last_page_len)
        return fail(err, FL_ERR_INVALID_ARG, "kv_indptr and last_page_len must not be NULL");
    if (in.kv_indptr[0] != 0)
        return fail(err, FL_ERR_INVALID_ARG, "kv_indptr[0] = %lld, expected 0", in.kv_indptr[0]);
    if (in.qo_indptr && in.qo_indptr[0] != 0)
        return fail(err, FL_ERR_INVALID_ARG, "qo_indptr[0] = %lld, expected 0", in.qo_indptr[0]);
    if (in.num_pages <= 0 || in.num_pages > INT32_MAX)
        return fail(err, FL_ERR_INVALID_ARG, "num_pages %lld outside [1, 2^31)", in.num_pages);

    // ---- validate every request -----------------------------------------------------
    for (int32_t r = 0; r < B; ++r) {
        const int64_t np = (int64_t)in.kv_indptr[r + 1] - in.kv_indptr[r];
        if (np < 1)
            return fail(err, FL_ERR_INVALID_ARG,
                        "request %lld holds %lld pages; every request needs >= 1", r, np);
        const int32_t last = in.last_page_len[r];
        if (last < 1 || last > P)
            return fail(err, FL_ERR_INVALID_ARG,
                        "last_page_len[%lld] = %lld outside [1, page_size=%lld]", r, last, P);
        const int64_t kv_len = (np - 1) * P + last;
        if (kv_len > INT32_MAX / 2)
            return fail(err, FL_ERR_INVALID_ARG, "request %lld: kv_len %lld too large", r, kv_len);
        const int64_t ql = in.qo_indptr ? (int64_t)in.qo_indptr[r + 1] - in.qo_indptr[r] : 1;
        if (ql < 0)
            return fail(err, FL_ERR_INVALID_ARG, "qo_indptr decreases at request %lld", r);
        if (in.causal && ql > kv_len)
            return fail(err, FL_ERR_INVALID_ARG,
                        "request %lld: %lld query rows on %lld cached tokens with causal mask",
                        r, ql, kv_len);
    }
    const int64_t nnz = in.kv_indptr[B];
    const int64_t rows = in.qo_indptr ? in.qo_indptr[B] : B;
    if (nnz > lim.max_kv_pages)
        return fail(err, FL_ERR_CAPACITY, "%lld page-table entries exceed max_kv_pages %lld", nnz,
                    lim.max_kv_pages);
    if (rows > lim.max_qo_rows)
        return fail(err, FL_ERR_CAPACITY, "%lld query rows exceed max_qo_rows %lld", rows,
                    lim.max_qo_rows);
    if (nnz > 0 && !in.kv_indices)
        return fail(err, FL_ERR_INVALID_ARG, "kv_indices must not be NULL");
    for (int64_t j = 0; j < nnz; ++j) {
        const int32_t pg = in.kv_indices[j];
        if (pg < 0 || pg >= in.num_pages)
            return fail(err, FL_ERR_INVALID_ARG, "kv_indices[%lld] = %lld outside [0, %lld)", j,
                        pg, in.num_pages);
    }
    out.nnz = nnz;

    // ---- row blocks -------------------------------------------------------------------
    std::vector<Block> blocks;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t np = in.kv_indptr[r + 1] - in.kv_indptr[r];
        const int32_t kv_len = (np - 1) * P + in.last_page_len[r];
        const int32_t ql = in.qo_indptr ? in.qo_indptr[r + 1] - in.qo_indptr[r] : 1;
        const int32_t nflat = ql * G;
        for (int32_t h = 0; h < Hkv; ++h)
            for (int32_t f0 = 0; f0 < nflat; f0 += kBlockRows) {
                const int32_t nr = std::min(kBlockRows, nflat - f0);
                const int32_t i_last = (f0 + nr - 1) / G;
                const int32_t kv_end = in.causal ? kv_len - ql + i_last + 1 : kv_len;
                blocks.push_back({r, h, f0, nr, kv_end});
            }
    }
    const int64_t nblocks = (int64_t)blocks.size();
    std::vector<int64_t> tiles(nblocks);
    int64_t total_tiles = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        tiles[b] = ceil_div(blocks[b].kv_end, kTileTokens);
        total_tiles += tiles[b];
    }

    // ---- slices per block ----------------------------------------------------------------
    // tiles per slice for block b given a slice budget; balanced so no slice is empty.
    std::vector<int64_t> nsplit(nblocks), per(nblocks);
    auto assign = [&](int64_t chunk_tiles, int64_t fixed) {
        int64_t items = 0, prows = 0;
        for (int64_t b = 0; b < nblocks; ++b) {
            int64_t s = fixed > 0 ? std::min<int64_t>(fixed, tiles[b]) : ceil_div(tiles[b], chunk_tiles);
            s = std::max<int64_t>(1, s);
            const int64_t p = ceil_div(tiles[b], s);
            s = ceil_div(tiles[b], p);
            nsplit[b] = s;
            per[b] = p;
            items += s;
            if (s > 1) prows += s * blocks[b].nrows;
        }
        return std::make_pair(items, prows);
    };
    std::pair<int64_t, int64_t> use;
    if (in.num_splits > 0) {
        use = assign(0, in.num_splits);
        if (use.first > lim.item_cap || use.second > lim.part_rows_cap)
            return fail(err, FL_ERR_CAPACITY,
                        "num_splits %lld needs %lld work items (cap %lld); lower it or raise "
                        "split_items_per_cu", in.num_splits, use.first, lim.item_cap);
    } else {
        const int64_t target = (int64_t)lim.num_cus * lim.split_items_per_cu;
        const int64_t min_tiles = std::max<int64_t>(1, lim.min_split_tokens / kTileTokens);
        int64_t chunk = std::max(min_tiles, ceil_div(total_tiles, std::max<int64_t>(1, target)));
        use = assign(chunk, 0);
        while (use.first > lim.item_cap || use.second > lim.part_rows_cap) {
            chunk *= 2;
            use = assign(chunk, 0);
        }
    }
    if (use.first > INT32_MAX)
        return fail(err, FL_ERR_CAPACITY, "too many work items (%lld)", use.first);

    // ---- emit items: longest slices first, so the tail of the launch holds short work --
    struct Pending {
        int64_t block, split, tok_begin, tok_end, part_row;
    };
    std::vector<Pending> pend;
    pend.reserve((size_t)use.first);
    int64_t part_next = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        const Block &bl = blocks[b];
        const int64_t s = nsplit[b];
        const int64_t base = s > 1 ? part_next : -1;
        if (s > 1) {
            out.merges.insert(out.merges.end(), kMergeInts, 0);
            int32_t *m = &out.merges[out.merges.size() - kMergeInts];
            m[MI_Q_START] = in.qo_indptr ? in.qo_indptr[bl.req] : bl.req;
            m[MI_KV_HEAD] = bl.kvh;
            m[MI_ROW_BEGIN] = bl.row_begin;
            m[MI_NUM_ROWS] = bl.nrows;
            m[MI_PART_ROW] = (int32_t)base;
            m[MI_NUM_SPLITS] = (int32_t)s;
            part_next += s * bl.nrows;
        }
        for (int64_t j = 0; j < s; ++j) {
            const int64_t t0 = j * per[b] * kTileTokens;
            const int64_t t1 = std::min<int64_t>((j + 1) * per[b] * kTileTokens, bl.kv_end);
            pend.push_back({b, j, t0, t1, s > 1 ? base + j * bl.nrows : -1});
        }
        out.max_splits = std::max<int32_t>(out.max_splits, (int32_t)s);
    }
    std::stable_sort(pend.begin(), pend.end(), [](const Pending &a, const Pending &b) {
        return (a.tok_end - a.tok_begin) > (b.tok_end - b.tok_begin);
    });
    out.items.assign(pend.size() * FL_WORK_ITEM_INTS, 0);
    for (size_t k = 0; k < pend.size(); ++k) {
        const Pending &p = pend[k];
        const Block &bl = blocks[p.block];
        int32_t *it = &out.items[k * FL_WORK_ITEM_INTS];
        const int32_t np = in.kv_indptr[bl.req + 1] - in.kv_indptr[bl.req];
        it[FL_WI_Q_START] = in.qo_indptr ? in.qo_indptr[bl.req] : bl.req;
        it[FL_WI_QO_LEN] = in.qo_indptr ? in.qo_indptr[bl.req + 1] - in.qo_indptr[bl.req] : 1;
        it[FL_WI_KV_LEN] = (np - 1) * P + in.last_page_len[bl.req];
        it[FL_WI_PAGE_BASE] = in.kv_indptr[bl.req];
        it[FL_WI_KV_HEAD] = bl.kvh;
        it[FL_WI_ROW_BEGIN] = bl.row_begin;
        it[FL_WI_NUM_ROWS] = bl.nrows;
        it[FL_WI_TOK_BEGIN] = (int32_t)p.tok_begin;
        it[FL_WI_TOK_END] = (int32_t)p.tok_end;
        it[FL_WI_PART_ROW] = (int32_t)p.part_row;
        it[FL_WI_REQUEST] = bl.req;
        it[FL_WI_SPLIT] = (int32_t)p.split;
        it[FL_WI_NUM_SPLITS] = (int32_t)nsplit[p.block];
    }
    out.num_items = (int32_t)pend.size();
    out.num_merges = (int32_t)(out.merges.size() / kMergeInts);
    out.part_rows = part_next;
    return FL_OK;
}

}  // namespace fl
