// Host planner: validates one step's page-table metadata and lays the attention work out
// for the gfx950 kernel. Integer arithmetic only; no HIP calls.
//
// Work decomposition.
//   * A row block is up to 16 flattened query rows of one request and one kv head, the
//     flattened row being (query row i) * G + (head within the group). Decode rows give
//     one block of G rows per kv head; a prefill chunk of qo_len rows gives
//     ceil(qo_len * G / 16) blocks. All rows of a block share the block's K/V stream.
//   * A block's keys are [0, kv_end): kv_end = kv_len, or with the causal mask the last
//     key its final row may see plus one (kv_len - qo_len + i_last + 1); they form
//     ceil(kv_end / 16) tiles.
//   * Every block's tiles are laid in one sequence (request, kv head, row block order) and
//     the sequence is cut into contiguous shares of equal estimated time (ring steps plus
//     a charge per segment fold), one per workgroup, one or two workgroups per compute
//     unit. Long histories thereby spread over many compute units and short ones pack
//     together ("A library kernel for decode", What changed: one history's slices run on
//     many processor groups; What I expected: the longest histories set the step's cost).
//     A block cut by a share boundary becomes several pieces whose partial results are
//     merged by log-sum-exp; only the first and last piece of a share can be partial.
//   * Within a share's segment, tile j runs on wave j % NW as that wave's step j / NW, and
//     each segment's per-wave step count but the share's last is padded to a multiple of
//     the ring depth, so segment boundaries fall on the same step in every wave and on a
//     ring group's first step. For each wave and step the
//     plan records the pool row of the tile's first key, (page * P + slot) * Hkv + kv_head,
//     so the kernel addresses K and V without reading the page table.
//   * The plan depends on the lengths only; page ids enter only the recorded pool rows.
#include <algorithm>
#include <cstdio>
#include <numeric>

#include "fl_internal.h"

namespace fl {

namespace {

struct Block {
    int32_t req, kvh, row_begin, nrows, kv_end;
    int32_t tile_cost;  // kStreamTileCost, or kSharedTileCost when the request has several
                        // blocks per kv head; tilted by the head's odd-half share
};

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

fl_status fail(std::string *err, fl_status st, const char *fmt, long long a = 0,
               long long b = 0, long long c = 0, long long d = 0) {
    char buf[256];
    std::snprintf(buf, sizeof buf, fmt, a, b, c, d);
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
    {  // a fresh plan that keeps the previous one's vector storage (a plan per step)
        Plan fresh;
        std::vector<int32_t> *keep[] = {&out.segs, &out.wg_rec, &out.step_rows, &out.append_rows,
                                        &out.append_pos};
        std::vector<int32_t> *into[] = {&fresh.segs, &fresh.wg_rec, &fresh.step_rows, &fresh.append_rows,
                                        &fresh.append_pos};
        for (int i = 0; i < 5; ++i) {
            keep[i]->clear();
            into[i]->swap(*keep[i]);
        }
        out = std::move(fresh);
    }
    const int32_t B = in.batch;
    const int32_t P = lim.page_size;
    const int32_t Hkv_real = lim.num_kv_heads;
    if (B < 0) return fail(err, FL_ERR_INVALID_ARG, "batch %lld < 0", B);
    if (B > lim.max_batch)
        return fail(err, FL_ERR_CAPACITY, "batch %lld exceeds max_batch %lld", B, lim.max_batch);
    if (in.num_splits < 0)
        return fail(err, FL_ERR_INVALID_ARG, "num_splits %lld < 0", in.num_splits);
    out.forced = in.num_splits > 0;
    if (B == 0) {
        // nothing to do; the plan still has the launch shape of a decode step
        out.append_ok = true;  // nothing to append
        out.decode_only = true;
        out.whole_rows = lim.whole_rows_ok && lim.whole_rows_always;
        out.groups_per_cu = lim.groups_per_cu > 0 ? lim.groups_per_cu : 1;
        return FL_OK;
    }
    if (!in.kv_indptr || !in.last_page_len)
        return fail(err, FL_ERR_INVALID_ARG, "kv_indptr and last_page_len must not be NULL");
    if (in.kv_indptr[0] != 0)
        return fail(err, FL_ERR_INVALID_ARG, "kv_indptr[0] = %lld, expected 0", in.kv_indptr[0]);
    if (in.qo_indptr && in.qo_indptr[0] != 0)
        return fail(err, FL_ERR_INVALID_ARG, "qo_indptr[0] = %lld, expected 0", in.qo_indptr[0]);
    if (in.num_pages <= 0 || in.num_pages > INT32_MAX)
        return fail(err, FL_ERR_INVALID_ARG, "num_pages %lld outside [1, 2^31)", in.num_pages);
    if (in.num_pages * P * Hkv_real > INT32_MAX)
        return fail(err, FL_ERR_UNSUPPORTED,
                    "pool of %lld pages x %lld slots x %lld kv heads exceeds 2^31 rows", in.num_pages,
                    P, Hkv_real);

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

    // ---- append slots: query row i of request r stands for token kv_len - qo_len + i -----
    // (the position the bottom-right causal mask gives it); its K/V row goes to that
    // token's page slot. Recorded as the token row page * P + slot (below 2^31 / Hkv).
    out.append_rows.assign((size_t)rows, 0);
    out.append_pos.assign((size_t)rows, 0);
    out.append_ok = true;
    for (int32_t r = 0; r < B && out.append_ok; ++r) {
        const int32_t np = in.kv_indptr[r + 1] - in.kv_indptr[r];
        const int32_t kv_len = (np - 1) * P + in.last_page_len[r];
        const int32_t q0 = in.qo_indptr ? in.qo_indptr[r] : r;
        const int32_t ql = in.qo_indptr ? in.qo_indptr[r + 1] - q0 : 1;
        if (ql > kv_len) {
            char buf[160];
            std::snprintf(buf, sizeof buf, "request %d has %d query rows but %d cached tokens: "
                          "no slot to append them to", r, ql, kv_len);
            out.append_ok = false;
            out.append_err = buf;
            break;
        }
        const int32_t *pages = in.kv_indices + in.kv_indptr[r];
        for (int32_t i = 0; i < ql; ++i) {
            const int32_t t = kv_len - ql + i;
            out.append_rows[q0 + i] = pages[t / P] * P + t % P;
            out.append_pos[q0 + i] = t;
        }
    }
    if (out.append_ok && rows > 1) {
        // two rows appending to one slot (a new token placed in a page shared by two
        // requests) would race; such a plan still serves attention
        std::vector<int32_t> sorted(out.append_rows);
        std::sort(sorted.begin(), sorted.end());
        const auto dup = std::adjacent_find(sorted.begin(), sorted.end());
        if (dup != sorted.end()) {
            char buf[160];
            std::snprintf(buf, sizeof buf, "two query rows append to page %d slot %d (a page "
                          "shared by two requests)", *dup / P, *dup % P);
            out.append_ok = false;
            out.append_err = buf;
        }
    }

    // ---- block shape ------------------------------------------------------------------
    // Decode-only steps may give each request one block of all its query heads over whole
    // token rows: a virtual single kv head of Hkv * D values whose operand rows are zero
    // outside the row's own kv head. The tiles then read every kv head's slice of a token
    // row together (whole 4 KB pages at page size 16) at the same MFMA count.
    // Measured (saturated-style decode, 300 tokens, 14/2 heads, d 64, bf16): whole rows take
    // 10.98 vs 11.19 us at 256 requests and 18.97 vs 20.00 at 512, but at 128 requests they
    // leave half the compute units idle (8.59 vs 7.17 us, one request per workgroup) or cut
    // every request in two (10.41 us), so by default they need a request per compute unit.
    bool decode_only = true;
    int64_t decode_rows = 0;
    for (int32_t r = 0; r < B && decode_only; ++r) {
        const int32_t ql = in.qo_indptr ? in.qo_indptr[r + 1] - in.qo_indptr[r] : 1;
        decode_only = ql <= 1;
        decode_rows += ql;
    }
    out.decode_only = decode_only;
    out.whole_rows = lim.whole_rows_ok && decode_only &&
                     (lim.whole_rows_always || decode_rows >= lim.num_cus);
    const int32_t Hkv = out.whole_rows ? 1 : Hkv_real;
    const int32_t G = out.whole_rows ? lim.num_qo_heads : lim.num_qo_heads / Hkv_real;
    // Workgroups per compute unit: a step with prefill rows is bound by the per-tile
    // arithmetic, which two workgroups per unit overlap better, where their LDS fits
    // (head_dim 64, 16-bit: measured 23 vs 33 us on the ragged mixed step); decode-only
    // steps are bound by memory latency and do best with one (saturated decode 7.1 vs
    // 10.5 us, the extra split's merge dominates). The choice depends only on the step's
    // kind, so every step of one kind launches the same grid.
    const bool prefill = !decode_only;
    const int gpc = lim.groups_per_cu > 0 ? lim.groups_per_cu
                                          : (prefill && lim.head_dim <= 64 && lim.dtype != FL_F32 ? 2 : 1);
    out.groups_per_cu = gpc;

    // ---- row blocks -------------------------------------------------------------------
    // per kv head: the share of its row slice in odd 256-byte halves, in percent; 50 (no
    // tilt) unless token rows span whole 512-byte units
    const int64_t elem = lim.dtype == FL_F32 ? 4 : 2;
    const int64_t slice = (int64_t)lim.head_dim * elem, row_bytes = slice * Hkv;
    std::vector<int64_t> odd_pct(Hkv, 50);
    if (row_bytes % 512 == 0 && !out.whole_rows)
        for (int32_t h = 0; h < Hkv; ++h) {
            int64_t odd = 0;
            for (int64_t x = h * slice; x < (h + 1) * slice; x += 16) odd += (x / 256) & 1;
            odd_pct[h] = 100 * odd / (slice / 16);
        }
    // Prefill units: in a 16-bit type, a request with more than one row block per kv head (a
    // prefill chunk) runs in units of up to kQuadBlocks consecutive blocks (one per wave)
    // over 64-key steps whose K/V the waves share through LDS. Every block of a unit spans
    // the unit's keys (the keys of its last row); the kernel masks each row at its own
    // causal limit.
    const bool quads_ok = lim.dtype != FL_F32 && !out.whole_rows;
    std::vector<Block> blocks;
    struct Quad {
        int64_t block0;
        int32_t nblocks, kv_end;
    };
    std::vector<Quad> quads;
    for (int32_t r = 0; r < B; ++r) {
        const int32_t np = in.kv_indptr[r + 1] - in.kv_indptr[r];
        const int32_t kv_len = (np - 1) * P + in.last_page_len[r];
        const int32_t ql = in.qo_indptr ? in.qo_indptr[r + 1] - in.qo_indptr[r] : 1;
        const int32_t nflat = ql * G;
        const int32_t base_cost = nflat > kBlockRows ? kSharedTileCost : kStreamTileCost;
        const bool quad = quads_ok && nflat > kBlockRows;
        for (int32_t h = 0; h < Hkv; ++h) {
            const int64_t first = (int64_t)blocks.size();
            for (int32_t f0 = 0; f0 < nflat; f0 += kBlockRows) {
                const int32_t tile_cost =
                    (int32_t)(base_cost * (10000 + kOddHalfPercent * (odd_pct[h] - 50)) / 10000);
                const int32_t nr = std::min(kBlockRows, nflat - f0);
                const int32_t i_last = (f0 + nr - 1) / G;
                const int32_t kv_end = in.causal ? kv_len - ql + i_last + 1 : kv_len;
                blocks.push_back({r, h, f0, nr, kv_end, tile_cost});
            }
            if (!quad) continue;
            for (int64_t b0 = first; b0 < (int64_t)blocks.size(); b0 += kQuadBlocks) {
                const int32_t n = (int32_t)std::min<int64_t>(kQuadBlocks, (int64_t)blocks.size() - b0);
                const int32_t kv_end = blocks[b0 + n - 1].kv_end;
                for (int32_t w = 0; w < n; ++w) blocks[b0 + w].kv_end = kv_end;
                quads.push_back({b0, n, kv_end});
            }
        }
    }
    const int64_t nblocks = (int64_t)blocks.size();
    std::vector<char> in_quad(nblocks, 0);
    for (const Quad &qd : quads)
        for (int32_t w = 0; w < qd.nblocks; ++w) in_quad[qd.block0 + w] = 1;
    std::vector<int64_t> dblocks;  // blocks of the decode path
    std::vector<int64_t> tiles(nblocks, 0);
    int64_t T = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        if (in_quad[b]) continue;
        dblocks.push_back(b);
        tiles[b] = ceil_div(blocks[b].kv_end, kTileTokens);
        T += tiles[b];
    }
    const int64_t nquads = (int64_t)quads.size();
    out.units = nquads > 0;
    std::vector<int64_t> qsteps(nquads);
    int64_t QS = 0;
    for (int64_t q = 0; q < nquads; ++q) {
        qsteps[q] = ceil_div(quads[q].kv_end, kQuadStepTokens);
        QS += qsteps[q];
    }

    // ---- pieces: (block or quad, tile or step range), grouped by workgroup --------------
    // Workgroups 0 .. Gp-1 run the quads' pieces (the prefill path), the rest the decode
    // blocks' pieces.
    struct Piece {
        bool quad;
        int64_t idx, lo, hi, group;
    };
    std::vector<Piece> pieces;
    int64_t Gp = 0, G_wg = 0;
    if (in.num_splits > 0) {
        // every block or quad in num_splits balanced pieces (fewer for short ones), one
        // workgroup each
        auto cut = [&](bool is_quad, int64_t idx, int64_t n) {
            int64_t s = std::max<int64_t>(1, std::min<int64_t>(in.num_splits, n));
            const int64_t per = ceil_div(n, s);
            s = ceil_div(n, per);
            for (int64_t j = 0; j < s; ++j)
                pieces.push_back({is_quad, idx, j * per, std::min<int64_t>((j + 1) * per, n), G_wg++});
        };
        for (int64_t q = 0; q < nquads; ++q) cut(true, q, qsteps[q]);
        Gp = G_wg;
        for (int64_t b : dblocks) cut(false, b, tiles[b]);
    } else {
        // Contiguous shares of each sequence (quad steps; decode tiles) with equal estimated
        // time. A decode piece of n tiles costs the ring steps it occupies in all waves (n
        // rounded up to whole step groups, at its block's tile cost) plus a fixed charge for
        // its fold; a block cut inside a share is cut at a multiple of a step group, so only
        // a block's last piece carries padding (a share's last piece is emitted with whole
        // steps only, which the estimate does not count on). A quad piece of n steps costs n steps plus
        // its finish. The smallest per-share budget that needs at most the given number of
        // shares is found by bisection. The grid's workgroups are divided between the two
        // paths in proportion to their estimated totals.
        const int64_t kFoldCost = prefill ? kFoldCostMixed : out.whole_rows ? kFoldCostWhole : kFoldCostDecode;
        const int64_t kCutCost = prefill ? kCutCostMixed : out.whole_rows ? kCutCostWhole : kCutCostDecode;
        const int64_t want = (int64_t)lim.num_cus * gpc;
        constexpr int64_t U = (int64_t)kMaxWaves * kRingDepth;  // tiles of one ring group
        auto dcost = [&](int64_t b, int64_t n, bool cut) {
            return blocks[b].tile_cost * U * ceil_div(n, U) + kFoldCost + (cut ? kCutCost : 0);
        };
        auto qcost = [&](int64_t, int64_t n, bool cut) {
            return kQuadStepCost * n + kQuadSegCost + (cut ? kQuadCutCost : 0);
        };
        int64_t Cd = 0, Cp = 0;
        for (int64_t b : dblocks) Cd += dcost(b, tiles[b], false);
        for (int64_t q = 0; q < nquads; ++q) Cp += qcost(q, qsteps[q], false);
        int64_t Gp_max = 0, Gd_max = 0;
        if (nquads == 0) {
            Gd_max = want;
        } else if (dblocks.empty()) {
            Gp_max = want;
        } else {
            Gp_max = std::min<int64_t>(want - 1, std::max<int64_t>(1, (want * Cp + (Cp + Cd) / 2) / (Cp + Cd)));
            Gd_max = want - Gp_max;
        }
        Gp_max = std::min(Gp_max, QS);
        Gd_max = std::min(std::max<int64_t>(dblocks.empty() ? 0 : 1, std::min(Gd_max, ceil_div(T, lim.min_group_tiles))), T);
        // walk the units filling shares of budget C; emit pieces (group = first_group +
        // share) when `emit` is set. cost(u, n, cut); unit sizes n_of(u); step granularity;
        // whole[i]: cost of the whole of units[i] (the common case, computed once).
        std::vector<int64_t> whole;
        auto fill = [&](const std::vector<int64_t> &units, auto n_of, auto cost, int64_t gran, bool is_quad,
                        int64_t C, int64_t first_group, bool emit) {
            int64_t shares = 0, i = 0, pos = 0;
            const int64_t nu = (int64_t)units.size();
            while (i < nu) {
                int64_t budget = C;
                while (i < nu) {
                    const int64_t u = units[i];
                    const int64_t r = n_of(u) - pos;
                    const int64_t c = pos == 0 ? whole[i] : cost(u, r, true);
                    if (c <= budget) {
                        if (emit) pieces.push_back({is_quad, u, pos, n_of(u), first_group + shares});
                        budget -= c;
                        ++i;
                        pos = 0;
                        continue;
                    }
                    // the largest whole number of step groups that fits the remaining budget
                    const int64_t step_cost = cost(u, gran, true) - cost(u, 0, true);
                    const int64_t fixed = cost(u, 0, true);
                    const int64_t n = budget >= fixed + step_cost ? gran * ((budget - fixed) / step_cost) : 0;
                    if (n > 0) {
                        if (emit) pieces.push_back({is_quad, u, pos, pos + n, first_group + shares});
                        pos += n;
                    }
                    break;
                }
                ++shares;
            }
            return shares;
        };
        auto balance = [&](const std::vector<int64_t> &units, auto n_of, auto cost, int64_t gran, bool is_quad,
                           int64_t G_max, int64_t least, int64_t first_group) {
            if (units.empty() || G_max <= 0) return (int64_t)0;
            int64_t total = 0;
            whole.resize(units.size());
            for (size_t i = 0; i < units.size(); ++i) total += whole[i] = cost(units[i], n_of(units[i]), false);
            // The share count only falls as the budget grows. The smallest budget that fits
            // lies within a few fixed charges of the even split: bracket it by doubling a step
            // from there (a budget of `total` always fits), then bisect.
            int64_t lo = std::max<int64_t>(least, ceil_div(total, G_max)), hi = std::max(total, least);
            for (int64_t d = least; lo + d < hi; d *= 2) {
                if (fill(units, n_of, cost, gran, is_quad, lo + d, first_group, false) <= G_max) {
                    hi = lo + d;
                    break;
                }
                lo = lo + d + 1;  // lo + d does not fit, nor does anything below it
            }
            while (lo < hi) {  // every budget >= least makes progress
                const int64_t mid = lo + (hi - lo) / 2;
                if (fill(units, n_of, cost, gran, is_quad, mid, first_group, false) <= G_max)
                    hi = mid;
                else
                    lo = mid + 1;
            }
            return fill(units, n_of, cost, gran, is_quad, lo, first_group, true);
        };
        std::vector<int64_t> qunits(nquads);
        std::iota(qunits.begin(), qunits.end(), 0);
        auto q_n = [&](int64_t q) { return qsteps[q]; };
        auto d_n = [&](int64_t b) { return tiles[b]; };
        Gp = balance(qunits, q_n, qcost, 1, true, Gp_max, qcost(0, 1, true), 0);
        int64_t max_tile_cost = 0;
        for (int64_t b : dblocks) max_tile_cost = std::max<int64_t>(max_tile_cost, blocks[b].tile_cost);
        G_wg = Gp + balance(dblocks, d_n, dcost, U, false, Gd_max, kFoldCost + kCutCost + max_tile_cost * U, Gp);
    }
    int64_t nslots = 0;  // segment slots: one per decode piece, kQuadBlocks per quad piece
    for (const Piece &pc : pieces) nslots += pc.quad ? kQuadBlocks : 1;
    if (nslots > lim.seg_cap || G_wg > lim.group_cap)
        return fail(err, FL_ERR_CAPACITY, "%lld work items (the handle holds %lld) and %lld "
                    "workgroups (it launches at most %lld): lower num_splits", nslots, lim.seg_cap,
                    G_wg, lim.group_cap);

    // pieces per block, partial rows and merge tickets (a quad's blocks are cut alike)
    std::vector<int32_t> npieces(nblocks, 0), piece_idx(pieces.size());
    for (size_t k = 0; k < pieces.size(); ++k) {
        const Piece &pc = pieces[k];
        const int64_t b0 = pc.quad ? quads[pc.idx].block0 : pc.idx;
        const int32_t nb = pc.quad ? quads[pc.idx].nblocks : 1;
        piece_idx[k] = npieces[b0];
        for (int32_t w = 0; w < nb; ++w) ++npieces[b0 + w];
    }
    std::vector<int64_t> part_base(nblocks, -1);
    std::vector<int32_t> merge_of(nblocks, -1);
    int64_t part_next = 0;
    int32_t merges = 0;
    for (int64_t b = 0; b < nblocks; ++b) {
        out.max_splits = std::max(out.max_splits, npieces[b]);
        if (npieces[b] > 1) {
            part_base[b] = part_next;
            part_next += (int64_t)npieces[b] * blocks[b].nrows;
            merge_of[b] = merges++;
        }
    }
    if (part_next > lim.part_rows_cap)
        return fail(err, FL_ERR_CAPACITY, "%lld partial rows exceed the workspace (%lld rows)",
                    part_next, lim.part_rows_cap);

    // ---- emit segments, workgroup tables and step rows ----------------------------------
    // Decode pieces: one segment each; within it tile j goes to wave j % NW as that wave's
    // step j / NW; every segment's per-wave step count but a share's last is rounded up to a
    // multiple of the ring depth, the same in all waves (every share has at least one
    // ring group of steps). Padding steps repeat a real tile of the segment (never scored).
    // Quad pieces: kQuadBlocks segment slots each (slots past the quad's blocks hold
    // num_rows 0), and per 64-key step the pool rows of its four 16-key tiles.
    constexpr int NW = kMaxWaves;
    int64_t total = 0;
    std::vector<int64_t> seg_steps(pieces.size());
    for (size_t k = 0; k < pieces.size(); ++k) {
        const int64_t n = pieces[k].hi - pieces[k].lo;
        if (pieces[k].quad) {
            seg_steps[k] = n;
            total += n * kQuadStepTiles;
        } else {
            // a share's last segment needs no padding to whole ring groups (the kernel's
            // last group may be short), only every share at least one group in all
            const bool last = k + 1 == pieces.size() || pieces[k + 1].group != pieces[k].group;
            const bool first = k == 0 || pieces[k - 1].group != pieces[k].group;
            seg_steps[k] = last ? std::max<int64_t>(ceil_div(n, NW), first ? kRingDepth : 1)
                                : ceil_div(ceil_div(n, NW), kRingDepth) * kRingDepth;
            total += seg_steps[k] * NW;
        }
    }
    if (total > lim.max_tiles)
        return fail(err, FL_ERR_CAPACITY, "%lld tile steps exceed max_tiles %lld", total,
                    lim.max_tiles);
    out.segs.assign((size_t)nslots * FL_WORK_ITEM_INTS, 0);
    out.wg_rec.assign(G_wg * kRecInts, 0);
    out.step_rows.assign((size_t)total, 0);
    // Workgroups b and b + kXcds run on one XCD (the XCDs take a launch's workgroups in turn:
    // XCD (b + c) % kXcds, c fixed within a launch), and each XCD has its own L2. Shares next
    // to each other in a sequence hold neighbouring row
    // blocks, which for a prefill chunk read the same K/V, so share s of a path with n shares
    // (starting at workgroup `first`) goes to the workgroup that puts runs of consecutive
    // shares on one XCD: the first ceil(n / kXcds) shares on one XCD, the next on the next.
    const auto workgroup_of = [&](int64_t share, int64_t n, int64_t first) -> int64_t {
        if (!kXcdAwareLayout) return first + share;
        int64_t lo = 0;
        for (int64_t x = 0; x < kXcds; ++x) {
            const int64_t n_x = (n - x + kXcds - 1) / kXcds;  // shares on this XCD
            if (share < lo + n_x) return first + (share - lo) * kXcds + x;
            lo += n_x;
        }
        return first + share;  // not reached
    };
    auto fill_item = [&](int32_t *it, const Block &bl, int64_t t0, int64_t t1, int64_t b, int32_t pidx,
                         int64_t wg, int64_t pos) {
        const int32_t np = in.kv_indptr[bl.req + 1] - in.kv_indptr[bl.req];
        it[FL_WI_Q_START] = in.qo_indptr ? in.qo_indptr[bl.req] : bl.req;
        it[FL_WI_QO_LEN] = in.qo_indptr ? in.qo_indptr[bl.req + 1] - in.qo_indptr[bl.req] : 1;
        it[FL_WI_KV_LEN] = (np - 1) * P + in.last_page_len[bl.req];
        it[FL_WI_PAGE_BASE] = in.kv_indptr[bl.req];
        it[FL_WI_KV_HEAD] = bl.kvh;
        it[FL_WI_ROW_BEGIN] = bl.row_begin;
        it[FL_WI_NUM_ROWS] = bl.nrows;
        it[FL_WI_TOK_BEGIN] = (int32_t)t0;
        it[FL_WI_TOK_END] = (int32_t)t1;
        it[FL_WI_PART_ROW] = npieces[b] > 1 ? (int32_t)(part_base[b] + (int64_t)pidx * bl.nrows) : -1;
        it[FL_WI_REQUEST] = bl.req;
        it[FL_WI_SPLIT] = pidx;
        it[FL_WI_NUM_SPLITS] = npieces[b];
        it[FL_WI_MERGE] = merge_of[b];
        it[FL_WI_GROUP] = (int32_t)wg;
        it[FL_WI_POS_BEGIN] = (int32_t)pos;
    };
    const int lp = __builtin_ctz((unsigned)P);  // the page size is a power of two
    auto pool_row = [&](const Block &bl, int64_t t) {
        const int32_t *pages = in.kv_indices + in.kv_indptr[bl.req];
        return (int32_t)((((int64_t)pages[t >> lp] << lp) + (t & (P - 1))) * Hkv + bl.kvh);
    };
    size_t k = 0;
    int64_t slot = 0, off = 0;
    int32_t real_segs = 0;
    for (int64_t g = 0; g < G_wg; ++g) {
        const bool pg = g < Gp;
        const int64_t wg = pg ? workgroup_of(g, Gp, 0) : workgroup_of(g - Gp, G_wg - Gp, Gp);
        int32_t *rec = &out.wg_rec[wg * kRecInts];
        size_t k_end = k;
        int64_t steps = 0, slots = 0;
        while (k_end < pieces.size() && pieces[k_end].group == g) {
            steps += seg_steps[k_end];
            slots += pieces[k_end].quad ? kQuadBlocks : 1;
            ++k_end;
        }
        rec[REC_KIND] = pg ? 1 : 0;
        rec[REC_SEG_BEGIN] = (int32_t)slot;
        rec[REC_SEG_END] = (int32_t)(slot + slots);
        rec[REC_POS] = (int32_t)off;
        rec[REC_STEPS] = (int32_t)steps;
        rec[REC_FIRST_END] = (int32_t)seg_steps[k];
        const int64_t slot_first = slot;
        int64_t pos = 0;
        for (; k < k_end; ++k) {
            const Piece &pc = pieces[k];
            if (pc.quad) {
                const Quad &qd = quads[pc.idx];
                const Block &b0 = blocks[qd.block0];
                const int64_t t0 = pc.lo * kQuadStepTokens;
                const int64_t t1 = std::min<int64_t>(pc.hi * kQuadStepTokens, qd.kv_end);
                for (int32_t w = 0; w < kQuadBlocks; ++w, ++slot) {
                    int32_t *it = &out.segs[slot * FL_WORK_ITEM_INTS];
                    if (w < qd.nblocks) {
                        fill_item(it, blocks[qd.block0 + w], t0, t1, qd.block0 + w, piece_idx[k], wg, pos);
                        ++real_segs;
                    } else {  // an empty slot: the same request and keys, no rows
                        fill_item(it, b0, t0, t1, qd.block0, piece_idx[k], wg, pos);
                        it[FL_WI_NUM_ROWS] = 0;
                        it[FL_WI_MERGE] = -1;
                        it[FL_WI_PART_ROW] = -1;
                    }
                }
                // per step, the pool rows of its four 16-key tiles (tiles past the keys
                // repeat the last real one; their keys are never scored)
                const int64_t last_tile = (qd.kv_end - 1) / kTileTokens * kTileTokens;
                for (int64_t s = pc.lo; s < pc.hi; ++s)
                    for (int32_t u = 0; u < kQuadStepTiles; ++u) {
                        const int64_t t = std::min<int64_t>(s * kQuadStepTokens + u * kTileTokens, last_tile);
                        out.step_rows[off + (s - pc.lo) * kQuadStepTiles + u] = pool_row(b0, t);
                    }
                off += (pc.hi - pc.lo) * kQuadStepTiles;
            } else {
                const Block &bl = blocks[pc.idx];
                const int64_t t0 = pc.lo * kTileTokens;
                const int64_t t1 = std::min<int64_t>(pc.hi * kTileTokens, bl.kv_end);
                fill_item(&out.segs[slot * FL_WORK_ITEM_INTS], bl, t0, t1, pc.idx, piece_idx[k], wg, pos);
                ++slot;
                ++real_segs;
                const int64_t nt = pc.hi - pc.lo;
                for (int64_t q = 0; q < seg_steps[k]; ++q)
                    for (int w = 0; w < NW; ++w) {
                        int64_t j = q * NW + w;
                        if (j >= nt) j = (nt - 1 - w >= 0) ? nt - 1 - ((nt - 1 - w) % NW) : 0;
                        out.step_rows[off + w * steps + pos + q] = pool_row(bl, t0 + j * kTileTokens);
                    }
            }
            pos += seg_steps[k];
        }
        if (!pg) {
            std::copy_n(&out.segs[slot_first * FL_WORK_ITEM_INTS], FL_WORK_ITEM_INTS, rec + REC_HEAD);
            for (int w = 0; w < NW; ++w)  // every share has >= kRingDepth steps per wave
                for (int q = 0; q < kRingDepth; ++q)
                    rec[REC_ROWS + w * kRingDepth + q] = out.step_rows[off + w * steps + q];
            off += steps * NW;
        }
    }
    out.num_groups = (int32_t)G_wg;
    out.num_prefill_groups = (int32_t)Gp;
    out.num_segs = real_segs;
    out.num_seg_slots = (int32_t)nslots;
    out.num_merges = merges;
    out.part_rows = part_next;
    return FL_OK;
}

}  // namespace fl
