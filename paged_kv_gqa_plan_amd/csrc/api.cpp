// C interface of the paged GQA attention library: handles, plan staging and launches.
//
// A handle owns persistent device buffers for the per-step metadata (plan header, work
// list, merge tickets, per-wave pool rows, append slots) that plan() refreshes in place and
// the kernels read (flashlet README, design bullets: metadata in persistent device
// buffers, updated in place each step; pinned-to-device metadata path). A launch depends
// only on the handle and the plan's launch class (the kernel variant and a grid fixed per
// variant); the plan header tells the kernels how many workgroups have work and every
// per-step scalar, so one captured launch serves every later plan of its class.
// The host side stages each plan into one of two pinned buffers and copies it with one
// asynchronous transfer on the caller's stream; an event per staging buffer keeps a new
// plan from overwriting a buffer whose copy is still in flight.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <new>
#include <string>

#include "fl_internal.h"

using fl::Plan;
using fl::PlanLimits;

namespace {

thread_local std::string g_last_error;

fl_status set_err(fl_status st, const std::string &msg) { return fl::set_error(st, msg); }

fl_status hip_err(hipError_t e, const char *what) {
    return set_err(FL_ERR_HIP, std::string(what) + ": " + hipGetErrorName(e) + " (" +
                                   hipGetErrorString(e) + ")");
}

int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

}  // namespace

struct fl_paged_attn {
    fl_config cfg{};
    PlanLimits lim{};
    int device = -1;
    bool host_only = true;
    int32_t group = 1;
    int32_t log2_page = 0;

    // device buffers
    char *d_meta = nullptr;      // [segments | plan header + workgroup records | merge tickets |
                                 //  step rows | append slots | status word]
    float *d_part_o = nullptr;   // [part_rows_cap, head_dim]
    float *d_part_lse = nullptr; // [part_rows_cap]
    int64_t off_wg_rec = 0, off_tickets = 0, off_steps = 0, off_append = 0, off_pos = 0,
            off_status = 0, meta_bytes = 0;
    int32_t waves = 4;
    int32_t part_width = 64;     // floats per partial row: head_dim, or 128 for whole rows

    // pinned staging, double-buffered
    char *h_stage[2] = {nullptr, nullptr};
    char *d_stage[2] = {nullptr, nullptr};   // the same buffers as the device addresses them
    hipEvent_t ev[2] = {nullptr, nullptr};
    bool ev_live[2] = {false, false};
    int cur = 0;

    // current plan
    bool planned = false;
    Plan plan;
    int32_t hdr_host[fl::kHdrInts] = {};  // its plan header (as staged to the device)
    int32_t causal = 1;
    float scale_log2 = 0.f;
};

fl_status fl::set_error(fl_status st, const std::string &msg) {
    g_last_error = msg;
    return st;
}

void fl::clear_error() { g_last_error.clear(); }

namespace {

fl_status check_config(const fl_config *c) {
    if (!c) return set_err(FL_ERR_INVALID_ARG, "config is NULL");
    if (c->num_kv_heads < 1 || c->num_qo_heads < 1 || c->num_qo_heads % c->num_kv_heads)
        return set_err(FL_ERR_INVALID_ARG,
                       "num_qo_heads must be a positive multiple of num_kv_heads >= 1");
    if (c->head_dim != 64 && c->head_dim != 128)
        return set_err(FL_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
    const int p = c->page_size;
    if (p < 16 || p > 256 || (p & (p - 1)))
        return set_err(FL_ERR_UNSUPPORTED, "page_size must be a power of two in [16, 256]");
    if (c->dtype != FL_F16 && c->dtype != FL_BF16 && c->dtype != FL_F32)
        return set_err(FL_ERR_UNSUPPORTED, "dtype must be FL_F16, FL_BF16 or FL_F32");
    if (c->max_batch < 0 || c->max_qo_rows < 0 || c->max_kv_pages < 0)
        return set_err(FL_ERR_INVALID_ARG, "capacities must be >= 0");
    if (c->num_cus < 0 || c->groups_per_cu < 0 || c->min_group_tokens < 0 || c->max_tiles < 0)
        return set_err(FL_ERR_INVALID_ARG, "num_cus, groups_per_cu, min_group_tokens and "
                                           "max_tiles must be >= 0");
    if (c->waves_per_group != 0 && c->waves_per_group != 4)
        return set_err(FL_ERR_UNSUPPORTED, "waves_per_group must be 0 or 4");
    if (c->whole_rows < -1 || c->whole_rows > 1)
        return set_err(FL_ERR_INVALID_ARG, "whole_rows must be -1, 0 or 1");
    if (c->whole_rows == 1) {
        // asked for on every decode step: refuse a shape that can never take them
        const char *why = c->dtype == FL_F32 ? "fp32 (whole-row blocks are 16-bit only)"
                          : c->num_kv_heads < 2 ? "one kv head (its tiles already read whole rows)"
                          : c->num_kv_heads * c->head_dim != 128 ? "num_kv_heads * head_dim != 128"
                          : c->num_qo_heads > fl::kBlockRows ? "more than 16 query heads"
                          : ((uint64_t)c->max_qo_rows * c->num_qo_heads + 16) * c->num_qo_heads >=
                                    (1ull << 32)
                              ? "(max_qo_rows * num_qo_heads + 16) * num_qo_heads >= 2^32"
                              : nullptr;
        if (why) return set_err(FL_ERR_UNSUPPORTED, std::string("whole_rows = 1 on a shape that "
                                                               "cannot take whole-row blocks: ") + why);
    }
    // the kernels divide flattened rows of a request (below max_qo_rows * G + 16) by G
    // with a 32-bit reciprocal multiply, exact while the dividend stays below 2^32 / G
    const uint64_t g = (uint64_t)(c->num_qo_heads / c->num_kv_heads);
    if (((uint64_t)c->max_qo_rows * g + 16) * g >= (1ull << 32))
        return set_err(FL_ERR_UNSUPPORTED, "(max_qo_rows * G + 16) * G must be below 2^32 "
                                           "(G = num_qo_heads / num_kv_heads)");
    return FL_OK;
}

void release(fl_paged_attn *h) {
    if (!h) return;
    if (!h->host_only) {
        (void)hipSetDevice(h->device);
        for (int i = 0; i < 2; ++i) {
            if (h->ev[i]) {
                (void)hipEventSynchronize(h->ev[i]);
                (void)hipEventDestroy(h->ev[i]);
            }
            if (h->h_stage[i]) (void)hipHostFree(h->h_stage[i]);
        }
        (void)hipDeviceSynchronize();
        if (h->d_meta) (void)hipFree(h->d_meta);
        if (h->d_part_o) (void)hipFree(h->d_part_o);
        if (h->d_part_lse) (void)hipFree(h->d_part_lse);
    }
    delete h;
}

// Kernel arguments of the current plan (whole-row blocks: one virtual kv head of Hkv * D
// values shared by every query head).
fl::AttnArgs attn_args(const fl_paged_attn *h, const void *q, const void *k_pool, const void *v_pool,
                       void *out, float *lse) {
    fl::AttnArgs a{};
    a.segs = (const int32_t *)h->d_meta;
    a.wg_rec = (const int32_t *)(h->d_meta + h->off_wg_rec);
    a.step_rows = (const int32_t *)(h->d_meta + h->off_steps);
    a.tickets = (int32_t *)(h->d_meta + h->off_tickets);
    a.status = (int32_t *)(h->d_meta + h->off_status);
    a.q = q;
    a.k = k_pool;
    a.v = v_pool;
    a.out = out;
    a.lse = lse;
    a.part_o = h->d_part_o;
    a.part_lse = h->d_part_lse;
    a.num_qo_heads = h->cfg.num_qo_heads;
    return a;
}

// The launch a plan needs: kernel variant and grid. Every auto plan of one kind (decode
// only, or with prefill rows; whole-row blocks or not) gets the same grid, num_cus x the
// workgroups per compute unit of its kind; forced-split plans launch one workgroup per
// piece. The class stamp names the variant and the grid, so two plans of one class launch
// identically.
struct LaunchDesc {
    int grid = 0;
    int cls = 0;        // run(): attention alone
    int fcls = 0;       // run_append in one launch; 0 when the plan cannot take it
    int head_dim = 0;   // kernel's row width (Hkv * D for whole-row blocks)
    bool early = false; // refill a ring slot before the tile's arithmetic
    bool wr = false;
};
LaunchDesc launch_desc(const fl_paged_attn *h, const Plan &p) {
    LaunchDesc d;
    d.wr = p.whole_rows;
    d.head_dim = p.whole_rows ? h->cfg.num_kv_heads * h->cfg.head_dim : h->cfg.head_dim;
    // fp32 keeps a register ring (refilled after the arithmetic); at head_dim 128 the
    // arithmetic hides the LDS reads, so the refill always goes first; at 64 it goes first
    // on the memory-bound steps (one workgroup per compute unit)
    d.early = h->cfg.dtype != FL_F32 && (d.head_dim >= 128 || p.groups_per_cu == 1);
    d.grid = p.forced ? std::max<int32_t>(1, p.num_groups) : h->lim.num_cus * p.groups_per_cu;
    d.cls = (d.grid << 3) | (d.early << 2) | (d.wr << 1) | 1;
    // the one-launch append: decode-only plans in a 16-bit type whose rows run no prefill
    // unit (its kernel has no unit path), i.e. at most 16 query heads per kv head (above
    // that a decode row spans two 16-row blocks, which run as a unit)
    if (p.decode_only && h->cfg.dtype != FL_F32 && p.append_ok && h->group <= fl::kBlockRows && !p.units)
        d.fcls = (1 << 30) | (d.grid << 3) | (1 << 2) | (d.wr << 1) | 1;
    return d;
}

// The plan header for the current plan (kHdrInts int32).
void fill_header(const fl_paged_attn *h, const LaunchDesc &d, int32_t *hdr) {
    const Plan &p = h->plan;
    std::memset(hdr, 0, fl::kHdrInts * 4);
    const int32_t group = p.whole_rows ? h->cfg.num_qo_heads : h->group;
    hdr[fl::HDR_NUM_GROUPS] = p.num_groups;
    hdr[fl::HDR_CLASS] = d.cls;
    hdr[fl::HDR_FCLASS] = d.fcls;
    hdr[fl::HDR_CAUSAL] = h->causal;
    std::memcpy(&hdr[fl::HDR_SCALE_LOG2], &h->scale_log2, 4);
    hdr[fl::HDR_HKV] = p.whole_rows ? 1 : h->cfg.num_kv_heads;
    hdr[fl::HDR_GROUP] = group;
    hdr[fl::HDR_GROUP_MAGIC] = group > 1 ? (int32_t)(uint32_t)(((1ull << 32) + group - 1) / group) : 0;
    hdr[fl::HDR_REAL_GROUP] = h->group;
    hdr[fl::HDR_APPEND_ROWS] = p.append_ok ? (int32_t)p.append_rows.size() : -1;
}

}  // namespace

fl_status fl::noalloc_view(fl_handle h, NoallocView *v) {
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "run before a successful plan()");
    const Plan &p = h->plan;
    const LaunchDesc d = launch_desc(h, p);
    v->device = h->host_only ? -1 : h->device;
    v->hdr = h->hdr_host;
    v->recs = p.wg_rec.data();
    v->rec_bytes = (int64_t)p.wg_rec.size() * 4;
    v->segs = p.segs.data();
    v->seg_bytes = (int64_t)p.segs.size() * 4;
    v->steps = p.step_rows.data();
    v->step_bytes = (int64_t)p.step_rows.size() * 4;
    v->num_merges = p.num_merges;
    v->part_rows = p.part_rows;
    v->part_width = d.head_dim;  // the kernel's row width for this plan
    v->dtype = h->cfg.dtype;
    v->head_dim = d.head_dim;
    v->waves = h->waves;
    v->grid = d.grid;
    v->launch_class = d.cls;
    v->num_qo_heads = h->cfg.num_qo_heads;
    v->early = d.early;
    v->whole_rows = d.wr;
    return FL_OK;
}

extern "C" {

const char *fl_last_error(void) { return g_last_error.c_str(); }

fl_status fl_paged_attn_create(const fl_config *cfg, int device, fl_handle *out) {
    g_last_error.clear();
    if (!out) return set_err(FL_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    fl_status st = check_config(cfg);
    if (st != FL_OK) return st;
    if (device < -1) return set_err(FL_ERR_INVALID_ARG, "device must be >= -1");

    fl_paged_attn *h = new (std::nothrow) fl_paged_attn();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "out of host memory");
    h->cfg = *cfg;
    h->device = device;
    h->host_only = device < 0;
    h->group = cfg->num_qo_heads / cfg->num_kv_heads;
    h->waves = cfg->waves_per_group ? cfg->waves_per_group : 4;
    while ((1 << h->log2_page) < cfg->page_size) ++h->log2_page;

    int num_cus = cfg->num_cus;
    if (!h->host_only) {
        hipError_t e = hipSetDevice(device);
        if (e != hipSuccess) {
            release(h);
            return hip_err(e, "hipSetDevice");
        }
        if (num_cus == 0) {
            int n = 0;
            e = hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, device);
            if (e != hipSuccess) {
                release(h);
                return hip_err(e, "hipDeviceGetAttribute(CU count)");
            }
            num_cus = n;
        }
    }
    if (num_cus == 0) num_cus = 256;

    PlanLimits &L = h->lim;
    L.num_qo_heads = cfg->num_qo_heads;
    L.num_kv_heads = cfg->num_kv_heads;
    L.head_dim = cfg->head_dim;
    L.page_size = cfg->page_size;
    L.dtype = cfg->dtype;
    L.max_batch = cfg->max_batch;
    L.max_qo_rows = cfg->max_qo_rows;
    L.max_kv_pages = cfg->max_kv_pages;
    L.num_cus = num_cus;
    L.groups_per_cu = cfg->groups_per_cu;  // 0: the plan picks per step
    L.waves = h->waves;
    L.min_group_tiles =
        cfg->min_group_tokens > 0 ? (int32_t)((cfg->min_group_tokens + 15) / 16) : 8;
    L.whole_rows_always = cfg->whole_rows == 1;
    L.whole_rows_ok = cfg->whole_rows >= 0 && cfg->dtype != FL_F32 &&
                      cfg->num_kv_heads * cfg->head_dim == 128 && cfg->num_kv_heads > 1 &&
                      cfg->num_qo_heads <= fl::kBlockRows &&
                      ((uint64_t)cfg->max_qo_rows * cfg->num_qo_heads + 16) * cfg->num_qo_heads <
                          (1ull << 32);  // the kernels' division of flattened rows by Hq
    h->part_width = L.whole_rows_ok ? 128 : cfg->head_dim;
    const int64_t blocks = fl::row_block_bound(L);
    L.group_cap = std::max<int64_t>((int64_t)num_cus * std::max(L.groups_per_cu, 2), 16384);
    if (L.group_cap >= (1 << 26)) {  // the launch class stamp holds the grid in 26 bits
        release(h);
        return set_err(FL_ERR_UNSUPPORTED, "num_cus x groups_per_cu too large");
    }
    L.seg_cap = blocks + fl::kQuadBlocks * L.group_cap;  // quad pieces take kQuadBlocks slots
    // steps: every row block may read at most all of the plan's pages; each work item adds
    // at most one ring group of padding per wave
    const int64_t tiles_bound = blocks * ((L.max_kv_pages * L.page_size + 15) / 16 + 1) +
                                L.seg_cap * fl::kRingDepth * h->waves;
    L.max_tiles = cfg->max_tiles > 0 ? cfg->max_tiles : std::min<int64_t>(tiles_bound, 1LL << 24);
    // partial rows are addressed with 32-bit byte offsets: keep the workspace under 2 GiB
    L.part_rows_cap = std::min<int64_t>(L.seg_cap * fl::kBlockRows,
                                        (INT32_MAX / 4) / (h->part_width + 1));
    if (L.seg_cap > INT32_MAX / FL_WORK_ITEM_INTS || L.max_tiles > INT32_MAX) {
        release(h);
        return set_err(FL_ERR_CAPACITY, "capacities too large");
    }

    h->off_wg_rec = align_up(L.seg_cap * FL_WORK_ITEM_INTS * 4, 256);
    h->off_tickets = align_up(h->off_wg_rec + (fl::kHdrInts + L.group_cap * fl::kRecInts) * 4, 256);
    h->off_steps = align_up(h->off_tickets + blocks * 4, 256);
    h->off_append = align_up(h->off_steps + std::max<int64_t>(1, L.max_tiles) * 4, 256);
    // append regions: the rows' token slots, then their positions (max_qo_rows ints each)
    h->off_pos = align_up(h->off_append + std::max<int64_t>(1, cfg->max_qo_rows) * 4, 256);
    h->off_status = align_up(h->off_pos + std::max<int64_t>(1, cfg->max_qo_rows) * 4, 256);
    h->meta_bytes = h->off_status + 256;

    if (!h->host_only) {
        hipError_t e;
        if ((e = hipMalloc((void **)&h->d_meta, h->meta_bytes)) != hipSuccess ||
            (e = hipMalloc((void **)&h->d_part_o, L.part_rows_cap * h->part_width * 4)) !=
                hipSuccess ||
            (e = hipMalloc((void **)&h->d_part_lse, L.part_rows_cap * 4)) != hipSuccess) {
            release(h);
            return hip_err(e, "hipMalloc (handle buffers)");
        }
        // merge tickets start at zero once; runs keep them there. The status word counts
        // refused launches.
        if ((e = hipMemset(h->d_meta + h->off_tickets, 0, (size_t)(h->off_steps - h->off_tickets))) !=
                hipSuccess ||
            (e = hipMemset(h->d_meta + h->off_status, 0, 256)) != hipSuccess ||
            (e = hipStreamSynchronize(nullptr)) != hipSuccess) {
            release(h);
            return hip_err(e, "hipMemset (merge tickets)");
        }
        for (int i = 0; i < 2; ++i) {
            if ((e = hipHostMalloc((void **)&h->h_stage[i], h->meta_bytes, hipHostMallocDefault)) !=
                    hipSuccess ||
                (e = hipHostGetDevicePointer((void **)&h->d_stage[i], h->h_stage[i], 0)) !=
                    hipSuccess ||
                (e = hipEventCreateWithFlags(&h->ev[i], hipEventDisableTiming)) != hipSuccess) {
                release(h);
                return hip_err(e, "pinned staging / event");
            }
        }
    }
    *out = h;
    return FL_OK;
}

fl_status fl_paged_attn_destroy(fl_handle h) {
    g_last_error.clear();
    release(h);
    return FL_OK;
}

fl_status fl_paged_attn_plan(fl_handle h, int32_t batch, const int32_t *qo_indptr,
                             const int32_t *kv_indptr, const int32_t *kv_indices,
                             const int32_t *last_page_len, int64_t num_pages, int32_t causal,
                             float sm_scale, int32_t num_splits, void *stream) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    h->planned = false;
    if (!(sm_scale == sm_scale) || std::isinf(sm_scale))
        return set_err(FL_ERR_INVALID_ARG, "sm_scale must be finite");
    fl::PlanInput in{batch, qo_indptr, kv_indptr, kv_indices, last_page_len,
                     num_pages, causal ? 1 : 0, num_splits};
    std::string err;
    fl_status st = fl::build_plan(h->lim, in, h->plan, &err);
    if (st != FL_OK) return set_err(st, err);
    const double scale = sm_scale > 0.f ? (double)sm_scale : 1.0 / std::sqrt((double)h->cfg.head_dim);
    h->scale_log2 = (float)(scale * 1.4426950408889634);
    h->causal = causal ? 1 : 0;
    fill_header(h, launch_desc(h, h->plan), h->hdr_host);

    if (!h->host_only) {
        hipError_t e = hipSetDevice(h->device);
        if (e != hipSuccess) return hip_err(e, "hipSetDevice");
        const int slot = h->cur;
        h->cur ^= 1;
        if (h->ev_live[slot]) {
            // the copy that last used this staging buffer must have finished reading it
            if ((e = hipEventSynchronize(h->ev[slot])) != hipSuccess)
                return hip_err(e, "hipEventSynchronize (staging)");
        }
        char *st_buf = h->h_stage[slot];
        const Plan &p = h->plan;
        // The used part of each region goes over, read by one small kernel straight from
        // the pinned staging buffer. The merge tickets are not copied: they are zeroed at
        // create and every run leaves them at zero (the piece that merges a row block
        // resets its ticket).
        std::memcpy(st_buf, p.segs.data(), p.segs.size() * 4);
        std::memcpy(st_buf + h->off_wg_rec, h->hdr_host, fl::kHdrInts * 4);
        std::memcpy(st_buf + h->off_wg_rec + fl::kHdrInts * 4, p.wg_rec.data(), p.wg_rec.size() * 4);
        std::memcpy(st_buf + h->off_steps, p.step_rows.data(), p.step_rows.size() * 4);
        // append slots and positions
        const int64_t append_bytes = p.append_ok ? (int64_t)p.append_rows.size() * 4 : 0;
        const int64_t off_pos = h->off_pos;
        if (append_bytes) {
            std::memcpy(st_buf + h->off_append, p.append_rows.data(), append_bytes);
            std::memcpy(st_buf + off_pos, p.append_pos.data(), append_bytes);
        }
        fl::StageCopy sc{h->d_stage[slot], h->d_meta,
                         {0, h->off_wg_rec, h->off_steps, h->off_append, off_pos},
                         {(int64_t)p.segs.size() * 4, (int64_t)(fl::kHdrInts + p.wg_rec.size()) * 4,
                          (int64_t)p.step_rows.size() * 4, append_bytes, append_bytes}};
        hipStream_t s = (hipStream_t)stream;
        if ((e = (hipError_t)fl::launch_stage_copy(sc, s)) != hipSuccess)
            return hip_err(e, "plan metadata copy");
        if ((e = hipEventRecord(h->ev[slot], s)) != hipSuccess)
            return hip_err(e, "hipEventRecord (plan)");
        h->ev_live[slot] = true;
    }
    h->planned = true;
    return FL_OK;
}

fl_status fl_paged_attn_run(fl_handle h, const void *q, const void *k_pool, const void *v_pool,
                            void *out, float *lse, void *stream) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (h->host_only) return set_err(FL_ERR_UNSUPPORTED, "run() on a host-only handle");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "run() before a successful plan()");
    const Plan &p = h->plan;
    if (!q || !k_pool || !v_pool || !out)
        return set_err(FL_ERR_INVALID_ARG, "q, k_pool, v_pool and out must not be NULL");
    if (((uintptr_t)q | (uintptr_t)k_pool | (uintptr_t)v_pool | (uintptr_t)out) & 15)
        return set_err(FL_ERR_INVALID_ARG, "q, k_pool, v_pool and out must be 16-byte aligned");

    // an empty plan launches too (every workgroup idle), so that a captured launch exists
    fl::AttnArgs a = attn_args(h, q, k_pool, v_pool, out, lse);
    const LaunchDesc d = launch_desc(h, p);
    a.launch_class = d.cls;
    const int e = fl::launch_attention(h->cfg.dtype, d.head_dim, h->waves, d.early, d.wr, false,
                                       d.grid, a, stream);
    if (e != (int)hipSuccess) return hip_err((hipError_t)e, "attention launch");
    return FL_OK;
}

fl_status fl_paged_attn_run_append(fl_handle h, const void *q, const void *k_new, const void *v_new,
                                   void *k_pool, void *v_pool, void *out, float *lse, void *stream) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (h->host_only) return set_err(FL_ERR_UNSUPPORTED, "run_append on a host-only handle");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "run_append before a successful plan()");
    const Plan &p = h->plan;
    if (!p.append_ok) return set_err(FL_ERR_INVALID_ARG, "the plan has no append slots: " + p.append_err);
    const LaunchDesc d = launch_desc(h, p);
    if (!d.fcls) {
        // a prefill chunk's new keys are read by many workgroups: append first, then attend
        fl_status st = fl_paged_kv_append(h, k_new, v_new, k_pool, v_pool, stream);
        if (st != FL_OK) return st;
        return fl_paged_attn_run(h, q, k_pool, v_pool, out, lse, stream);
    }
    if (!q || !k_new || !v_new || !k_pool || !v_pool || !out)
        return set_err(FL_ERR_INVALID_ARG, "q, k_new, v_new, k_pool, v_pool and out must not be NULL");
    if (((uintptr_t)q | (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool |
         (uintptr_t)out) & 15)
        return set_err(FL_ERR_INVALID_ARG, "q, k_new, v_new, k_pool, v_pool and out must be 16-byte aligned");
    fl::AttnArgs a = attn_args(h, q, k_pool, v_pool, out, lse);
    a.k_new = k_new;
    a.v_new = v_new;
    a.append_rows = (const int32_t *)(h->d_meta + h->off_append);
    a.launch_class = d.fcls;
    const int e = fl::launch_attention(h->cfg.dtype, d.head_dim, h->waves, true, d.wr, true, d.grid, a,
                                       stream);
    if (e != (int)hipSuccess) return hip_err((hipError_t)e, "attention + append launch");
    return FL_OK;
}

fl_status fl_paged_kv_append(fl_handle h, const void *k_new, const void *v_new, void *k_pool,
                             void *v_pool, void *stream) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (h->host_only) return set_err(FL_ERR_UNSUPPORTED, "append on a host-only handle");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "append before a successful plan()");
    const Plan &p = h->plan;
    if (!p.append_ok) return set_err(FL_ERR_INVALID_ARG, "the plan has no append slots: " + p.append_err);
    if (!k_new || !v_new || !k_pool || !v_pool)
        return set_err(FL_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must not be NULL");
    if (((uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) & 15)
        return set_err(FL_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must be 16-byte aligned");
    const int64_t elem = h->cfg.dtype == FL_F32 ? 4 : 2;
    const int64_t row_bytes = (int64_t)h->cfg.num_kv_heads * h->cfg.head_dim * elem;
    const int64_t max_rows = std::max<int64_t>(1, h->cfg.max_qo_rows);
    if (max_rows * (row_bytes / 16) >= INT32_MAX)
        return set_err(FL_ERR_UNSUPPORTED, "max_qo_rows x 16-byte chunks per token row must stay below 2^31");
    // the grid covers max_qo_rows; the kernel reads the plan's row count from its header
    fl::AppendArgs a{(const int32_t *)(h->d_meta + h->off_wg_rec), (int32_t *)(h->d_meta + h->off_status),
                     (const int32_t *)(h->d_meta + h->off_append), k_new, v_new, k_pool, v_pool,
                     (int32_t)max_rows, (int32_t)row_bytes};
    const int le = fl::launch_kv_append(a, stream);
    if (le != (int)hipSuccess) return hip_err((hipError_t)le, "kv append launch");
    return FL_OK;
}

fl_status fl_paged_kv_append_rope(fl_handle h, void *q, const void *k_new, const void *v_new,
                                  void *k_pool, void *v_pool, float rope_theta, void *stream) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!(rope_theta > 0.f) || !std::isfinite(rope_theta))
        return set_err(FL_ERR_INVALID_ARG, "rope_theta must be positive and finite");
    if (h->cfg.head_dim > 2 * fl::kMaxRopePairs || h->cfg.head_dim % 2)
        return set_err(FL_ERR_UNSUPPORTED, "rotary embedding needs an even head_dim <= 128");
    if (h->host_only) return set_err(FL_ERR_UNSUPPORTED, "append on a host-only handle");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "append before a successful plan()");
    const Plan &p = h->plan;
    if (!p.append_ok) return set_err(FL_ERR_INVALID_ARG, "the plan has no append slots: " + p.append_err);
    if (!k_new || !v_new || !k_pool || !v_pool)
        return set_err(FL_ERR_INVALID_ARG, "k_new, v_new, k_pool and v_pool must not be NULL");
    const int64_t elem = h->cfg.dtype == FL_F32 ? 4 : 2;
    if (((uintptr_t)q | (uintptr_t)k_new | (uintptr_t)v_new | (uintptr_t)k_pool | (uintptr_t)v_pool) &
        (uintptr_t)(elem - 1))
        return set_err(FL_ERR_INVALID_ARG, "q, k_new, v_new, k_pool and v_pool must be aligned to the element size");
    fl::RopeArgs a{};
    a.hdr = (const int32_t *)(h->d_meta + h->off_wg_rec);
    a.status = (int32_t *)(h->d_meta + h->off_status);
    a.dst_rows = (const int32_t *)(h->d_meta + h->off_append);
    a.pos = (const int32_t *)(h->d_meta + h->off_pos);
    a.k_new = k_new;
    a.v_new = v_new;
    a.k_pool = k_pool;
    a.v_pool = v_pool;
    a.q = q;
    a.max_rows = std::max<int32_t>(1, h->cfg.max_qo_rows);
    a.num_kv_heads = h->cfg.num_kv_heads;
    a.num_qo_heads = h->cfg.num_qo_heads;
    a.head_dim = h->cfg.head_dim;
    a.dtype = h->cfg.dtype;
    // pair frequencies theta^(-2i/D), formed in double and rounded once to fp32
    for (int i = 0; i < h->cfg.head_dim / 2; ++i)
        a.inv_freq[i] = (float)std::pow((double)rope_theta, -2.0 * i / h->cfg.head_dim);
    const int le = fl::launch_kv_append_rope(a, stream);
    if (le != (int)hipSuccess) return hip_err((hipError_t)le, "kv append + rope launch");
    return FL_OK;
}

fl_status fl_paged_kv_append_slots(fl_handle h, int32_t *slots, int32_t capacity, int32_t *num_rows) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "no plan");
    if (capacity < 0 || (capacity > 0 && !slots))
        return set_err(FL_ERR_INVALID_ARG, "slots is NULL or capacity < 0");
    const Plan &p = h->plan;
    if (!p.append_ok) return set_err(FL_ERR_INVALID_ARG, "the plan has no append slots: " + p.append_err);
    const int32_t rows = (int32_t)p.append_rows.size();
    const int32_t n = std::min(capacity, rows);
    if (n > 0) std::memcpy(slots, p.append_rows.data(), (size_t)n * 4);
    if (num_rows) *num_rows = rows;
    return FL_OK;
}

fl_status fl_paged_attn_plan_info(fl_handle h, int32_t *num_work_items, int32_t *num_groups,
                                  int32_t *max_splits, int64_t *workspace_bytes) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "no plan");
    if (num_work_items) *num_work_items = h->plan.num_segs;
    if (num_groups) *num_groups = h->plan.num_groups;
    if (max_splits) *max_splits = h->plan.max_splits;
    const int64_t width = h->plan.whole_rows ? h->part_width : h->cfg.head_dim;
    if (workspace_bytes) *workspace_bytes = h->plan.part_rows * (width + 1) * 4;
    return FL_OK;
}

fl_status fl_paged_attn_plan_launch(fl_handle h, int32_t *launch_class, int32_t *fused_class,
                                    int32_t *grid, int32_t *busy_groups) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "no plan");
    const LaunchDesc d = launch_desc(h, h->plan);
    if (launch_class) *launch_class = d.cls;
    if (fused_class) *fused_class = d.fcls;
    if (grid) *grid = d.grid;
    if (busy_groups) *busy_groups = h->plan.num_groups;
    return FL_OK;
}

fl_status fl_paged_attn_refused_launches(fl_handle h, int32_t *count) {
    g_last_error.clear();
    if (!h || !count) return set_err(FL_ERR_INVALID_ARG, "handle or count is NULL");
    *count = 0;
    if (h->host_only) return FL_OK;
    hipError_t e;
    if ((e = hipSetDevice(h->device)) != hipSuccess) return hip_err(e, "hipSetDevice");
    if ((e = hipDeviceSynchronize()) != hipSuccess) return hip_err(e, "hipDeviceSynchronize");
    if ((e = hipMemcpy(count, h->d_meta + h->off_status, 4, hipMemcpyDeviceToHost)) != hipSuccess)
        return hip_err(e, "hipMemcpy (status)");
    if ((e = hipMemset(h->d_meta + h->off_status, 0, 4)) != hipSuccess ||
        (e = hipDeviceSynchronize()) != hipSuccess)
        return hip_err(e, "hipMemset (status)");
    return FL_OK;
}

fl_status fl_paged_attn_get_work_items(fl_handle h, int32_t *items, int32_t capacity,
                                       int32_t *num_items) {
    g_last_error.clear();
    if (!h) return set_err(FL_ERR_INVALID_ARG, "handle is NULL");
    if (!h->planned) return set_err(FL_ERR_NOT_PLANNED, "no plan");
    if (capacity < 0 || (capacity > 0 && !items))
        return set_err(FL_ERR_INVALID_ARG, "items is NULL or capacity < 0");
    // the plan's segment slots without the empty ones of quads with fewer than four blocks
    const Plan &p = h->plan;
    int32_t n = 0;
    for (int32_t i = 0; i < p.num_seg_slots && n < capacity; ++i) {
        const int32_t *it = &p.segs[(size_t)i * FL_WORK_ITEM_INTS];
        if (it[FL_WI_NUM_ROWS] == 0) continue;
        std::memcpy(items + (size_t)n * FL_WORK_ITEM_INTS, it, FL_WORK_ITEM_INTS * 4);
        if (p.whole_rows)  // the kernel's virtual kv head 0 is every real kv head
            items[(size_t)n * FL_WORK_ITEM_INTS + FL_WI_KV_HEAD] = -1;
        ++n;
    }
    if (num_items) *num_items = p.num_segs;
    return FL_OK;
}

}  // extern "C"
