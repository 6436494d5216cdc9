/*
 * fl_paged_attn.h — batched grouped-query attention over a paged KV cache (gfx950).
 *
 * One plan per scheduling step, one run per layer, following the plan()/run() split of
 * an attention backend (flashlet README, repository layout: backends/base.py) and the
 * practice of keeping per-step metadata in persistent device buffers that are updated
 * in place (flashlet README, design bullets: metadata updated in place each step, so the
 * launches can be captured in a graph; Torchlet README, Implemented Versions: static
 * buffers, then the decode step captured once and replayed).
 *
 * Graph replay. Every plan has a launch class (fl_paged_attn_plan_launch). Two plans of
 * one class make run() -- and each of the append calls -- enqueue exactly the same
 * launches (grid, kernel, arguments): everything that differs between them (lengths, page
 * ids, request count, causal flag, scale, how many workgroups have work) travels in the
 * handle's device metadata, which plan() rewrites in place. So a HIP graph captured from
 * run() calls replays correctly after any later plan of the same class, as long as the
 * captured q / out / lse / new-row buffers hold that plan's rows (size them for
 * max_qo_rows) and the pools hold its pages. The class depends only on the kind of step:
 * decode-only steps (every request at most one query row) share one class per handle,
 * steps with prefill rows another (at head_dim 64 in a 16-bit type they run two
 * workgroups per compute unit), decode steps in whole-row blocks (fl_config.whole_rows)
 * a third; a plan with num_splits > 0 has a class of its own grid. A launch replayed
 * after a plan of another class does not compute: it touches no memory but the handle's
 * status word, where fl_paged_attn_refused_launches() counts it.
 *
 * Operation (run). For request r with query rows qo_indptr[r] .. qo_indptr[r+1] and
 * pages kv_indices[kv_indptr[r] .. kv_indptr[r+1]) holding
 *     kv_len[r] = (kv_indptr[r+1] - kv_indptr[r] - 1) * page_size + last_page_len[r]
 * cached tokens (token t lives in page kv_indices[kv_indptr[r] + t / page_size], slot
 * t % page_size), every query row i and query head h computes softmax attention
 *     out[row, h, :] = sum_t softmax_t(sm_scale * q[row, h, :] . K[t, h / G, :]) V[t, h / G, :]
 * with G = num_qo_heads / num_kv_heads (grouped-query attention, Torchlet README) over the
 * keys t <= kv_len - qo_len + i when causal (bottom-right alignment: a decode row sees its
 * whole history, a prefill chunk's rows see the history plus the chunk up to themselves;
 * flashlet README, design bullets: one ragged call covers prefill chunks and decode rows
 * and the causal mask covers both), or all kv_len keys otherwise.
 * Long histories are cut into slices that run on different compute units and the
 * per-slice results are merged by log-sum-exp ("A library kernel for decode",
 * What changed); the result is the same attention up to floating-point rounding.
 *
 * Memory layout (all row-major, contiguous):
 *   q, out       [rows, num_qo_heads, head_dim]           rows = qo_indptr[batch]
 *   k_pool,
 *   v_pool       [num_pages, page_size, num_kv_heads, head_dim]   one layer
 *                (the NHD pool of the flashlet README, design bullets)
 *   lse          [rows, num_qo_heads] float, natural log of the softmax denominator
 *                plus the row maximum (optional)
 * q, the pools and out share one element type (fl_dtype). Accumulation is fp32.
 *
 * Ownership. The caller owns every pointer it passes. fl_paged_attn_plan copies the host
 * arrays before it returns. The handle owns its persistent device metadata buffers, its
 * fp32 partial-result workspace (sized at create time from fl_config) and two pinned host
 * staging buffers.
 *
 * Streams. plan() validates and partitions on the host, then enqueues one host-to-device
 * copy of the work list on `stream`. run() only enqueues kernels on `stream`; it neither
 * allocates nor synchronises. plan() and run() of one handle must be ordered on one
 * stream (or the caller orders them). A handle is not thread-safe.
 *
 * Errors. Every call returns an fl_status; on failure fl_last_error() gives a message
 * (thread-local, valid until the next call on that thread). No exception crosses this
 * interface. A failed plan leaves the handle un-planned; run() then returns
 * FL_ERR_NOT_PLANNED. Page ids are checked on the host at plan time; kernels do no
 * bounds checks of their own.
 */
#ifndef FL_PAGED_ATTN_H
#define FL_PAGED_ATTN_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FL_OK = 0,
    FL_ERR_INVALID_ARG = -1,   /* inconsistent metadata, NULL pointer, bad sizes       */
    FL_ERR_UNSUPPORTED = -2,   /* head_dim, page_size, dtype or group outside the set   */
    FL_ERR_CAPACITY = -3,      /* batch, rows, pages or splits beyond the handle's caps */
    FL_ERR_NOT_PLANNED = -4,   /* run() before a successful plan()                      */
    FL_ERR_HIP = -5            /* a HIP runtime call failed (message has the HIP error) */
} fl_status;

typedef enum { FL_F16 = 1, FL_BF16 = 2, FL_F32 = 3 } fl_dtype;

typedef struct fl_paged_attn *fl_handle;

typedef struct {
    int32_t num_qo_heads;      /* Hq, a multiple of num_kv_heads                         */
    int32_t num_kv_heads;      /* Hkv >= 1                                               */
    int32_t head_dim;          /* 64 or 128                                              */
    int32_t page_size;         /* power of two in [16, 256]                              */
    int32_t dtype;             /* fl_dtype of q, pools and out                           */
    int32_t max_batch;         /* most requests one plan may hold                        */
    int32_t max_qo_rows;       /* most query rows one plan may hold (qo_indptr[batch]);
                                  (max_qo_rows * G + 16) * G must be below 2^32          */
    int64_t max_kv_pages;      /* most page-table entries one plan may hold              */
    int32_t num_cus;           /* compute units to plan for; 0 = ask the device
                                  (a host-only handle then plans for 256)                */
    int32_t groups_per_cu;     /* workgroups per compute unit the plan spreads work over;
                                  0 = chosen per step (2 when the step has prefill rows
                                  at head_dim 64 in a 16-bit type, else 1)               */
    int32_t min_group_tokens;  /* fewest keys (per row block piece) a workgroup's share
                                  may hold before fewer workgroups are used; 0 = default */
    int32_t waves_per_group;   /* wavefronts per workgroup: 4 (0 = the same)              */
    int64_t max_tiles;         /* most 16-key tiles (over all row blocks) one plan may
                                  hold; 0 = a bound derived from the other capacities     */
    int32_t whole_rows;        /* Whole-row blocks: one row block holds all query heads
                                  of a request and streams whole token rows (every kv
                                  head) at once. They apply to decode-only steps (every
                                  request has at most one query row) with num_kv_heads *
                                  head_dim = 128, num_kv_heads > 1, at most 16 query heads
                                  and a 16-bit type. 0: used where they apply and the step
                                  has at least one query row per compute unit; 1: used on
                                  every decode-only step (create returns
                                  FL_ERR_UNSUPPORTED for a shape that cannot take them);
                                  -1: never (one block per kv head)                       */
} fl_config;

/*
 * Create a handle for one configuration on HIP device `device` (>= 0). device == -1 makes
 * a host-only handle: plan() validates and builds the work list without any HIP call
 * (for inspecting plans on machines without a GPU); run() on it returns
 * FL_ERR_UNSUPPORTED. On success *out receives the handle.
 */
fl_status fl_paged_attn_create(const fl_config *cfg, int device, fl_handle *out);

/* Free the handle and everything it owns. Waits for the handle's pending work. NULL is a no-op. */
fl_status fl_paged_attn_destroy(fl_handle h);

/*
 * Build the work list for one step (once per step, shared by every layer's run()).
 *   batch            number of requests, 0 <= batch <= max_batch
 *   qo_indptr        host int32[batch+1], prefix sums of query rows per request, [0] = 0;
 *                    NULL means one row per request (pure decode). A request may have
 *                    0 rows. With causal != 0 each request needs qo_len <= kv_len.
 *   kv_indptr        host int32[batch+1], prefix sums of pages per request, [0] = 0;
 *                    every request holds at least one page (kv_len >= 1)
 *   kv_indices       host int32[kv_indptr[batch]], physical page ids in [0, num_pages);
 *                    requests may share pages (read-only prefix sharing)
 *   last_page_len    host int32[batch], each in [1, page_size]
 *   num_pages        pool size, the bound for page ids
 *   causal           nonzero: bottom-right causal mask (a no-op for single decode rows)
 *   sm_scale         softmax scale; <= 0 means 1/sqrt(head_dim)
 *   num_splits       0: the planner spreads all row blocks' tiles evenly over the compute
 *                    units; > 0: cut every row block's keys into that many pieces (fewer
 *                    when the history has fewer 16-token tiles), one workgroup each
 *   stream           hipStream_t for the host-to-device copy (NULL: the null stream)
 * The work list depends only on the lengths, never on page ids, so two plans over the
 * same lengths give bit-identical results for any page assignment.
 */
fl_status fl_paged_attn_plan(fl_handle h, int32_t batch, const int32_t *qo_indptr,
                             const int32_t *kv_indptr, const int32_t *kv_indices,
                             const int32_t *last_page_len, int64_t num_pages, int32_t causal,
                             float sm_scale, int32_t num_splits, void *stream);

/*
 * Compute attention for one layer with the current plan: one kernel launch (also for an
 * empty plan, whose workgroups all exit at once). Row blocks cut into several pieces are
 * merged inside the same launch by the piece that finishes last. Device pointers:
 *   q       [rows, num_qo_heads, head_dim]
 *   k_pool  [num_pages, page_size, num_kv_heads, head_dim]
 *   v_pool  same layout as k_pool
 *   out     [rows, num_qo_heads, head_dim], written in full
 *   lse     float[rows, num_qo_heads] or NULL
 * All pointers 16-byte aligned. Enqueues on `stream` and returns; never synchronises or
 * allocates, so it may be captured into a HIP graph (valid for every later plan of the
 * same launch class; see "Graph replay" above).
 */
fl_status fl_paged_attn_run(fl_handle h, const void *q, const void *k_pool, const void *v_pool,
                            void *out, float *lse, void *stream);

/*
 * fl_paged_attn_run without any device allocation, for callers that cannot allocate
 * device memory (code that may not call hipMalloc: tight serving loops, harnesses that
 * forbid it). The same attention as fl_paged_attn_run on the handle's current plan, with
 * the same kernel and launch (so the same bits), but every device buffer beyond q, the
 * pools, out and lse -- the plan's metadata, the merge tickets and the fp32 partial rows
 * -- lives in one fixed device array of the library (16 MiB per GPU, held by each GPU the
 * library runs on until the process ends). The handle may be host-only (device -1:
 * created and planned without any HIP call); the call then runs on the current device.
 * Each call copies the plan's metadata from the handle's host memory (pageable; the copies
 * have read their source when the call returns) and clears the merge tickets with a small
 * kernel, on `stream`. Calls on one GPU share the array: calls that overlap on one GPU
 * (different streams or threads) race; calls ordered on one stream do not.
 * Pointers and layouts as for fl_paged_attn_run. Errors: those of fl_paged_attn_run, and
 * FL_ERR_CAPACITY (with the sizes) when the plan needs more than the array holds.
 */
fl_status fl_paged_attn_run_noalloc(fl_handle h, const void *q, const void *k_pool,
                                    const void *v_pool, void *out, float *lse, void *stream);

/*
 * Append one layer's new K and V rows to the paged pools with the current plan, before
 * that layer's run() reads them (flashlet README, design bullets: set_kv writes the new
 * tokens into the NHD pool in place with one indexed copy; the pool keeps every layer's
 * pages in the same layout). One kernel launch.
 *
 * Query row i of request r (global row qo_indptr[r] + i) stands for the request's token
 * kv_len[r] - qo_len[r] + i, the position the causal mask gives it: the kv_len passed to
 * plan() already counts the step's new tokens. That token lives in page
 * kv_indices[kv_indptr[r] + t / page_size], slot t % page_size. Its K row
 *     k_pool[page, slot, :, :] = k_new[qo_indptr[r] + i, :, :]
 * and likewise for V; every other slot of the pools is left as it was. The copy moves
 * bytes, so it is exact for every element type.
 * Device pointers:
 *   k_new, v_new    [rows, num_kv_heads, head_dim], rows = qo_indptr[batch] of the plan
 *   k_pool, v_pool  [num_pages, page_size, num_kv_heads, head_dim], one layer
 * All pointers 16-byte aligned; the element type is the handle's fl_dtype. Enqueues on
 * `stream` and returns; never synchronises or allocates. The launch is the same for every
 * plan of the handle (its grid covers max_qo_rows rows; the row count and slots come from
 * the device metadata), so a captured append replays correctly after any later plan; a
 * replay after a plan without valid append slots writes nothing and is counted by
 * fl_paged_attn_refused_launches().
 * Errors: FL_ERR_NOT_PLANNED before a successful plan; FL_ERR_INVALID_ARG when a request
 * of the plan has more query rows than cached tokens (possible without the causal mask),
 * when two rows would write the same slot (a new token in a page two requests share), or
 * for NULL or misaligned pointers; FL_ERR_UNSUPPORTED on a host-only handle, or when
 * max_qo_rows x (token row bytes / 16) reaches 2^31. A plan of zero rows writes nothing.
 */
fl_status fl_paged_kv_append(fl_handle h, const void *k_new, const void *v_new, void *k_pool,
                             void *v_pool, void *stream);

/*
 * The same append fused with the rotary position embedding (RoPE) of the step's new rows:
 * one kernel launch rotates each new row's key heads by its token's position before they
 * are written to the pool, copies its value heads unchanged, and rotates its query heads in
 * place for the run() that follows. The pages apply RoPE in the Qwen2.5-style decoder they
 * run (Torchlet README, the running example; flashlet README, roadmap: a RoPE fusion
 * kernel) without spelling it out; this follows that model family's rotate-half form.
 *
 * Row i of request r has position t = kv_len[r] - qo_len[r] + i (as for the plain append).
 * For each head vector x (head_dim D) and i < D/2, with f_i = rope_theta^(-2i/D) rounded
 * to fp32 and the fp32 angle a = (float)t * f_i:
 *     x'[i]       = x[i] cos a - x[i + D/2] sin a
 *     x'[i + D/2] = x[i + D/2] cos a + x[i] sin a
 * computed in fp32 and rounded once to the element type. Then
 *     k_pool[page, slot, :, :] = rotated k_new[qo_indptr[r] + i, :, :]
 *     v_pool[page, slot, :, :] = v_new[qo_indptr[r] + i, :, :]
 *     q[qo_indptr[r] + i, :, :] = rotated q[...]          (skipped when q is NULL)
 * Device pointers: q [rows, num_qo_heads, head_dim] (read and written; may be NULL),
 * k_new, v_new, k_pool, v_pool as for fl_paged_kv_append, each aligned to the element size.
 * rope_theta: the base (e.g. 1e4, or 1e6 for Qwen2.5). Enqueues on `stream`; never
 * synchronises or allocates; one launch for every plan of the handle, as for
 * fl_paged_kv_append (graph-capturable).
 * Errors: as fl_paged_kv_append, plus FL_ERR_INVALID_ARG for rope_theta <= 0 or not finite
 * and FL_ERR_UNSUPPORTED for an odd head_dim or one above 128.
 */
fl_status fl_paged_kv_append_rope(fl_handle h, void *q, const void *k_new, const void *v_new,
                                  void *k_pool, void *v_pool, float rope_theta, void *stream);

/*
 * Append one layer's new K/V rows and compute that layer's attention in one call: the
 * result equals fl_paged_kv_append followed by fl_paged_attn_run (same pointers, same
 * plan), up to the floating-point summation order. On decode-only plans (every request has
 * at most one query row) in a 16-bit type with at most 16 query heads per kv head it is
 * one kernel launch: the new token is the
 * newest key of its request, so the workgroup whose tiles hold that key takes its K and V
 * from k_new / v_new instead of the pool and also writes them to the pool for later steps
 * (flashlet README, design bullets: the NHD pool is written in place before attention reads
 * it; one launch less per layer). Other plans (prefill chunks, whose new keys many
 * workgroups read; decode rows of more than 16 query heads per kv head, which run as
 * prefill units; fp32) make the two launches in order.
 * Device pointers as for fl_paged_kv_append and fl_paged_attn_run; all 16-byte aligned.
 * Errors: those of the two calls (FL_ERR_INVALID_ARG when the plan has no valid append
 * slots). Enqueues on `stream`; never synchronises or allocates (graph-capturable: the
 * one-launch form carries the plan's fused class, fl_paged_attn_plan_launch).
 */
fl_status fl_paged_attn_run_append(fl_handle h, const void *q, const void *k_new, const void *v_new,
                                   void *k_pool, void *v_pool, void *out, float *lse, void *stream);

/*
 * Copy the current plan's append destinations to host memory: for each query row, the
 * token row page * page_size + slot that fl_paged_kv_append writes it to. *num_rows
 * receives the row count; at most `capacity` entries are written. Works on host-only
 * handles. FL_ERR_INVALID_ARG (with the reason) when the plan has no valid slots.
 */
fl_status fl_paged_kv_append_slots(fl_handle h, int32_t *slots, int32_t capacity,
                                   int32_t *num_rows);

/*
 * Facts about the current plan: the number of work items (segments, see below), the
 * number of workgroups of the attention launch, the largest number of pieces any row block
 * was cut into, and the fp32 partial-result bytes the plan uses. Outputs may be NULL.
 */
fl_status fl_paged_attn_plan_info(fl_handle h, int32_t *num_work_items, int32_t *num_groups,
                                  int32_t *max_splits, int64_t *workspace_bytes);

/*
 * The launch the current plan needs (works on host-only handles, which plan as the device
 * would): *launch_class names the kernel variant and grid of fl_paged_attn_run, and
 * *fused_class those of the one-launch fl_paged_attn_run_append (0 when the plan takes two
 * launches there: prefill rows, more than 16 query heads per kv head, fp32, or no valid
 * append slots); *grid is the number of workgroups launched and *busy_groups how many of
 * them have work (the rest exit at once).
 * Plans with equal classes launch identically, so a graph captured under one replays
 * correctly under the other. Outputs may be NULL. FL_ERR_NOT_PLANNED without a plan.
 */
fl_status fl_paged_attn_plan_launch(fl_handle h, int32_t *launch_class, int32_t *fused_class,
                                    int32_t *grid, int32_t *busy_groups);

/*
 * Number of launches of this handle refused since the last call (then reset to zero): a
 * launch refuses when the plan current at its execution has another launch class than
 * the one it was enqueued for (a graph replayed after a plan of another kind), or, for the
 * append kernels, when that plan has no valid append slots. A refused launch writes no
 * output. Waits for all work on the handle's device first (hipDeviceSynchronize).
 * Host-only handles report 0.
 */
fl_status fl_paged_attn_refused_launches(fl_handle h, int32_t *count);

/*
 * Copy the current plan's work items to host memory: FL_WORK_ITEM_INTS int32 per item,
 * fields as named by FL_WI_* below, ordered by workgroup. A work item (segment) is one
 * piece of a row block: up to 16 flattened query rows (query row * G + head in group) of
 * one request and kv head, over one range of keys. The plan lays every row block's 16-key
 * tiles in one sequence and gives each workgroup an equal contiguous share, so a
 * workgroup runs a few segments back to back and a long row block may span several
 * workgroups (its pieces are merged by log-sum-exp). On decode-only steps that qualify for
 * whole_rows (fl_config), a block holds all query heads of one request instead (flattened
 * row query row * num_qo_heads + head, FL_WI_KV_HEAD = -1) and streams every kv head's
 * slice of each token row at once. *num_items receives the item count; at most `capacity`
 * items are written.
 */
#define FL_WORK_ITEM_INTS 16
enum {
    FL_WI_Q_START = 0,   /* first query row of the request                              */
    FL_WI_QO_LEN = 1,    /* query rows of the request                                   */
    FL_WI_KV_LEN = 2,    /* cached tokens of the request                                */
    FL_WI_PAGE_BASE = 3, /* kv_indptr[request]                                          */
    FL_WI_KV_HEAD = 4,   /* -1: the block covers every kv head (whole token rows); its
                            flattened row is query row * num_qo_heads + head            */
    FL_WI_ROW_BEGIN = 5, /* first flattened row of the block                            */
    FL_WI_NUM_ROWS = 6,  /* rows in the block (<= 16)                                   */
    FL_WI_TOK_BEGIN = 7, /* key range [tok_begin, tok_end)                               */
    FL_WI_TOK_END = 8,
    FL_WI_PART_ROW = 9,  /* -1: writes the final output; else its rows in the workspace */
    FL_WI_REQUEST = 10,
    FL_WI_SPLIT = 11,    /* piece index within its row block                            */
    FL_WI_NUM_SPLITS = 12,
    FL_WI_MERGE = 13,    /* row block's merge ticket (-1 when the block is one piece)   */
    FL_WI_GROUP = 14,    /* workgroup that runs this item                               */
    FL_WI_POS_BEGIN = 15 /* first step of the item in its workgroup's per-wave sequence   */
};
fl_status fl_paged_attn_get_work_items(fl_handle h, int32_t *items, int32_t capacity,
                                       int32_t *num_items);

/* Message for the last failed call on this thread ("" if none). */
const char *fl_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* FL_PAGED_ATTN_H */
