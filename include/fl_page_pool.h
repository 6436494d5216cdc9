/*
 * fl_page_pool.h — the page allocator that produces the page tables fl_paged_attn_plan
 * reads, and the poisoning of freed pages.
 *
 * A pool of num_pages fixed-size pages (page_size token slots each) is handed out from a
 * free list, and every page carries an explicit reference count, so requests that share a
 * cached prompt prefix hold the same physical pages read-only (flashlet README: repository
 * layout, kv_cache.py: paged KV pool, free-list allocator, radix cache with refcounts;
 * design bullets: radix prefix cache with explicit page refcounts). Space is reserved a
 * whole page at a time: a request needing n slots holds ceil(n / page_size) pages ("A
 * library kernel for decode", What changed). When a page's last holder releases it, the
 * page returns to the free list and the caller may poison its K/V contents on the GPU so
 * that any later read of it shows up as NaN ("A library kernel for decode", closing
 * paragraph: freed-page poisoning among the engine's gates).
 *
 * The allocator is host bookkeeping only: it never touches device memory. Which free page
 * an allocation returns is unspecified (any free page is correct); today the free list is
 * last-in first-out, starting with page 0, 1, 2, ... on a fresh pool. Reference counts,
 * free counts and which pages a release frees are fully determined.
 *
 * Errors: the status codes and fl_last_error() of fl_paged_attn.h. A call that fails
 * changes nothing. A pool handle is not thread-safe (one scheduler thread owns it).
 */
#ifndef FL_PAGE_POOL_H
#define FL_PAGE_POOL_H

#include <stdint.h>

#include "fl_paged_attn.h"

#ifdef __cplusplus
extern "C" {
#endif

typedef struct fl_page_pool *fl_page_pool_t;

/* A pool of num_pages pages in [1, 2^31) of page_size >= 1 slots, all free. */
fl_status fl_page_pool_create(int64_t num_pages, int32_t page_size, fl_page_pool_t *out);

/* Free the pool's bookkeeping. NULL is a no-op. */
fl_status fl_page_pool_destroy(fl_page_pool_t pool);

/*
 * Take n >= 0 free pages, each with reference count 1; their ids go to page_ids[0..n).
 * All or nothing: FL_ERR_CAPACITY (nothing taken) when fewer than n pages are free.
 */
fl_status fl_page_pool_alloc(fl_page_pool_t pool, int32_t n, int32_t *page_ids);

/*
 * Reserve room for `tokens` >= 0 slots a whole page at a time: ceil(tokens / page_size)
 * pages, as fl_page_pool_alloc. *num_pages receives the page count; FL_ERR_CAPACITY
 * (nothing taken) when it exceeds `capacity` or the free pages.
 */
fl_status fl_page_pool_reserve(fl_page_pool_t pool, int64_t tokens, int32_t *page_ids,
                               int32_t capacity, int32_t *num_pages);

/*
 * One more holder for each listed page (a page listed twice gains two), for a request
 * that adopts pages another request holds (a shared prefix). Every page must be held
 * already: FL_ERR_INVALID_ARG otherwise, and nothing changes.
 */
fl_status fl_page_pool_retain(fl_page_pool_t pool, const int32_t *page_ids, int32_t n);

/*
 * One holder fewer for each listed page. Pages whose count reaches zero return to the
 * free list; their ids are written to freed[0 .. *num_freed) (freed may be NULL; it needs
 * room for n ids) in the order the counts reach zero while the list is walked from first
 * to last. FL_ERR_INVALID_ARG, with nothing changed, when a page is listed more often
 * than it is held (a free page included).
 */
fl_status fl_page_pool_release(fl_page_pool_t pool, const int32_t *page_ids, int32_t n,
                               int32_t *freed, int32_t *num_freed);

/* Reference counts of the listed pages (0 = free) into refs[0..n). */
fl_status fl_page_pool_refcounts(fl_page_pool_t pool, const int32_t *page_ids, int32_t n,
                                 int32_t *refs);

/* Free and held page counts; either output may be NULL. */
fl_status fl_page_pool_info(fl_page_pool_t pool, int64_t *num_free, int64_t *num_held);

/*
 * Poison pages of one layer's pools on the GPU: every element of each listed page of
 * k_pool (and v_pool, unless NULL), laid out [num_pages, page_size, num_kv_heads,
 * head_dim] in fl_dtype `dtype`, becomes that type's quiet NaN with a clear sign and a
 * zero payload (fp16 0x7E00, bf16 0x7FC0, fp32 0x7FC00000). Other pages are untouched; a
 * page listed twice is poisoned once.
 *   page_ids   host int32[n], each in [0, num_pages); copied into the launch arguments
 *              (ceil(n / 256) launches), so the array may be reused when this returns
 *   k_pool     device, 16-byte aligned; v_pool likewise or NULL
 *   stream     hipStream_t (NULL: the null stream); enqueues and returns, allocates
 *              nothing
 * Errors: FL_ERR_INVALID_ARG for an id outside the pool, a NULL or misaligned pool, or a
 * page whose byte size is not a multiple of 16; FL_ERR_UNSUPPORTED for an unknown dtype;
 * FL_ERR_HIP if a launch fails.
 */
fl_status fl_paged_kv_poison(int32_t dtype, int32_t page_size, int32_t num_kv_heads,
                             int32_t head_dim, int64_t num_pages, const int32_t *page_ids,
                             int32_t n, void *k_pool, void *v_pool, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* FL_PAGE_POOL_H */
