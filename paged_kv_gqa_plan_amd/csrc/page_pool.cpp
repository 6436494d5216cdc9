// Page allocator for the paged KV pool: a free list plus one reference count per page,
// host bookkeeping only (flashlet README: kv_cache.py's free-list allocator and page
// refcounts for shared prompt prefixes; "A library kernel for decode", What changed:
// space reserved a whole page at a time). The poisoning of freed pages is the GPU's part
// (fl_paged_kv_poison, kv_poison.hip).
#include <algorithm>
#include <cstdint>
#include <new>
#include <string>
#include <vector>

#include "fl_internal.h"
#include "fl_page_pool.h"

struct fl_page_pool {
    int64_t num_pages = 0;
    int32_t page_size = 1;
    std::vector<int32_t> free_list;  // a stack: the last page pushed is handed out first
    std::vector<int32_t> refs;       // 0 = free
};

namespace {

using fl::set_error;

// Holders each listed page loses in one release, checked against its count before
// anything changes; returns false with a message on the first violation.
bool check_release(const fl_page_pool *p, const int32_t *ids, int32_t n, std::string *msg) {
    std::vector<int32_t> s(ids, ids + n);
    std::sort(s.begin(), s.end());
    for (size_t i = 0; i < s.size();) {
        size_t j = i;
        while (j < s.size() && s[j] == s[i]) ++j;
        const int32_t id = s[i];
        if (id < 0 || id >= p->num_pages) {
            *msg = "release of page " + std::to_string(id) + ", outside the pool of " +
                   std::to_string(p->num_pages);
            return false;
        }
        if ((int64_t)(j - i) > p->refs[id]) {
            *msg = "release of page " + std::to_string(id) + " " + std::to_string(j - i) +
                   " time(s) with " + std::to_string(p->refs[id]) + " holder(s)";
            return false;
        }
        i = j;
    }
    return true;
}

}  // namespace

extern "C" {

fl_status fl_page_pool_create(int64_t num_pages, int32_t page_size, fl_page_pool_t *out) {
    fl::clear_error();
    if (!out) return set_error(FL_ERR_INVALID_ARG, "out is NULL");
    *out = nullptr;
    if (num_pages < 1 || num_pages > INT32_MAX)
        return set_error(FL_ERR_INVALID_ARG, "num_pages must be in [1, 2^31)");
    if (page_size < 1) return set_error(FL_ERR_INVALID_ARG, "page_size must be >= 1");
    fl_page_pool *p = new (std::nothrow) fl_page_pool();
    if (!p) return set_error(FL_ERR_CAPACITY, "out of host memory");
    try {
        p->free_list.resize((size_t)num_pages);
        p->refs.assign((size_t)num_pages, 0);
    } catch (const std::bad_alloc &) {
        delete p;
        return set_error(FL_ERR_CAPACITY, "out of host memory");
    }
    p->num_pages = num_pages;
    p->page_size = page_size;
    for (int64_t i = 0; i < num_pages; ++i)  // page 0 on top
        p->free_list[(size_t)i] = (int32_t)(num_pages - 1 - i);
    *out = p;
    return FL_OK;
}

fl_status fl_page_pool_destroy(fl_page_pool_t pool) {
    fl::clear_error();
    delete pool;
    return FL_OK;
}

fl_status fl_page_pool_alloc(fl_page_pool_t pool, int32_t n, int32_t *page_ids) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0 || (n > 0 && !page_ids)) return set_error(FL_ERR_INVALID_ARG, "n < 0 or page_ids is NULL");
    if ((size_t)n > pool->free_list.size())
        return set_error(FL_ERR_CAPACITY, std::to_string(n) + " pages asked, " +
                                              std::to_string(pool->free_list.size()) + " free");
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = pool->free_list.back();
        pool->free_list.pop_back();
        pool->refs[id] = 1;
        page_ids[i] = id;
    }
    return FL_OK;
}

fl_status fl_page_pool_reserve(fl_page_pool_t pool, int64_t tokens, int32_t *page_ids,
                               int32_t capacity, int32_t *num_pages) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (tokens < 0 || capacity < 0) return set_error(FL_ERR_INVALID_ARG, "tokens or capacity < 0");
    const int64_t need = (tokens + pool->page_size - 1) / pool->page_size;
    if (num_pages) *num_pages = (int32_t)std::min<int64_t>(need, INT32_MAX);
    if (need > capacity)
        return set_error(FL_ERR_CAPACITY, std::to_string(tokens) + " slots need " +
                                              std::to_string(need) + " pages; room for " +
                                              std::to_string(capacity) + " ids");
    return fl_page_pool_alloc(pool, (int32_t)need, page_ids);
}

fl_status fl_page_pool_retain(fl_page_pool_t pool, const int32_t *page_ids, int32_t n) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0 || (n > 0 && !page_ids)) return set_error(FL_ERR_INVALID_ARG, "n < 0 or page_ids is NULL");
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = page_ids[i];
        if (id < 0 || id >= pool->num_pages || pool->refs[id] == 0)
            return set_error(FL_ERR_INVALID_ARG, "retain of page " + std::to_string(id) +
                                                     ", which is not held");
    }
    for (int32_t i = 0; i < n; ++i)
        if (pool->refs[page_ids[i]] == INT32_MAX)
            return set_error(FL_ERR_CAPACITY, "page " + std::to_string(page_ids[i]) +
                                                  " has 2^31 - 1 holders");
    for (int32_t i = 0; i < n; ++i) ++pool->refs[page_ids[i]];
    return FL_OK;
}

fl_status fl_page_pool_release(fl_page_pool_t pool, const int32_t *page_ids, int32_t n,
                               int32_t *freed, int32_t *num_freed) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0 || (n > 0 && !page_ids)) return set_error(FL_ERR_INVALID_ARG, "n < 0 or page_ids is NULL");
    std::string msg;
    if (!check_release(pool, page_ids, n, &msg)) return set_error(FL_ERR_INVALID_ARG, msg);
    int32_t nf = 0;
    for (int32_t i = 0; i < n; ++i) {
        const int32_t id = page_ids[i];
        if (--pool->refs[id] == 0) {
            pool->free_list.push_back(id);
            if (freed) freed[nf] = id;
            ++nf;
        }
    }
    if (num_freed) *num_freed = nf;
    return FL_OK;
}

fl_status fl_page_pool_refcounts(fl_page_pool_t pool, const int32_t *page_ids, int32_t n,
                                 int32_t *refs) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (n < 0 || (n > 0 && (!page_ids || !refs)))
        return set_error(FL_ERR_INVALID_ARG, "n < 0 or a NULL array");
    for (int32_t i = 0; i < n; ++i)
        if (page_ids[i] < 0 || page_ids[i] >= pool->num_pages)
            return set_error(FL_ERR_INVALID_ARG, "page " + std::to_string(page_ids[i]) + " outside the pool");
    for (int32_t i = 0; i < n; ++i) refs[i] = pool->refs[page_ids[i]];
    return FL_OK;
}

fl_status fl_page_pool_info(fl_page_pool_t pool, int64_t *num_free, int64_t *num_held) {
    fl::clear_error();
    if (!pool) return set_error(FL_ERR_INVALID_ARG, "pool is NULL");
    if (num_free) *num_free = (int64_t)pool->free_list.size();
    if (num_held) *num_held = pool->num_pages - (int64_t)pool->free_list.size();
    return FL_OK;
}

}  // extern "C"
