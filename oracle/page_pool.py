"""Reference bookkeeping for a paged-KV page allocator.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): the tests drive the library's
allocator and this model side by side. The model shares nothing with the library.

What it follows:
  * a pool of fixed-size pages handed out from a free list, with an explicit reference
    count per page so that requests sharing a cached prompt prefix hold the same pages
    (flashlet README: repository layout, kv_cache.py; design bullets: radix prefix cache
    with explicit page refcounts);
  * space reserved a whole page at a time: a request needing n slots holds
    ceil(n / page_size) pages ("A library kernel for decode", What changed: 300 slots on
    256-slot pages hold 512);
  * a page whose last holder lets go returns to the free list (and is poisoned there;
    "A library kernel for decode", closing paragraph).

Which free page an allocation returns is the allocator's choice (any free page is
correct), so ``alloc`` takes the ids the allocator chose and checks that they were valid
choices. Everything else is determined: reference counts, the free count, and which pages
a release frees, in the order their counts reach zero while the released list is walked
from first to last.
"""
from __future__ import annotations

from typing import List, Sequence


class PoolModelError(ValueError):
    pass


class PagePoolModel:
    def __init__(self, num_pages: int, page_size: int):
        if num_pages < 1 or page_size < 1:
            raise PoolModelError("num_pages and page_size must be >= 1")
        self.num_pages = num_pages
        self.page_size = page_size
        self.refs = [0] * num_pages

    def pages_for(self, tokens: int) -> int:
        """Whole pages that hold `tokens` slots."""
        if tokens < 0:
            raise PoolModelError("tokens < 0")
        return (tokens + self.page_size - 1) // self.page_size

    @property
    def num_free(self) -> int:
        return sum(1 for r in self.refs if r == 0)

    @property
    def num_live(self) -> int:
        return self.num_pages - self.num_free

    def can_alloc(self, n: int) -> bool:
        return 0 <= n <= self.num_free

    def alloc(self, chosen: Sequence[int]) -> None:
        """Accept the allocator's choice of pages: distinct, in range, all free."""
        chosen = list(chosen)
        if len(set(chosen)) != len(chosen):
            raise PoolModelError(f"allocation returned a page twice: {chosen}")
        for p in chosen:
            if not 0 <= p < self.num_pages:
                raise PoolModelError(f"page {p} outside the pool")
            if self.refs[p] != 0:
                raise PoolModelError(f"page {p} handed out while held ({self.refs[p]} refs)")
        for p in chosen:
            self.refs[p] = 1

    def retain(self, ids: Sequence[int]) -> None:
        """One more holder for each listed page (listed twice: two more). Every page must
        be held already; on error nothing changes."""
        for p in ids:
            if not 0 <= p < self.num_pages or self.refs[p] == 0:
                raise PoolModelError(f"retain of page {p}, which is not held")
        for p in ids:
            self.refs[p] += 1

    def release(self, ids: Sequence[int]) -> List[int]:
        """One holder fewer for each listed page; returns the pages that became free, in the
        order their counts reach zero. A page may not be released more often than it is
        held; on error nothing changes."""
        need = {}
        for p in ids:
            if not 0 <= p < self.num_pages:
                raise PoolModelError(f"release of page {p}, outside the pool")
            need[p] = need.get(p, 0) + 1
        for p, c in need.items():
            if c > self.refs[p]:
                raise PoolModelError(f"release of page {p} {c} times with {self.refs[p]} refs")
        freed = []
        for p in ids:
            self.refs[p] -= 1
            if self.refs[p] == 0:
                freed.append(p)
        return freed
