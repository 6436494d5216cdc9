"""The library's page allocator against the reference bookkeeping (oracle/page_pool.py).

Which free page an allocation returns is the allocator's choice, so the model accepts
any valid choice (distinct, in range, free); reference counts, free counts and the pages
a release frees (and their order) must match exactly. CPU only.
"""
import numpy as np
import pytest

import paged_kv_gqa_plan_amd as fl
from oracle.page_pool import PagePoolModel, PoolModelError


def _expect(status, fn, *a, **kw):
    with pytest.raises(fl.FlError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_worked_sequence():
    """Request A takes two pages, B adopts A's first page and takes one of its own; A ends
    (frees only its private page), then B ends (frees both remaining pages, in list order)."""
    pool = fl.PagePool(4, 16)
    m = PagePoolModel(4, 16)
    a = pool.alloc(2)
    m.alloc(a)
    pool.retain(a[:1])
    m.retain(a[:1])
    b_own = pool.alloc(1)
    m.alloc(b_own)
    assert pool.refcounts(range(4)).tolist() == m.refs
    assert pool.info() == (m.num_free, m.num_live) == (1, 3)
    assert pool.release(a).tolist() == m.release(a) == [int(a[1])]
    b = [int(b_own[0]), int(a[0])]
    assert pool.release(b).tolist() == m.release(b) == b
    assert pool.info() == (4, 0)


def test_whole_page_reservation():
    pool = fl.PagePool(8, 256)
    assert len(pool.reserve(300)) == 2          # 300 slots hold 512
    assert len(pool.reserve(256)) == 1 and len(pool.reserve(257)) == 2
    assert len(pool.reserve(0)) == 0
    assert pool.info() == (3, 5)
    _expect(fl.FL_ERR_CAPACITY, pool.reserve, 4 * 256)   # 4 pages, 3 free: nothing taken
    assert pool.info() == (3, 5)
    _expect(fl.FL_ERR_CAPACITY, fl.fl_page_pool_reserve, pool.handle, 3 * 256, 2)  # too few ids
    assert pool.info() == (3, 5)


def test_fresh_pool_hands_out_low_pages_first_and_reuses_the_last_freed():
    pool = fl.PagePool(16, 16)
    assert pool.alloc(3).tolist() == [0, 1, 2]
    pool.release([1])
    assert pool.alloc(2).tolist() == [1, 3]


def test_errors_change_nothing():
    pool = fl.PagePool(4, 16)
    ids = pool.alloc(3)
    before = (pool.info(), pool.refcounts(range(4)).tolist())
    _expect(fl.FL_ERR_CAPACITY, pool.alloc, 2)
    _expect(fl.FL_ERR_INVALID_ARG, pool.release, [int(ids[0]), int(ids[0])])   # held once
    _expect(fl.FL_ERR_INVALID_ARG, pool.release, [int(ids[1]), 3])             # 3 is free
    _expect(fl.FL_ERR_INVALID_ARG, pool.release, [4])
    _expect(fl.FL_ERR_INVALID_ARG, pool.retain, [int(ids[2]), 3])
    _expect(fl.FL_ERR_INVALID_ARG, pool.retain, [-1])
    _expect(fl.FL_ERR_INVALID_ARG, pool.refcounts, [4])
    assert (pool.info(), pool.refcounts(range(4)).tolist()) == before
    _expect(fl.FL_ERR_INVALID_ARG, fl.fl_page_pool_create, 0, 16)
    _expect(fl.FL_ERR_INVALID_ARG, fl.fl_page_pool_create, 1 << 31, 16)
    _expect(fl.FL_ERR_INVALID_ARG, fl.fl_page_pool_create, 4, 0)
    fl.fl_page_pool_destroy(None)


@pytest.mark.parametrize("seed", range(6))
def test_random_serving_sequences_match_the_model(seed):
    """Requests arrive (reserving whole pages, some adopting a live request's prefix pages),
    grow by a page, and finish; every result is checked against the model."""
    rng = np.random.default_rng(seed)
    N, P = int(rng.integers(8, 200)), int(rng.choice([16, 64, 256]))
    pool, m = fl.PagePool(N, P), PagePoolModel(N, P)
    live = {}   # request -> list of pages it holds
    nxt = 0
    for _ in range(400):
        op = rng.integers(0, 4)
        if op == 0:                                   # admit a request
            tokens = int(rng.integers(0, 6 * P))
            need = m.pages_for(tokens)
            prefix = []
            if live and rng.random() < 0.5:
                donor = live[list(live)[int(rng.integers(len(live)))]]
                prefix = donor[:int(rng.integers(0, len(donor) + 1))]
            if m.can_alloc(need):
                if prefix:
                    pool.retain(prefix)
                    m.retain(prefix)
                ids = pool.reserve(tokens)
                assert len(ids) == need
                m.alloc(ids.tolist())
                live[nxt] = list(prefix) + ids.tolist()
                nxt += 1
            else:
                _expect(fl.FL_ERR_CAPACITY, pool.reserve, tokens)
        elif op == 1 and live:                        # a request grows by one page
            r = list(live)[int(rng.integers(len(live)))]
            if m.can_alloc(1):
                ids = pool.alloc(1)
                m.alloc(ids.tolist())
                live[r].append(int(ids[0]))
            else:
                _expect(fl.FL_ERR_CAPACITY, pool.alloc, 1)
        elif op == 2 and live:                        # a request finishes
            r = list(live)[int(rng.integers(len(live)))]
            pages = live.pop(r)
            assert pool.release(pages).tolist() == m.release(pages)
        elif op == 3:                                 # an invalid release is refused
            page = int(rng.integers(N))
            bad = [page] * (m.refs[page] + 1)         # one more time than it is held
            try:
                m.release(bad)
                raise AssertionError("model accepted an over-release")
            except PoolModelError:
                pass
            _expect(fl.FL_ERR_INVALID_ARG, pool.release, bad)
        assert pool.refcounts(range(N)).tolist() == m.refs
        assert pool.info() == (m.num_free, m.num_live)
