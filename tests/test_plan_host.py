"""Host-side checks of the C interface: exported symbols and the planner (no GPU needed).

The planner is exercised through host-only handles (device = -1), which validate the
metadata and build the work list without any HIP call.
"""
import os
import re

import numpy as np
import pytest

import paged_kv_gqa_plan_amd as fl
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fl_paged_attn.h")


def test_library_exports_every_declared_function():
    import glob
    text = "".join(open(h).read() for h in sorted(glob.glob(os.path.join(ROOT, "include", "*.h"))))
    declared = set(re.findall(r"^\s*(?:fl_status|const char \*)\s*(fl_\w+)\s*\(", text, re.M))
    assert declared == set(fl.EXPORTED)
    lib = fl.load_library()
    for name in declared:
        assert hasattr(lib, name), name


def host_handle(Hq=14, Hkv=2, D=64, P=16, dtype="bf16", max_batch=256, max_rows=4096,
                max_pages=1 << 20, **kw):
    return fl.PagedAttention(fl.make_config(Hq, Hkv, D, P, dtype, max_batch, max_rows, max_pages,
                                            **kw), device=-1)


def plan_batch(h, b, num_splits=0, causal=None):
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
           causal=b.causal if causal is None else causal, num_splits=num_splits)
    return h.work_items()


def quad_rows(b, r, whole=False):
    """Flattened rows per prefill unit of request r: 64 for a chunk of more than one 16-row
    block in a 16-bit type (the prefill path), else 0 (blocks of the decode path)."""
    G = b.num_qo_heads if whole else b.group
    return 64 if (b.dtype != "f32" and not whole and int(b.qo_lens[r]) * G > 16) else 0


def check_coverage(items, b, causal=True):
    """Every (request, kv head, flattened row) sees exactly its causal key range, once, in
    16-aligned non-empty slices; split items own disjoint partial rows. Whole-row items
    (kv_head -1) cover every kv head at once, their rows flattened over all query heads.
    Blocks of a prefill unit (64 flattened rows) span the keys of the unit's last row; the
    kernel masks each row at its own limit."""
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    col = lambda n: items[:, idx[n]]
    whole = bool((col("kv_head") == -1).any())
    assert not whole or (col("kv_head") == -1).all()
    G = b.num_qo_heads if whole else b.group
    kv_heads = [-1] if whole else range(b.num_kv_heads)
    assert (col("num_rows") >= 1).all() and (col("num_rows") <= 16).all()
    assert (col("tok_end") > col("tok_begin")).all()
    assert (col("tok_begin") % 16 == 0).all()
    cover = {}
    for it in items:
        key = (it[idx["request"]], it[idx["kv_head"]], it[idx["row_begin"]], it[idx["num_rows"]])
        cover.setdefault(key, []).append((it[idx["tok_begin"]], it[idx["tok_end"]], it[idx["split"]],
                                          it[idx["num_splits"]], it[idx["part_row"]]))
    seen_rows = {}
    part_used = set()
    for (r, h, f0, nr), sl in cover.items():
        kl, ql = int(b.kv_lens[r]), int(b.qo_lens[r])
        qr = quad_rows(b, r, whole)
        f_last = min(f0 // qr * qr + qr, ql * G) - 1 if qr else f0 + nr - 1
        kv_end = kl - ql + f_last // G + 1 if causal else kl
        sl.sort()
        assert sl[0][0] == 0 and sl[-1][1] == kv_end
        for a, c in zip(sl, sl[1:]):
            assert a[1] == c[0]
        ns = sl[0][3]
        assert len(sl) == ns and sorted(s[2] for s in sl) == list(range(ns))
        if ns == 1:
            assert sl[0][4] == -1
        else:
            for s in sl:
                rows = set(range(s[4], s[4] + nr))
                assert not (rows & part_used)
                part_used |= rows
        for f in range(f0, f0 + nr):
            seen_rows[(r, h, f)] = seen_rows.get((r, h, f), 0) + 1
    for r in range(b.batch_size):
        for h in kv_heads:
            for f in range(int(b.qo_lens[r]) * G):
                assert seen_rows.get((r, h, f)) == 1, (r, h, f)
    # a workgroup holds at most two cut pieces, its first and its last (the kernel keeps the
    # fields of two pending pieces for the merge tickets); the blocks of a quad piece are
    # one piece
    groups = col("group")
    for g in np.unique(groups):
        mine = np.nonzero(groups == g)[0]
        pieces, cut = [], set()
        for i in mine:
            it = items[i]
            r = it[idx["request"]]
            qr = quad_rows(b, r, whole)
            key = (r, it[idx["kv_head"]], it[idx["tok_begin"]],
                   it[idx["row_begin"]] // qr if qr else (-1, it[idx["row_begin"]]))
            if not pieces or pieces[-1] != key:
                pieces.append(key)
            if it[idx["part_row"]] >= 0:
                cut.add(len(pieces) - 1)
        assert len(cut) <= 2 and all(j in (0, len(pieces) - 1) for j in cut), (g, cut, len(pieces))
    # the items carry the right request facts
    for it in items:
        r = it[idx["request"]]
        assert it[idx["q_start"]] == b.qo_indptr[r] and it[idx["qo_len"]] == b.qo_lens[r]
        assert it[idx["kv_len"]] == b.kv_lens[r] and it[idx["page_base"]] == b.kv_indptr[r]


SHAPES = {
    "tiny_decode": lambda: W.tiny_decode(),
    "saturated_decode": lambda: W.saturated_decode(),
    "mixed_length_decode": lambda: W.make_batch(W.mixed_length_lengths(0), num_qo_heads=12, num_kv_heads=2,
                                                head_dim=64, page_size=256, dtype="f16", num_pages=1024),
    "long_context_skew": lambda: W.make_batch(W.long_context_lengths(0, long_len=4096), num_qo_heads=12,
                                              num_kv_heads=2, head_dim=64, page_size=256, dtype="f16"),
    "ragged_mixed_step": lambda: W.make_batch(*W.ragged_mixed_lengths(0), num_qo_heads=14, num_kv_heads=2,
                                              head_dim=64, page_size=16, dtype="bf16", num_pages=8192),
}


@pytest.mark.parametrize("name", sorted(SHAPES))
@pytest.mark.parametrize("splits", [0, 1, 3, 1000])
def test_plan_covers_every_row_and_key_once(name, splits):
    b = SHAPES[name]()
    h = host_handle(Hq=b.num_qo_heads, Hkv=b.num_kv_heads, D=64, P=b.page_size, dtype=b.dtype)
    if name == "ragged_mixed_step" and splits == 1000:
        # in fp32 (no prefill quads) every 16-key tile of the chunk's 448 row blocks its own
        # slice: beyond the handle's item capacity, reported as such
        hf = host_handle(Hq=b.num_qo_heads, Hkv=b.num_kv_heads, D=64, P=b.page_size, dtype="f32")
        assert "work items" in _expect(fl.FL_ERR_CAPACITY, plan_batch, hf, b, num_splits=splits)
    items = plan_batch(h, b, num_splits=splits)
    check_coverage(items, b)
    n, ng, ms, ws = h.info()
    assert n == len(items)
    assert ng == items[:, fl.WORK_ITEM_FIELDS.index("group")].max() + 1
    if splits == 1:
        assert ms == 1 and ws == 0


def _wide_plan_case(seed):
    """Lengths and shapes from a wide seeded space (page-table metadata only, no pools):
    head ratios 1-32, 1-8 kv heads, histories up to 9000 tokens, chunks up to 700 rows,
    requests without query rows, the mask, forced slices up to 50."""
    from types import SimpleNamespace
    r = np.random.default_rng(70000 + seed)
    dtype = ["bf16", "f16", "f32"][r.integers(3)]
    D = [64, 128][r.integers(2)]
    P = [16, 32, 64, 128, 256][r.integers(5)]
    Hkv = [1, 2, 4, 8][r.integers(4)]
    G = [1, 2, 3, 4, 5, 6, 7, 8, 12, 14, 16, 17, 20, 24, 31, 32][r.integers(16)]
    B = int(r.integers(1, 65))
    kinds = r.integers(5, size=B)
    kv = np.where(kinds == 0, r.integers(1, 40, size=B),
         np.where(kinds == 1, 16 * r.integers(1, 60, size=B),
         np.where(kinds == 2, P * r.integers(1, 8, size=B),
         np.where(kinds == 3, r.integers(40, 3000, size=B), r.integers(3000, 9000, size=B)))))
    qo = np.where(r.random(B) < 0.2, np.minimum(kv, r.integers(2, 700, size=B)), 1)
    if r.random() < 0.1:
        qo = np.where(r.random(B) < 0.3, 0, qo)
    causal = bool(r.random() < 0.85)
    splits = int([0, 0, 0, 0, 1, 2, 3, 7, 50][r.integers(9)])
    qo_indptr, kv_indptr, kv_indices, last, pool = _meta(kv, qo, P, r)
    b = SimpleNamespace(num_qo_heads=G * Hkv, num_kv_heads=Hkv, group=G, head_dim=D, page_size=P,
                        dtype=dtype, batch_size=B, kv_lens=kv.astype(np.int64), qo_lens=qo.astype(np.int64),
                        qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                        last_page_len=last, num_pages=pool, causal=causal)
    return b, splits


@pytest.mark.parametrize("seed", range(60))
def test_plan_covers_every_row_and_key_once_over_a_wide_space(seed):
    """Coverage, cut and request facts of the work list over 60 seeded shapes: every
    flattened row of every kv head sees exactly its causal key range, once. A plan beyond
    the handle's capacity (forced slices) is refused with FL_ERR_CAPACITY, nothing else."""
    b, splits = _wide_plan_case(seed)
    h = host_handle(Hq=b.num_qo_heads, Hkv=b.num_kv_heads, D=b.head_dim, P=b.page_size, dtype=b.dtype,
                    max_batch=64, max_rows=int(b.qo_lens.sum()) + 1, max_pages=int(b.num_pages) + 1,
                    num_cus=256)
    try:
        items = plan_batch(h, b, num_splits=splits)
    except fl.FlError as e:
        assert e.status == fl.FL_ERR_CAPACITY and splits > 0, str(e)
        return
    check_coverage(items, b, causal=b.causal)


def test_plan_non_causal_prefill_covers_whole_history():
    b = W.make_batch([60, 9, 300], [7, 3, 20], num_qo_heads=4, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="f32", causal=False)
    h = host_handle(Hq=4, Hkv=2, P=16, dtype="f32")
    items = plan_batch(h, b)
    check_coverage(items, b, causal=False)


def test_plan_depends_only_on_lengths():
    b = W.saturated_decode()
    b2 = W.relabel_pages(b, W.rng_for(5, 0, 0).permutation(b.num_pages))
    h = host_handle()
    i1 = plan_batch(h, b)
    i2 = plan_batch(h, b2)
    assert np.array_equal(i1, i2)
    assert np.array_equal(plan_batch(h, b), i1)   # and deterministic


def tiles_per_group(items):
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    g = items[:, idx["group"]]
    t = -(-(items[:, idx["tok_end"]] - items[:, idx["tok_begin"]]) // 16)
    return np.bincount(g, weights=t).astype(int)


STEP_GROUP = 8        # tiles of one ring step group of a 4-wave workgroup (4 waves x 2)
FOLD_COST = 6         # the planner's charge for one segment fold, in tiles (decode-only step)
CUT_COST = 4          # and for a piece of a block cut by a share boundary


def cost_per_group(items):
    """The planner's time estimate per workgroup of a decode-only step: each piece's tiles
    rounded up to whole step groups, plus one fold charge per piece and a cut charge per
    piece of a block that was cut."""
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    g = items[:, idx["group"]]
    t = -(-(items[:, idx["tok_end"]] - items[:, idx["tok_begin"]]) // 16)
    c = STEP_GROUP * -(-t // STEP_GROUP) + FOLD_COST + CUT_COST * (items[:, idx["num_splits"]] > 1)
    return np.bincount(g, weights=c).astype(int)


def test_long_histories_are_spread_and_shares_are_balanced():
    lens = W.long_context_lengths(0)
    b = W.make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=64, page_size=256,
                     dtype="f16", num_pages=1200, poison=False)
    h = host_handle(Hq=12, Hkv=2, P=256, dtype="f16", max_pages=4096, num_cus=256, whole_rows=-1)
    items = plan_batch(h, b)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    kvl = items[:, idx["kv_len"]]
    ns = items[:, idx["num_splits"]]
    assert ns[kvl == 32768].min() >= 8          # one long history runs on many CUs
    assert ns[kvl == 512].max() <= 2            # short ones stay (nearly) whole
    tpg = tiles_per_group(items)
    assert len(tpg) == 256                      # one share per compute unit
    assert tpg.sum() == -(-b.kv_lens // 16).sum() * 2
    # equal estimated time: no share above the ideal average of whole blocks by more than
    # one step group, one fold and its two cut charges
    whole = (STEP_GROUP * -(-(-(-b.kv_lens // 16)) // STEP_GROUP) + FOLD_COST).sum() * 2
    cpg = cost_per_group(items)
    assert cpg.max() <= -(-whole // 256) + STEP_GROUP + FOLD_COST + 2 * CUT_COST
    # a block is cut only at multiples of a step group (its last piece takes the rest)
    t = -(-(items[:, idx["tok_end"]] - items[:, idx["tok_begin"]]) // 16)
    not_last = items[:, idx["tok_end"]] < items[:, idx["kv_len"]]
    assert (t[not_last] % STEP_GROUP == 0).all()
    # a share cuts at most its first and last segment out of a longer row block
    g = items[:, idx["group"]]
    for gg in range(256):
        sel = np.where(g == gg)[0]
        inner = sel[1:-1]
        assert (items[inner, idx["num_splits"]] == 1).all()


def test_odd_half_kv_heads_get_smaller_shares():
    # d 128 fp16 with 2 kv heads: a token row is 512 bytes and kv head 1 reads its odd
    # 256-byte half, which streams slower; the plan gives its shares fewer tiles
    lens = np.full(8, 32768, np.int32)
    b = W.make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=128, page_size=256,
                     dtype="f16", num_pages=1100, poison=False)
    h = host_handle(Hq=12, Hkv=2, D=128, P=256, dtype="f16", max_pages=4096, num_cus=256)
    items = plan_batch(h, b)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    t = -(-(items[:, idx["tok_end"]] - items[:, idx["tok_begin"]]) // 16)
    whole = items[:, idx["num_splits"]] > 2  # interior pieces of the long blocks
    head = items[:, idx["kv_head"]]
    m0, m1 = np.median(t[whole & (head == 0)]), np.median(t[whole & (head == 1)])
    assert 1.15 < m0 / m1 < 1.30, (m0, m1)
    # with d 64 the rows are 256 bytes, each head's slice spans both halves: no tilt
    b2 = W.make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=64, page_size=256,
                      dtype="f16", num_pages=1100, poison=False)
    h2 = host_handle(Hq=12, Hkv=2, D=64, P=256, dtype="f16", max_pages=4096, num_cus=256,
                     whole_rows=-1)
    it2 = plan_batch(h2, b2)
    t2 = -(-(it2[:, idx["tok_end"]] - it2[:, idx["tok_begin"]]) // 16)
    w2 = it2[:, idx["num_splits"]] > 2
    hd2 = it2[:, idx["kv_head"]]
    assert np.median(t2[w2 & (hd2 == 0)]) == np.median(t2[w2 & (hd2 == 1)])


def test_decode_batch_of_equal_histories_is_not_split():
    b = W.saturated_decode()
    h = host_handle(num_cus=256, whole_rows=-1)
    items = plan_batch(h, b)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    assert (items[:, idx["num_splits"]] == 1).all()
    assert len(items) == 256 and (tiles_per_group(items) == 19).all()


def test_whole_rows_only_where_they_apply():
    """Decode-only steps with Hkv * D = 128, Hq <= 16 and a 16-bit type take whole-row
    blocks (all query heads of a request, every kv head's slice of each token row); steps
    with a prefill chunk, fp32, wider rows, more heads, or whole_rows = -1 do not."""
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    b = W.saturated_decode()
    items = plan_batch(host_handle(num_cus=256, whole_rows=1), b)
    assert (items[:, idx["kv_head"]] == -1).all() and (items[:, idx["num_rows"]] == 14).all()
    check_coverage(items, b)
    assert (plan_batch(host_handle(num_cus=256, whole_rows=-1), b)[:, idx["kv_head"]] >= 0).all()
    # by default only with a query row per compute unit: 128 requests on 256 units do not,
    # on 128 units they do
    assert (plan_batch(host_handle(num_cus=256), b)[:, idx["kv_head"]] >= 0).all()
    assert (plan_batch(host_handle(num_cus=128), b)[:, idx["kv_head"]] == -1).all()
    r = W.make_batch([40, 300, 17], [5, 1, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                     page_size=16)
    assert (plan_batch(host_handle(whole_rows=1), r)[:, idx["kv_head"]] >= 0).all()  # prefill rows
    # the default and -1 plan such shapes per kv head
    for kw, shape in ((dict(dtype="f32"), dict(dtype="f32")),                    # fp32
                      (dict(D=128), dict(head_dim=128)),                         # 2 x 128 wide
                      (dict(Hq=32), dict(num_qo_heads=32))):                     # 32 heads
        bb = W.make_batch([40, 300, 17], **{**dict(num_qo_heads=14, num_kv_heads=2, head_dim=64,
                                                   page_size=16), **shape})
        for wr in (0, -1):
            it = plan_batch(host_handle(whole_rows=wr, num_cus=2, **kw), bb)
            assert (it[:, idx["kv_head"]] >= 0).all(), kw
            check_coverage(it, bb)
    bb = W.make_batch([40, 300], num_qo_heads=8, num_kv_heads=1, head_dim=128, page_size=16)
    assert (plan_batch(host_handle(Hq=8, Hkv=1, D=128, num_cus=2), bb)[:, idx["kv_head"]] == 0).all()
    _expect(fl.FL_ERR_INVALID_ARG, host_handle, whole_rows=2)


@pytest.mark.parametrize("kw,why", [
    (dict(dtype="f32"), "fp32"),
    (dict(D=128), "head_dim"),
    (dict(Hq=32), "16 query heads"),
    (dict(Hq=8, Hkv=1, D=128), "one kv head"),
    (dict(Hq=16, Hkv=4, D=64), "head_dim"),
])
def test_whole_rows_forced_on_a_shape_that_cannot_take_them_is_refused(kw, why):
    """whole_rows = 1 asks for whole-row blocks on every decode step: a shape that can never
    take them is refused at create instead of silently planned per kv head."""
    msg = _expect(fl.FL_ERR_UNSUPPORTED, host_handle, whole_rows=1, **kw)
    assert "whole_rows" in msg and why in msg, msg
    host_handle(whole_rows=0, **kw)
    host_handle(whole_rows=-1, **kw)


def test_forced_splits_are_capped_by_tiles():
    b = W.tiny_decode()
    h = host_handle()
    items = plan_batch(h, b, num_splits=1000)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    for it in items:
        assert it[idx["num_splits"]] == -(-int(b.kv_lens[it[idx["request"]]]) // 16)


def _expect(status, fn, *a, **kw):
    with pytest.raises(fl.FlError) as e:
        fn(*a, **kw)
    assert e.value.status == status, str(e.value)
    return str(e.value)


def test_plan_rejects_bad_metadata_with_codes():
    b = W.tiny_decode()
    h = host_handle()
    good = dict(qo_indptr=b.qo_indptr, kv_indptr=b.kv_indptr, kv_indices=b.kv_indices,
                last_page_len=b.last_page_len, num_pages=b.num_pages)

    def plan(**kw):
        a = {**good, **kw}
        h.plan(a["qo_indptr"], a["kv_indptr"], a["kv_indices"], a["last_page_len"], a["num_pages"])

    bad = b.kv_indices.copy(); bad[5] = b.num_pages
    assert "kv_indices" in _expect(fl.FL_ERR_INVALID_ARG, plan, kv_indices=bad)
    bad = b.kv_indices.copy(); bad[0] = -1
    _expect(fl.FL_ERR_INVALID_ARG, plan, kv_indices=bad)
    last = b.last_page_len.copy(); last[2] = 0
    assert "last_page_len" in _expect(fl.FL_ERR_INVALID_ARG, plan, last_page_len=last)
    last[2] = 17
    _expect(fl.FL_ERR_INVALID_ARG, plan, last_page_len=last)
    kvp = b.kv_indptr.copy(); kvp[2] = kvp[1]                    # a request with no pages
    _expect(fl.FL_ERR_INVALID_ARG, plan, kv_indptr=kvp)
    kvp = b.kv_indptr.copy(); kvp[0] = 1
    _expect(fl.FL_ERR_INVALID_ARG, plan, kv_indptr=kvp)
    qo = np.array([0, 1, 2, 1, 2], np.int32)                      # decreasing
    _expect(fl.FL_ERR_INVALID_ARG, plan, qo_indptr=qo)
    qo = np.array([0, 1, 3, 4, 5], np.int32)                      # 2 rows on a 17... fine
    plan(qo_indptr=qo)
    qo = np.array([0, 2, 3, 4, 5], np.int32)                      # 2 causal rows on 1 token
    assert "causal" in _expect(fl.FL_ERR_INVALID_ARG, plan, qo_indptr=qo)
    _expect(fl.FL_ERR_INVALID_ARG, plan, num_pages=0)
    # a failed plan leaves the handle un-planned
    assert "no plan" in _expect(fl.FL_ERR_NOT_PLANNED, h.info)
    with pytest.raises(fl.FlError):
        h.work_items()


def test_capacity_limits():
    b = W.tiny_decode()
    h = host_handle(max_batch=3)
    _expect(fl.FL_ERR_CAPACITY, plan_batch, h, b)
    h = host_handle(max_rows=3)
    _expect(fl.FL_ERR_CAPACITY, plan_batch, h, b)
    h = host_handle(max_pages=20)
    _expect(fl.FL_ERR_CAPACITY, plan_batch, h, b)


def test_empty_batch_plans_to_nothing():
    h = host_handle()
    h.plan(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 1)
    assert h.info()[:2] == (0, 0)


def test_create_rejects_unsupported_configs():
    for kw in (dict(D=96), dict(D=32), dict(P=8), dict(P=512), dict(P=48)):
        _expect(fl.FL_ERR_UNSUPPORTED, host_handle, **kw)
    _expect(fl.FL_ERR_INVALID_ARG, host_handle, Hq=14, Hkv=4)
    cfg = fl.make_config(14, 2, 64, 16, "bf16", 8, 8, 64)
    cfg.dtype = 7
    _expect(fl.FL_ERR_UNSUPPORTED, fl.fl_paged_attn_create, cfg, -1)
    # flattened rows must stay below 2^32 / G for the kernels' division by G
    _expect(fl.FL_ERR_UNSUPPORTED, host_handle, Hq=128, Hkv=1, max_rows=(1 << 18))
    host_handle(Hq=128, Hkv=1, max_rows=(1 << 18) - 1)


def test_run_needs_a_device_handle_and_a_plan():
    h = host_handle()
    msg = _expect(fl.FL_ERR_UNSUPPORTED, fl.fl_paged_attn_run, h.handle, 16, 16, 16, 16)
    assert "host-only" in msg


# ---------------------------------------------------------------------------------------
# KV append destinations
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_append_slots_point_where_the_generator_put_the_new_tokens(name):
    """The generator scattered every request's whole history into the pool; the slot the
    plan gives each query row must hold exactly that row's token (compared byte for byte
    with the newest tokens cut from the dense history)."""
    b = W.WORKLOADS[name](keep_dense=True)
    st = W.append_step(b)
    h = host_handle(Hq=b.num_qo_heads, Hkv=b.num_kv_heads, D=b.head_dim, P=b.page_size,
                    dtype=b.dtype, max_batch=b.batch_size, max_rows=b.rows,
                    max_pages=int(b.kv_indptr[-1]))
    plan_batch(h, b)
    slots = h.append_slots()
    assert slots.shape == (b.rows,)
    assert len(np.unique(slots)) == b.rows
    flat_k = b.k_pool.reshape(b.num_pages * b.page_size, b.num_kv_heads, b.head_dim)
    flat_v = b.v_pool.reshape(b.num_pages * b.page_size, b.num_kv_heads, b.head_dim)
    assert np.array_equal(flat_k[slots].view(np.uint8), st.k_new.view(np.uint8))
    assert np.array_equal(flat_v[slots].view(np.uint8), st.v_new.view(np.uint8))


def test_append_slots_worked_out_by_hand():
    """r0: pages [2, 0], 17 tokens -> token 16 at page 0 slot 0; r1: page [3], 16 tokens ->
    token 15 at page 3 slot 15; r2: page [1], 5 tokens, 3 new rows -> page 1 slots 2, 3, 4."""
    h = host_handle(Hq=2, Hkv=1)
    h.plan(np.array([0, 1, 2, 5]), np.array([0, 2, 3, 4]), np.array([2, 0, 3, 1]),
           np.array([1, 16, 5]), 4)
    assert h.append_slots().tolist() == [0 * 16 + 0, 3 * 16 + 15, 1 * 16 + 2, 1 * 16 + 3, 1 * 16 + 4]


def test_append_slots_refused_but_attention_planned():
    h = host_handle(Hq=2, Hkv=1)
    # non-causal: 3 query rows on a 2-token history is fine for attention, not for append
    h.plan(np.array([0, 3]), np.array([0, 1]), np.array([0]), np.array([2]), 1, causal=False)
    assert h.info()[0] > 0
    msg = _expect(fl.FL_ERR_INVALID_ARG, h.append_slots)
    assert "no slot" in msg
    # two requests whose newest token sits in one shared page slot
    h.plan(None, np.array([0, 1, 2]), np.array([5, 5]), np.array([7, 7]), 8)
    assert h.info()[0] > 0
    msg = _expect(fl.FL_ERR_INVALID_ARG, h.append_slots)
    assert "page 5 slot 6" in msg
    # requests sharing a page but appending to their own pages are fine
    h.plan(None, np.array([0, 2, 4]), np.array([5, 1, 5, 2]), np.array([3, 3]), 8)
    assert h.append_slots().tolist() == [1 * 16 + 2, 2 * 16 + 2]


def test_append_on_empty_plan_and_host_handle():
    h = host_handle()
    _expect(fl.FL_ERR_NOT_PLANNED, h.append_slots)
    h.plan(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 1)
    assert h.append_slots().size == 0
    msg = _expect(fl.FL_ERR_UNSUPPORTED, fl.fl_paged_kv_append, h.handle, 16, 16, 16, 16)
    assert "host-only" in msg
    msg = _expect(fl.FL_ERR_UNSUPPORTED, fl.fl_paged_kv_append_rope, h.handle, 16, 16, 16, 16, 16, 1e4)
    assert "host-only" in msg
    for theta in (0.0, -1.0, float("inf"), float("nan")):
        _expect(fl.FL_ERR_INVALID_ARG, fl.fl_paged_kv_append_rope, h.handle, 16, 16, 16, 16, 16, theta)


def test_neighbouring_shares_share_an_xcd():
    """Workgroups b and b + 8 run on one XCD: the plan hands runs of consecutive shares (neighbouring
    row blocks, which for a prefill chunk read the same K/V) to one XCD, in equal numbers."""
    for b, dtype in ((W.ragged_mixed_step(), "bf16"), (W.ragged_mixed_step(), "f32")):
        # bf16: the chunk in prefill quads (workgroups 0 .. Gp-1) and the decode blocks (the
        # rest), each path in its own runs; fp32: one sequence of 16-row blocks
        h = host_handle(num_cus=256, dtype=dtype)
        items = plan_batch(h, b)
        idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
        g = items[:, idx["group"]]
        first = np.r_[True, g[1:] != g[:-1]]
        order = g[first]                                  # workgroups in share order
        n = h.info()[1]
        assert sorted(order.tolist()) == list(range(n))   # a permutation of the workgroups
        prefill = (b.qo_lens[items[first, idx["request"]]] > 1) & (dtype != "f32")
        gp = int(prefill.sum())
        assert (order[prefill] < gp).all() and (order[~prefill] >= gp).all()
        for part in (order[prefill], order[~prefill]):
            if part.size == 0:
                continue
            xcd = part % 8
            assert (np.diff(xcd) != 0).sum() <= 7        # one contiguous run per XCD
            counts = np.bincount(xcd, minlength=8)
            assert counts.max() - counts.min() <= 1


# ---- launch shape: one launch per kind of step -----------------------------------------------
def _meta(kv_lens, qo_lens, P, rng):
    """Page-table metadata for the given lengths, pages drawn at random from a large pool."""
    kv_lens = np.asarray(kv_lens, np.int64)
    pages = -(-kv_lens // P)
    kv_indptr = np.concatenate([[0], np.cumsum(pages)]).astype(np.int32)
    pool = int(kv_indptr[-1]) + 64
    kv_indices = rng.permutation(pool)[:kv_indptr[-1]].astype(np.int32)
    last = (kv_lens - (pages - 1) * P).astype(np.int32)
    qo_indptr = np.concatenate([[0], np.cumsum(qo_lens)]).astype(np.int32)
    return qo_indptr, kv_indptr, kv_indices, last, pool


def _serving_lengths(steps, seed, start=96, cap=160, max_prompt=4096):
    """Decode steps of a serving loop: every request grows by one token per step, some
    finish, new ones join with prompts of assorted lengths."""
    rng = np.random.default_rng(seed)
    live = list(rng.integers(1, max_prompt, size=start))
    for _ in range(steps):
        yield list(live)
        live = [k + 1 for k in live]
        for _ in range(int(rng.integers(0, 4))):           # finish
            if live:
                live.pop(int(rng.integers(len(live))))
        for _ in range(int(rng.integers(0, 5))):           # join
            if len(live) < cap:
                live.insert(int(rng.integers(len(live) + 1)), int(rng.integers(1, max_prompt)))


@pytest.mark.parametrize("shape", [
    dict(Hq=14, Hkv=2, D=64, P=16, dtype="bf16"),
    dict(Hq=12, Hkv=2, D=128, P=256, dtype="f16"),
    dict(Hq=14, Hkv=2, D=64, P=16, dtype="bf16", whole_rows=1),
    dict(Hq=12, Hkv=2, D=128, P=64, dtype="f32"),
])
def test_every_plan_of_a_kind_launches_the_same(shape):
    """64 decode steps of a serving loop (histories grow, requests finish and join) give one
    launch class and one grid; the workgroups past each plan's busy count are idle (no work
    item names them). A step with a prefill chunk has its own class where its launch differs
    (two workgroups per compute unit at head_dim 64 in a 16-bit type) and never the
    one-launch append class."""
    P = shape["P"]
    wr = shape.get("whole_rows", 0)
    h = host_handle(Hq=shape["Hq"], Hkv=shape["Hkv"], D=shape["D"], P=P, dtype=shape["dtype"],
                    max_batch=256, max_rows=2048, max_pages=1 << 20, num_cus=256, whole_rows=wr)
    rng = np.random.default_rng(5)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    seen = set()
    batches = 0
    for kv in _serving_lengths(64, seed=11):
        qo, kp, ki, last, pool = _meta(kv, [1] * len(kv), P, rng)
        h.plan(qo, kp, ki, last, pool)
        cls, fcls, grid, busy = h.launch()
        seen.add((cls, fcls, grid))
        assert grid == 256 and 1 <= busy <= grid
        groups = h.work_items()[:, idx["group"]]
        assert set(groups.tolist()) == set(range(busy))      # the rest of the grid is idle
        batches += 1
    assert batches == 64 and len(seen) == 1, seen
    (cls, fcls, grid), = seen
    assert (fcls != 0) == (shape["dtype"] != "f32")
    # an empty step launches the same way (every workgroup idle)
    h.plan(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 1)
    if not wr:
        assert h.launch()[:3] == (cls, fcls, grid) and h.launch()[3] == 0
    # mixed steps: chunks of 2..600 rows on top of the decodes
    mixed = set()
    for s, kv in enumerate(_serving_lengths(8, seed=12)):
        ql = [1] * len(kv)
        for j in range(1 + s % 3):
            ql[j] = min(kv[j], 2 + 73 * (s + j))
        qo, kp, ki, last, pool = _meta(kv, ql, P, rng)
        h.plan(qo, kp, ki, last, pool)
        c, f, g, b = h.launch()
        mixed.add((c, f, g))
        assert f == 0 and 1 <= b <= g
    assert len(mixed) == 1
    (c, f, g), = mixed
    two_per_cu = shape["D"] == 64 and shape["dtype"] != "f32"
    assert g == (512 if two_per_cu else 256)
    assert (c == cls) == (not two_per_cu and not wr)


def test_decode_class_changes_only_where_whole_rows_switch_on():
    """With the default whole_rows = 0 a decode step takes whole-row blocks from one query row
    per compute unit on: the class switches there and nowhere else."""
    h = host_handle(max_batch=512, max_rows=512, num_cus=256)
    rng = np.random.default_rng(6)
    classes = {}
    for n in (1, 100, 255, 256, 300, 512):
        qo, kp, ki, last, pool = _meta([300] * n, [1] * n, 16, rng)
        h.plan(qo, kp, ki, last, pool)
        classes[n] = h.launch()[0]
    assert classes[1] == classes[100] == classes[255]
    assert classes[256] == classes[300] == classes[512] != classes[255]


@pytest.mark.parametrize("Hq,Hkv", [(32, 1), (17, 1), (16, 1), (12, 2)])
def test_decode_rows_of_more_than_16_heads_run_as_units_and_never_fused(Hq, Hkv):
    """A decode row of more than 16 query heads per kv head spans two 16-row blocks, which
    run as a prefill unit: such a handle's decode steps never take the one-launch append,
    whose kernel has no unit path. At head_dim 128 decode and prefill steps share one
    launch class."""
    G = Hq // Hkv
    h = host_handle(Hq=Hq, Hkv=Hkv, D=128, P=16, dtype="f16", max_rows=256)
    idx = {n: i for i, n in enumerate(fl.WORK_ITEM_FIELDS)}
    rng = np.random.default_rng(14)
    qo, kp, ki, last, pool = _meta([100, 40, 300], [1, 1, 1], 16, rng)
    h.plan(qo, kp, ki, last, pool)
    items = h.work_items()
    assert (items[:, idx["row_begin"]] > 0).any() == (G > 16)  # a second block per row
    cls, fcls, grid, busy = h.launch()
    assert (fcls == 0) == (G > 16)
    qo, kp, ki, last, pool = _meta([100, 40, 300], [1, 9, 1], 16, rng)
    h.plan(qo, kp, ki, last, pool)
    c2, f2, g2, _ = h.launch()
    assert f2 == 0 and g2 == grid and c2 == cls


def test_forced_splits_launch_one_workgroup_per_piece():
    b = W.tiny_decode()
    h = host_handle()
    plan_batch(h, b, num_splits=3)
    cls, fcls, grid, busy = h.launch()
    assert grid == busy == h.info()[1] == len(h.work_items())


def test_allocation_free_run_refuses_plans_beyond_its_array():
    """The allocation-free run checks the plan's needs against its fixed device array before
    any HIP call: 16384 forced pieces of 6 rows need ~50 MB of partial rows."""
    lens = [8192] * 16
    b = W.make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=128, page_size=256, dtype="f16",
                     num_pages=16 * 32, seed=1)
    h = host_handle(Hq=12, Hkv=2, D=128, P=256, dtype="f16", max_batch=16, max_rows=16,
                    max_pages=1 << 12, num_cus=256)
    plan_batch(h, b, num_splits=512)
    assert h.info()[1] == 16384
    msg = _expect(fl.FL_ERR_CAPACITY, fl.fl_paged_attn_run_noalloc, h.handle, 256, 256, 256, 256)
    assert "scratch" in msg and "16777216" in msg, msg
    # NULL and misaligned pointers are refused first, also without a GPU
    _expect(fl.FL_ERR_INVALID_ARG, fl.fl_paged_attn_run_noalloc, h.handle, 0, 256, 256, 256)
    _expect(fl.FL_ERR_INVALID_ARG, fl.fl_paged_attn_run_noalloc, h.handle, 258, 256, 256, 256)
    h2 = host_handle()
    _expect(fl.FL_ERR_NOT_PLANNED, fl.fl_paged_attn_run_noalloc, h2.handle, 256, 256, 256, 256)
