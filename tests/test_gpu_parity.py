"""GPU parity: the HIP path against the CPU oracle, through the C interface.

Tolerances (max-abs against the unrounded fp64 oracle): 4e-3 for bf16/fp16 outputs and
1e-5 for fp32; where the output type's own half-ulp at a cell's magnitude is larger than
4e-3 (bf16 |o| >= 2), half an ulp plus 1e-4 (see gpu_helpers.tolerance). Page-table indexing is checked bit-exactly with needle keys, and page
permutation, repeated runs and single-key histories give bit-identical results.
Unused slots and pages of every pool hold NaN.
"""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_plan_amd as fl
import workloads as W
from gpu_helpers import DeviceBatch, announce, compare, to_host_bits, to_host_f64

pytestmark = pytest.mark.gpu


def _check(b, num_splits=0, what="", **cfg_kw):
    announce(f"{what or b.name}: dtype={b.dtype} B={b.batch_size} rows={b.rows} "
             f"D={b.head_dim} P={b.page_size} G={b.group} splits={num_splits}")
    ref_out, ref_lse = oracle.attention(b)
    d = DeviceBatch(b, num_splits=num_splits, **cfg_kw)
    out, lse = d.run()
    compare(b, out, lse, ref_out, ref_lse, what or b.name)
    return d, ref_out


# ---- the five workloads at full size, planner defaults (the benchmark's launch setup) ----
def test_tiny_decode():
    _check(W.tiny_decode())


def test_saturated_decode_full():
    _check(W.saturated_decode())      # one block per kv head (128 requests < 256 compute units)


def test_saturated_decode_full_whole_rows():
    _check(W.saturated_decode(), what="saturated_decode in whole rows", whole_rows=1)


def test_tiny_decode_whole_rows():
    _check(W.tiny_decode(), what="tiny_decode in whole rows", whole_rows=1)


def test_decode_512_requests_whole_rows_by_default():
    """A decode batch with a request per compute unit takes whole rows without asking."""
    b = W.make_batch([300] * 512, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype="bf16", num_pages=512 * 19 + 40, seed=9)
    d, _ = _check(b, what="512 x 300 decode")
    assert (d.h.work_items()[:, fl.WORK_ITEM_FIELDS.index("kv_head")] == -1).all()


def test_mixed_length_decode_full():
    _check(W.mixed_length_decode())


def test_long_context_skew_full():
    _check(W.long_context_skew())


def test_ragged_mixed_step_full():
    _check(W.ragged_mixed_step())


def test_multi_chunk_step_full():
    """Four 128-row prefill chunks on 256..2048 cached tokens plus 124 decode rows in one call
    (the shape bench.py times)."""
    b = W.multi_chunk_step()
    assert (b.qo_lens[:4] == 128).all() and (b.qo_lens[4:] == 1).all() and b.batch_size == 128
    _check(b)


# ---- forced slice counts: the merge path ------------------------------------------------
@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
def test_split_counts(splits):
    b = W.make_batch([1, 17, 100, 300, 777], [1, 1, 1, 40, 1], num_qo_heads=14, num_kv_heads=2,
                     head_dim=64, page_size=16, dtype="bf16", seed=21, num_pages=120)
    _check(b, num_splits=splits, what=f"splits{splits}")


@pytest.mark.parametrize("splits", [1, 2, 3, 7, 1000])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_split_counts_whole_rows(splits, dtype):
    """Decode-only batch in whole-row blocks: cut pieces write 128-wide partial rows and the
    merge stores each head's own half."""
    b = W.make_batch([1, 17, 100, 300, 777, 64], num_qo_heads=12 if dtype == "f16" else 14,
                     num_kv_heads=2, head_dim=64, page_size=16, dtype=dtype, seed=22, num_pages=90)
    _check(b, num_splits=splits, what=f"whole-rows splits{splits} {dtype}", whole_rows=1)


# ---- dtype / head_dim / page_size / group coverage ----------------------------------------
VARIANTS = [
    dict(dtype="bf16", D=64, P=16, Hq=14, Hkv=2),
    dict(dtype="bf16", D=128, P=64, Hq=12, Hkv=2),
    dict(dtype="f16", D=64, P=32, Hq=14, Hkv=2),
    dict(dtype="f16", D=128, P=256, Hq=12, Hkv=2),
    dict(dtype="f32", D=64, P=16, Hq=14, Hkv=2),
    dict(dtype="f32", D=128, P=256, Hq=12, Hkv=2),
    dict(dtype="bf16", D=64, P=16, Hq=2, Hkv=2),      # G = 1
    dict(dtype="f16", D=128, P=128, Hq=16, Hkv=1),    # G = 16: a full 16-row block
    dict(dtype="bf16", D=64, P=16, Hq=32, Hkv=1),     # G = 32: two row blocks per decode row
    dict(dtype="f16", D=128, P=32, Hq=24, Hkv=1),     # G = 24: a full block and one of 8 rows
    dict(dtype="f32", D=64, P=64, Hq=8, Hkv=8),       # MHA
]


@pytest.mark.parametrize("v", VARIANTS, ids=lambda v: f"{v['dtype']}-D{v['D']}-P{v['P']}-G{v['Hq']//v['Hkv']}")
@pytest.mark.parametrize("ragged", [False, True])
def test_variants(v, ragged):
    kv = [1, 15, 16, 17, 255, 256, 257, 1000]
    qo = [1, 1, 9, 1, 1, 100, 1, 33] if ragged else None
    P = v["P"]
    b = W.make_batch(kv, qo, num_qo_heads=v["Hq"], num_kv_heads=v["Hkv"], head_dim=v["D"],
                     page_size=P, dtype=v["dtype"], seed=31,
                     num_pages=sum(-(-k // P) for k in kv) + 7)
    _check(b, what=f"variant-{v}-ragged{ragged}")


def _random_case(seed):
    """A seeded random configuration: dtype, head_dim, page size, heads, a batch of lengths
    mixing short, tile- and page-aligned and long histories, some prefill chunks, the mask
    and a forced slice count."""
    r = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f16", "f32"][r.integers(3)]
    D = [64, 128][r.integers(2)]
    P = [16, 32, 64, 128, 256][r.integers(5)]
    Hq, Hkv = [(14, 2), (12, 2), (8, 1), (4, 4), (32, 4), (6, 3), (24, 1)][r.integers(7)]
    B = int(r.integers(1, 25))
    kinds = r.integers(4, size=B)
    kv = np.where(kinds == 0, r.integers(1, 40, size=B),
         np.where(kinds == 1, 16 * r.integers(1, 40, size=B),
         np.where(kinds == 2, P * r.integers(1, 6, size=B), r.integers(40, 3000, size=B))))
    qo = np.where(r.random(B) < 0.25, np.minimum(kv, r.integers(2, 80, size=B)), 1)
    causal = bool(r.random() < 0.8)
    splits = int([0, 0, 0, 1, 2, 5][r.integers(6)])
    b = W.make_batch(kv.tolist(), qo.tolist(), num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     page_size=P, dtype=dtype, seed=seed, causal=causal,
                     num_pages=int(sum(-(-k // P) for k in kv)) + 3)
    return b, splits


@pytest.mark.parametrize("seed", range(40))
def test_random_configurations(seed):
    b, splits = _random_case(seed)
    _check(b, num_splits=splits, what=f"random-{seed}")


def _wide_case(seed):
    """A seeded configuration from a wider space than _random_case: head ratios 1-32 (17,
    20, 31 among them: a decode row's second 16-row block partly filled), up to 8 kv heads,
    histories up to 9000 tokens, prefill chunks up to 700 rows, requests without query rows,
    up to 50 forced slices per row block."""
    r = np.random.default_rng(50000 + seed)
    dtype = ["bf16", "f16", "f32"][r.integers(3)]
    D = [64, 128][r.integers(2)]
    P = [16, 32, 64, 128, 256][r.integers(5)]
    Hkv = [1, 2, 4, 8][r.integers(4)]
    G = [1, 2, 3, 4, 5, 6, 7, 8, 12, 14, 16, 17, 20, 24, 31, 32][r.integers(16)]
    B = int(r.integers(1, 41))
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
    b = W.make_batch(kv.tolist(), qo.tolist(), num_qo_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                     page_size=P, dtype=dtype, seed=seed, causal=causal,
                     num_pages=int(sum(-(-k // P) for k in kv)) + 5)
    return b, splits


# seeds of _wide_case chosen to span its corners (each plans within the handle's capacity)
WIDE_SEEDS = [341, 88, 590, 35, 475, 283, 105, 240, 346, 98, 294, 480, 577, 275, 249, 133]


@pytest.mark.parametrize("seed", WIDE_SEEDS)
def test_wide_configurations(seed):
    b, splits = _wide_case(seed)
    _check(b, num_splits=splits, what=f"wide-{seed}")


def test_fp32_long_context_skew_full():
    """The long-context skew batch at full size in fp32 (8 x 32768 + 56 x 512 cached tokens,
    12/2 heads, d 128, 256-slot pages): the most pieces per row block and the deepest
    log-sum-exp merge, against the 1e-5 bar."""
    b = W.long_context_skew(dtype="f32")
    d, _ = _check(b, what="f32-long-context-skew")
    assert d.h.info()[2] >= 8  # the long histories are cut into many pieces and merged


def test_fp32_saturated_decode():
    _check(W.saturated_decode(dtype="f32"), what="f32-saturated")


def test_non_causal_prefill():
    b = W.make_batch([60, 9, 300], [7, 3, 20], num_qo_heads=4, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="f32", causal=False, seed=3)
    _check(b, what="non-causal")


def test_request_with_no_query_rows():
    b = W.make_batch([40, 70, 5], [3, 0, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="bf16", seed=4)
    _check(b, what="zero-row request")


def test_custom_scale():
    b = W.make_batch([33, 200], num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype="bf16", seed=5, sm_scale=0.05)
    _check(b, what="scale 0.05")


# ---- bit-exact facts ----------------------------------------------------------------------
def _needle_batch(kv_lens, qo_lens, P, dtype):
    b = W.make_batch(kv_lens, qo_lens, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=P,
                     dtype=dtype, seed=11, num_pages=sum(-(-k // P) for k in kv_lens) + 9)
    zero = W.to_storage(np.zeros(1, np.float32), dtype)[0]
    for r, kl in enumerate(kv_lens):
        pages = b.kv_indices[b.kv_indptr[r]:b.kv_indptr[r + 1]]
        for t in range(kl):
            pg, sl = pages[t // P], t % P
            b.k_pool[pg, sl] = zero
            row = np.zeros((2, 64), np.float32)
            row[:, 0] = r + 1
            row[:, 1] = t % 256
            row[:, 2] = t // 256
            row[:, 3] = np.array([1, 2])
            row[:, 4:] = ((np.arange(60) * 7 + t + 3 * r) % 251) - 125
            b.v_pool[pg, sl] = W.to_storage(row, dtype)
    b.q[:] = zero
    return b


def _plant(b, r, t, rows=None):
    P = b.page_size
    pg = b.kv_indices[b.kv_indptr[r] + t // P]
    b.k_pool[pg, t % P, :, 0] = W.to_storage(np.array([256.0], np.float32), b.dtype)[0]
    q0, q1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
    sel = slice(q0, q1) if rows is None else rows
    b.q[sel, :, 0] = W.to_storage(np.array([32.0], np.float32), b.dtype)[0]


# whole-row blocks are 16-bit only (create refuses whole_rows = 1 for fp32)
@pytest.mark.parametrize("dtype,whole_rows", [("bf16", 1), ("bf16", -1), ("f16", 1), ("f16", -1),
                                              ("f32", -1)])
@pytest.mark.parametrize("P", [16, 64, 256])
@pytest.mark.parametrize("splits", [0, 1, 4])
def test_needles_bit_exact(dtype, whole_rows, P, splits):
    kv = [1, P, P + 1, 3 * P - 1, 300, 1000]
    spots = [0, P - 1, P, 3 * P - 2, 299, 517]
    b = _needle_batch(kv, None, P, dtype)
    for r, t in enumerate(spots):
        _plant(b, r, t)
    announce(f"needles dtype={dtype} P={P} splits={splits} whole_rows={whole_rows}")
    d = DeviceBatch(b, num_splits=splits, whole_rows=whole_rows)
    out, _ = d.run()
    got = to_host_bits(out, dtype)
    for r, t in enumerate(spots):
        pg = b.kv_indices[b.kv_indptr[r] + t // P]
        for h in range(14):
            want = b.v_pool[pg, t % P, h // 7]
            assert np.array_equal(got[r, h].view(np.uint8), np.ascontiguousarray(want).view(np.uint8)), (r, t, h)


def test_causal_limit_needles_bit_exact():
    P = 16
    b = _needle_batch([70, 300], [20, 1], P, "bf16")
    i = 9
    lim = 70 - 20 + i
    pg = b.kv_indices[lim // P]
    b.k_pool[pg, lim % P, :, 0] = W.to_storage(np.array([256.0], np.float32), "bf16")[0]
    b.q[i, :, 0] = W.to_storage(np.array([32.0], np.float32), "bf16")[0]
    # row i+1 plants nothing but sees the needle too; rows < i do not see it
    announce("causal-limit needles")
    ref, _ = oracle.attention(b)
    d = DeviceBatch(b)
    out, lse = d.run()
    got = to_host_bits(out, "bf16")
    assert np.array_equal(got[i, 0], b.v_pool[pg, lim % P, 0])
    compare(b, out, lse, ref, oracle.attention(b)[1], "causal-limit needles")


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_key_history_is_exact(dtype):
    b = W.make_batch([1] * 5, num_qo_heads=12, num_kv_heads=2, head_dim=128, page_size=16,
                     dtype=dtype, seed=6, keep_dense=True)
    announce(f"single-key {dtype}")
    d = DeviceBatch(b)
    out, _ = d.run()
    got = to_host_bits(out, dtype)
    for r in range(5):
        for h in range(12):
            assert np.array_equal(np.ascontiguousarray(got[r, h]).view(np.uint8),
                                  np.ascontiguousarray(b.dense_v[r][0, h // 6]).view(np.uint8))


def test_page_permutation_bit_identical():
    b = W.mixed_length_decode()
    b2 = W.relabel_pages(b, W.rng_for(77, 0, 0).permutation(b.num_pages))
    announce("page permutation")
    o1, l1 = DeviceBatch(b).run()
    o2, l2 = DeviceBatch(b2).run()
    assert np.array_equal(to_host_bits(o1, "f16").view(np.uint16), to_host_bits(o2, "f16").view(np.uint16))
    assert np.array_equal(l1.cpu().numpy().view(np.uint32), l2.cpu().numpy().view(np.uint32))


@pytest.mark.parametrize("name", ["ragged_mixed_step", "mixed_length_decode", "multi_chunk_step"])
def test_repeated_runs_bit_identical(name):
    """Outputs and lse, bit for bit, whichever workgroup happens to merge a cut block (the
    merge sums the pieces in split order whatever its layout); unrelated device work between
    the runs shifts which piece finishes last."""
    import torch
    b = W.WORKLOADS[name]()
    announce(f"determinism: {name}")
    d = DeviceBatch(b)
    out, lse = d.run()
    o1, l1 = to_host_bits(out, b.dtype).copy(), lse.cpu().numpy().view(np.uint32).copy()
    for i in range(4):
        x = torch.randn((1 + i) << 18, device="cuda:0")
        float(x.sum())
        out, lse = d.run()
        assert np.array_equal(to_host_bits(out, b.dtype), o1), f"run {i}"
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), l1), f"run {i} lse"


def test_page_size_relayout_within_tolerance():
    outs = []
    for P in (16, 64, 256):
        kv = [1, 17, 100, 300, 513]
        b = W.make_batch(kv, [1, 1, 1, 9, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                         page_size=P, dtype="bf16", seed=8, num_pages=sum(-(-k // P) for k in kv) + 3)
        announce(f"relayout P={P}")
        d, ref = _check(b, what=f"relayout P{P}")
        outs.append(to_host_f64(d.out))
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 8e-3


# ---- one plan, many layers; re-planning ---------------------------------------------------
def test_one_plan_many_layers_and_replanning():
    import dataclasses

    import torch
    b1 = W.tiny_decode(seed=1)
    # a second layer: same page table, different pool contents (K and V swapped)
    b2 = dataclasses.replace(b1, k_pool=b1.v_pool.copy(), v_pool=b1.k_pool.copy())
    announce("layers + replanning")
    d1 = DeviceBatch(b1)
    d2 = DeviceBatch(b2, handle=d1.h)
    r1, r2 = oracle.attention(b1), oracle.attention(b2)
    for _ in range(3):
        d1.plan(); o, l = d1.run(); compare(b1, o, l, *r1, "layer A")
        o, l = d2.run(); compare(b2, o, l, *r2, "layer B under the same plan")
    b3 = W.saturated_decode(seed=3)
    d3 = DeviceBatch(b3, handle=fl.PagedAttention(
        fl.make_config(14, 2, 64, 16, "bf16", 256, 256, 8192), device=0))
    r3 = oracle.attention(b3)
    b4 = W.make_batch([5, 700, 40], num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                      dtype="bf16", seed=4, num_pages=60)
    d4 = DeviceBatch(b4, handle=d3.h)
    r4 = oracle.attention(b4)
    for _ in range(3):                            # alternate plans: staging buffers rotate
        d3.plan(); o, l = d3.run(); compare(b3, o, l, *r3, "plan 3")
        d4.plan(); o, l = d4.run(); compare(b4, o, l, *r4, "plan 4")
    torch.cuda.synchronize()


def test_empty_batch_run_is_noop():
    import torch
    h = fl.PagedAttention(fl.make_config(14, 2, 64, 16, "bf16", 4, 4, 16), device=0)
    h.plan(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32), 1)
    x = torch.zeros(16, device="cuda:0")
    h.run(x, x, x, x)
    torch.cuda.synchronize()


def test_run_errors():
    import torch
    h = fl.PagedAttention(fl.make_config(14, 2, 64, 16, "bf16", 4, 4, 64), device=0)
    x = torch.zeros(1024, device="cuda:0")
    with pytest.raises(fl.FlError) as e:
        h.run(x, x, x, x)
    assert e.value.status == fl.FL_ERR_NOT_PLANNED
    b = W.tiny_decode()
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages)
    with pytest.raises(fl.FlError) as e:
        fl.fl_paged_attn_run(h.handle, x.data_ptr() + 2, x.data_ptr(), x.data_ptr(), x.data_ptr())
    assert e.value.status == fl.FL_ERR_INVALID_ARG
    with pytest.raises(fl.FlError) as e:
        fl.fl_paged_attn_run(h.handle, 0, x.data_ptr(), x.data_ptr(), x.data_ptr())
    assert e.value.status == fl.FL_ERR_INVALID_ARG


def test_pool_beyond_4_gib():
    """One layer's pools of 40960 pages of 128 KB (5.4 GB each, fp16, d 128, page size 256):
    the requests' pages sit past byte offset 2^32, so every address must be formed in 64
    bits (attention, append and poisoning). Only the used pages are filled."""
    import torch
    P, Hkv, D, Hq, N = 256, 2, 128, 12, 40960
    kv = [300, 1000, 5000, 257]
    small = W.make_batch(kv, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D, page_size=P,
                         dtype="f16", seed=97, num_pages=sum(-(-k // P) for k in kv), keep_dense=True)
    # move the used pages to the far end of a large pool (ids N - n .. N - 1, shuffled)
    n_used = small.num_pages
    perm = (N - n_used) + W.rng_for(97, 0, 7).permutation(n_used)
    indices = perm[small.kv_indices].astype(np.int32)
    announce(f"pool beyond 4 GiB: {N} pages x {P * Hkv * D * 2} B, pages {indices.min()}..{indices.max()}")
    k = torch.full((N, P, Hkv, D), float("nan"), dtype=torch.float16, device="cuda:0")
    v = torch.full((N, P, Hkv, D), float("nan"), dtype=torch.float16, device="cuda:0")
    idx = torch.from_numpy(perm.astype(np.int64)).to("cuda:0")
    k.index_copy_(0, idx, torch.from_numpy(small.k_pool).to("cuda:0"))
    v.index_copy_(0, idx, torch.from_numpy(small.v_pool).to("cuda:0"))
    assert int(indices.max()) * P * Hkv * D * 2 > (1 << 32)
    # the oracle on the small pool with the original page ids: the same logical batch
    ref_out, ref_lse = oracle.attention(small)
    big = W.Batch(**{**small.__dict__, "kv_indices": indices, "num_pages": N})
    h = fl.PagedAttention(fl.make_config(Hq, Hkv, D, P, "f16", 8, 8, 64), device=0)
    h.plan(big.qo_indptr, big.kv_indptr, big.kv_indices, big.last_page_len, N)
    q = torch.from_numpy(small.q).to("cuda:0")
    out = torch.full(q.shape, float("nan"), dtype=torch.float16, device="cuda:0")
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda:0")
    h.run(q, k, v, out, lse)
    torch.cuda.synchronize()
    compare(small, out, lse, ref_out, ref_lse, "pool beyond 4 GiB")
    # append: the step's new rows written past 4 GiB, byte for byte
    st = W.append_step(small)
    k.index_copy_(0, idx, torch.from_numpy(st.k_before).to("cuda:0"))
    v.index_copy_(0, idx, torch.from_numpy(st.v_before).to("cuda:0"))
    kn = torch.from_numpy(st.k_new).to("cuda:0")
    vn = torch.from_numpy(st.v_new).to("cuda:0")
    h.append(kn, vn, k, v)
    torch.cuda.synchronize()
    got_k = k.index_select(0, idx).cpu().numpy()
    assert np.array_equal(got_k.view(np.uint16), small.k_pool.view(np.uint16))
    # poison the big pages of small pages 0..2: exactly those become NaN, in both pools
    fl.fl_paged_kv_poison("f16", P, Hkv, D, N, perm[:3].astype(np.int32), k.data_ptr(), v.data_ptr())
    torch.cuda.synchronize()
    assert torch.isnan(k.index_select(0, idx[:3]).float()).all()
    assert torch.isnan(v.index_select(0, idx[:3]).float()).all()
    rest = k.index_select(0, idx[3:]).cpu().numpy()
    assert np.array_equal(rest.view(np.uint16), small.k_pool[3:].view(np.uint16))
