"""Pins for the CPU oracle: facts fixed by mathematics or by independent library routines.

Each pin is chosen so that a plausible slip in the oracle fails at least one of them:
a wrong head mapping (GQA vs repeated MHA, SDPA with enable_gqa), a wrong page/slot index
(needles at page edges, page permutation, page-size relayout), a wrong causal alignment
(needles at and past the limit, SDPA with a bottom-right mask), a dropped max-subtraction
or normaliser (closed forms, lse = log n at q = 0), a wrong merge (split invariance).
All of these run on the CPU only.
"""
import dataclasses
import json
import math
import os

import numpy as np
import pytest
import torch
from scipy.special import expit, logsumexp

import oracle
import workloads as W

HERE = os.path.dirname(os.path.abspath(__file__))


def dense_f64(b, arr_list):
    return [W.storage_to_f32(a, b.dtype).astype(np.float64) for a in arr_list]


def sdpa_reference(b):
    """torch's scaled_dot_product_attention (CPU, float64) on the generator's dense tensors,
    taken before they were scattered into pages; GQA via enable_gqa, bottom-right causal mask
    passed explicitly."""
    q_all = W.storage_to_f32(b.q, b.dtype).astype(np.float64)
    ks, vs = dense_f64(b, b.dense_k), dense_f64(b, b.dense_v)
    out = np.zeros(q_all.shape, dtype=np.float64)
    lse = np.zeros(q_all.shape[:2], dtype=np.float64)
    for r in range(b.batch_size):
        q0, q1 = int(b.qo_indptr[r]), int(b.qo_indptr[r + 1])
        ql, kl = q1 - q0, int(b.kv_lens[r])
        if ql == 0:
            continue
        qt = torch.from_numpy(q_all[q0:q1]).permute(1, 0, 2).unsqueeze(0)   # [1, Hq, ql, D]
        kt = torch.from_numpy(ks[r]).permute(1, 0, 2).unsqueeze(0)          # [1, Hkv, kl, D]
        vt = torch.from_numpy(vs[r]).permute(1, 0, 2).unsqueeze(0)
        i = torch.arange(ql).unsqueeze(1)
        t = torch.arange(kl).unsqueeze(0)
        mask = (t <= kl - ql + i) if b.causal else torch.ones(ql, kl, dtype=torch.bool)
        o = torch.nn.functional.scaled_dot_product_attention(
            qt, kt, vt, attn_mask=mask, scale=b.sm_scale, enable_gqa=True)
        out[q0:q1] = o[0].permute(1, 0, 2).numpy()
        # lse through scipy on scores from a library matmul, with the same mask
        G = b.group
        kr = np.repeat(ks[r], G, axis=1)                                     # [kl, Hq, D]
        s = np.einsum("ihd,thd->iht", q_all[q0:q1], kr) * b.sm_scale
        s = np.where(mask.numpy()[:, None, :], s, -np.inf)
        lse[q0:q1] = logsumexp(s, axis=-1)
    return out, lse


SDPA_CASES = [
    dict(kv=[1, 17, 100, 300], Hq=14, Hkv=2, D=64, P=16, dtype="bf16"),
    dict(kv=[5, 33, 70], Hq=2, Hkv=2, D=64, P=16, dtype="bf16"),             # G = 1
    dict(kv=[3, 129, 257], Hq=12, Hkv=2, D=128, P=256, dtype="f16"),         # G = 6, d 128
    dict(kv=[1, 40, 90], Hq=14, Hkv=2, D=64, P=64, dtype="f32"),
    dict(kv=[80, 17, 33], qo=[37, 1, 1], Hq=14, Hkv=2, D=64, P=16, dtype="bf16"),  # ragged causal
    dict(kv=[50, 20], qo=[50, 1], Hq=8, Hkv=1, D=64, P=16, dtype="f16"),     # chunk = whole history
    dict(kv=[60, 9], qo=[7, 3], Hq=4, Hkv=2, D=64, P=16, dtype="f32", causal=False),
]


@pytest.mark.parametrize("case", SDPA_CASES, ids=lambda c: f"{c['dtype']}-G{c['Hq']//c['Hkv']}-D{c['D']}-P{c['P']}-{'ragged' if 'qo' in c else 'decode'}")
def test_oracle_matches_torch_sdpa(case):
    b = W.make_batch(case["kv"], case.get("qo"), num_qo_heads=case["Hq"], num_kv_heads=case["Hkv"],
                     head_dim=case["D"], page_size=case["P"], dtype=case["dtype"],
                     num_pages=sum(-(-k // case["P"]) for k in case["kv"]) + 5, seed=7,
                     keep_dense=True, causal=case.get("causal", True))
    out, lse = oracle.attention(b)
    ref, ref_lse = sdpa_reference(b)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-11)


def test_golden_two_key_closed_form():
    fx = json.load(open(os.path.join(HERE, "golden", "two_key_closed_form.json")))
    P = 16
    k_pool = np.full((1, P, 1, 2), np.nan, dtype=np.float32)
    v_pool = np.full((1, P, 1, 2), np.nan, dtype=np.float32)
    k_pool[0, :2, 0] = fx["k"]
    v_pool[0, :2, 0] = fx["v"]
    q = np.array(fx["q"], dtype=np.float32).reshape(1, 1, 2)
    out, lse = oracle.paged_attention(3, [0, 1], [0, 1], [0], [2], 1, 1, 1, 2, P, q, k_pool, v_pool,
                                      True, math.log(3) / 2)
    np.testing.assert_allclose(out[0, 0], fx["expected_out"], rtol=0, atol=fx["tolerance"])
    assert abs(lse[0, 0] - math.log(4)) < fx["tolerance"]


@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_single_key_returns_value_row(dtype):
    b = W.make_batch([1, 1, 1], num_qo_heads=6, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype=dtype, seed=3, keep_dense=True)
    out, lse = oracle.attention(b)
    v = dense_f64(b, b.dense_v)
    for r in range(3):
        for h in range(6):
            assert np.array_equal(out[r, h], v[r][0, h // 3])   # bit-exact
    q = W.storage_to_f32(b.q, dtype).astype(np.float64)
    k = dense_f64(b, b.dense_k)
    for r in range(3):
        for h in range(6):
            s = b.sm_scale * float(np.dot(q[r, h], k[r][0, h // 3]))
            assert abs(lse[r, h] - s) < 1e-12


def test_zero_query_gives_mean_and_log_n():
    b = W.make_batch([1, 7, 40, 300], [1, 1, 5, 1], num_qo_heads=4, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="bf16", seed=4, keep_dense=True)
    b.q[:] = 0
    out, lse = oracle.attention(b)
    v = dense_f64(b, b.dense_v)
    for r in range(b.batch_size):
        ql, kl = int(b.qo_lens[r]), int(b.kv_lens[r])
        for i in range(ql):
            n = kl - ql + i + 1
            row = int(b.qo_indptr[r]) + i
            for h in range(4):
                np.testing.assert_allclose(out[row, h], v[r][:n, h // 2].mean(axis=0), rtol=0, atol=1e-14)
                assert abs(lse[row, h] - math.log(n)) < 1e-13


def test_identical_keys_give_uniform_weights():
    b = W.make_batch([23, 64], num_qo_heads=2, num_kv_heads=1, head_dim=64, page_size=16,
                     dtype="f32", seed=5, keep_dense=True)
    for r in range(2):
        # overwrite every key slot of request r with its token-0 key, through the page table
        pages = b.kv_indices[b.kv_indptr[r]:b.kv_indptr[r + 1]]
        k0 = b.dense_k[r][0].copy()
        for t in range(int(b.kv_lens[r])):
            b.k_pool[pages[t // 16], t % 16] = k0
    out, _ = oracle.attention(b)
    v = dense_f64(b, b.dense_v)
    for r in range(2):
        for h in range(2):
            np.testing.assert_allclose(out[r, h], v[r][:, 0].mean(axis=0), rtol=0, atol=1e-14)


def test_two_keys_sigmoid_closed_form():
    b = W.make_batch([2] * 6, num_qo_heads=3, num_kv_heads=1, head_dim=64, page_size=16,
                     dtype="f32", seed=6, keep_dense=True)
    out, _ = oracle.attention(b)
    q = W.storage_to_f32(b.q, "f32").astype(np.float64)
    for r in range(6):
        k = b.dense_k[r].astype(np.float64)
        v = b.dense_v[r].astype(np.float64)
        for h in range(3):
            d = b.sm_scale * (q[r, h] @ k[1, 0] - q[r, h] @ k[0, 0])
            ref = v[0, 0] + (v[1, 0] - v[0, 0]) * expit(d)
            np.testing.assert_allclose(out[r, h], ref, rtol=0, atol=1e-14)


def _needle_batch(kv_lens, qo_lens, P, dtype="bf16"):
    """Zero keys, value rows that spell (request, position) in small integers."""
    b = W.make_batch(kv_lens, qo_lens, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=P,
                     dtype=dtype, seed=11, keep_dense=False, num_pages=sum(-(-k // P) for k in kv_lens) + 9)
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
            row[:, 3] = np.array([1, 2])          # kv head
            row[:, 4:] = ((np.arange(60) * 7 + t + 3 * r) % 251) - 125
            b.v_pool[pg, sl] = W.to_storage(row, dtype)
    b.q[:] = zero
    return b


def _plant(b, r, t, c_q=32.0, c_k=256.0):
    P = b.page_size
    pg = b.kv_indices[b.kv_indptr[r] + t // P]
    b.k_pool[pg, t % P, :, 0] = W.to_storage(np.array([c_k], np.float32), b.dtype)[0]
    q0 = int(b.qo_indptr[r])
    b.q[q0:int(b.qo_indptr[r + 1]), :, 0] = W.to_storage(np.array([c_q], np.float32), b.dtype)[0]


@pytest.mark.parametrize("P", [16, 64, 256])
def test_needles_are_bit_exact(P):
    kv = [1, P, P + 1, 3 * P - 1, 300]
    b = _needle_batch(kv, None, P)
    spots = [0, P - 1, P, 3 * P - 2, 299]        # first slot, last slot of a page, first of next,
    for r, t in enumerate(spots):                # last valid token (last_page_len - 1), deep
        _plant(b, r, t)
    out, _ = oracle.attention(b)
    for r, t in enumerate(spots):
        pg = b.kv_indices[b.kv_indptr[r] + t // P]
        v = W.storage_to_f32(b.v_pool[pg, t % P], b.dtype).astype(np.float64)
        for h in range(14):
            assert np.array_equal(out[r, h], v[h // 7]), (r, t, h)


def test_causal_limit_needles():
    P = 16
    kv, qo = [70], [20]
    b = _needle_batch(kv, qo, P)
    i = 9                                         # row 9 sees keys t <= 70 - 20 + 9 = 59
    lim = kv[0] - qo[0] + i
    _plant(b, 0, lim)
    out, _ = oracle.attention(b)
    pg = b.kv_indices[lim // P]
    v = W.storage_to_f32(b.v_pool[pg, lim % P], "bf16").astype(np.float64)
    assert np.array_equal(out[i, 0], v[0])        # the limit itself is seen
    # rows before i do not see the needle: uniform mean over their own keys
    vd = np.stack([W.storage_to_f32(b.v_pool[b.kv_indices[t // P], t % P], "bf16") for t in range(70)]).astype(np.float64)
    for ii in range(i):
        n = kv[0] - qo[0] + ii + 1
        np.testing.assert_allclose(out[ii, 0], vd[:n, 0].mean(axis=0), rtol=0, atol=1e-13)
        assert np.isfinite(out[ii]).all()


def test_page_permutation_is_bit_identical():
    b = W.tiny_decode(seed=2)
    perm = W.rng_for(99, 0, 0).permutation(b.num_pages)
    b2 = W.relabel_pages(b, perm)
    o1, l1 = oracle.attention(b)
    o2, l2 = oracle.attention(b2)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_page_size_relayout_is_bit_identical():
    res = []
    for P in (16, 64, 256):
        b = W.make_batch([1, 17, 100, 300, 513], [1, 1, 1, 9, 1], num_qo_heads=14, num_kv_heads=2,
                         head_dim=64, page_size=P, dtype="bf16", seed=8,
                         num_pages=sum(-(-k // P) for k in [1, 17, 100, 300, 513]) + 3)
        res.append(oracle.attention(b))
    for o, l in res[1:]:
        assert np.array_equal(o, res[0][0]) and np.array_equal(l, res[0][1])


def test_gqa_equals_repeated_mha():
    b = W.make_batch([5, 60, 200], [1, 4, 1], num_qo_heads=12, num_kv_heads=2, head_dim=128,
                     page_size=64, dtype="f16", seed=9)
    G = b.group
    m = W.Batch(**{**b.__dict__})
    m.num_kv_heads = b.num_qo_heads
    m.k_pool = np.ascontiguousarray(np.repeat(b.k_pool, G, axis=2))
    m.v_pool = np.ascontiguousarray(np.repeat(b.v_pool, G, axis=2))
    o1, l1 = oracle.attention(b)
    o2, l2 = oracle.attention(m)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    # and the two kv heads really differ, so a wrong head map would show
    assert not np.array_equal(o1[:, 0], o1[:, G])


def test_shared_prefix_pages_equal_private_copies():
    P = 16
    b = W.make_batch([100, 100, 37], num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=P,
                     dtype="bf16", seed=10, num_pages=64)
    o_orig, _ = oracle.attention(b)
    s = b.kv_indptr
    # private: request 1's first 4 pages hold copies of request 0's first 4 pages
    kp, vp = b.k_pool.copy(), b.v_pool.copy()
    for j in range(4):
        kp[b.kv_indices[s[1] + j]] = b.k_pool[b.kv_indices[s[0] + j]]
        vp[b.kv_indices[s[1] + j]] = b.v_pool[b.kv_indices[s[0] + j]]
    private = dataclasses.replace(b, k_pool=kp, v_pool=vp)
    # shared: request 1's table points at request 0's physical pages for that prefix
    idx = b.kv_indices.copy()
    idx[s[1]:s[1] + 4] = b.kv_indices[s[0]:s[0] + 4]
    shared = dataclasses.replace(private, kv_indices=idx)
    o_private, l_private = oracle.attention(private)
    o_shared, l_shared = oracle.attention(shared)
    assert np.array_equal(o_private, o_shared) and np.array_equal(l_private, l_shared)
    assert not np.array_equal(o_orig[1], o_private[1])   # the prefix copy changed request 1


def test_last_prefill_row_equals_decode_row():
    P = 16
    b = W.make_batch([40, 40], [6, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=P,
                     dtype="bf16", seed=12, num_pages=10)
    # request 1 reads request 0's pages and asks with request 0's last query row
    s = b.kv_indptr
    b.kv_indices[s[1]:s[2]] = b.kv_indices[s[0]:s[1]]
    b.q[6] = b.q[5]
    out, lse = oracle.attention(b)
    assert np.array_equal(out[5], out[6]) and np.array_equal(lse[5], lse[6])


@pytest.mark.parametrize("splits", [2, 3, 7, 64, 1000])
def test_split_merge_matches_single_pass(splits):
    b = W.make_batch([1, 17, 100, 300, 700], [1, 1, 1, 30, 1], num_qo_heads=14, num_kv_heads=2,
                     head_dim=64, page_size=16, dtype="bf16", seed=13)
    o1, l1 = oracle.attention(b)
    o2, l2 = oracle.attention(b, num_splits=splits)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l2, l1, rtol=0, atol=1e-12)


def test_f16_decoder_matches_numpy_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(1, bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_bf16_decoder_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = oracle.decode(2, bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(got), nan)
    assert np.array_equal(got[~nan], ref[~nan])


def test_generator_rounding_matches_torch_bf16():
    x = W.rng_for(0, 0, 9).standard_normal(100000, dtype=np.float32)
    x[:4] = [1.00390625, 1.01171875, -2.0039062, 3.3e-39]     # ties and a subnormal
    ours = W.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_oracle_rejects_bad_metadata():
    b = W.tiny_decode()
    good = dict(qo=b.qo_indptr, kvp=b.kv_indptr, kvi=b.kv_indices, last=b.last_page_len)

    def run(**kw):
        a = {**good, **kw}
        return oracle.paged_attention(b.dtype_code, a["qo"], a["kvp"], a["kvi"], a["last"], b.num_pages,
                                      14, 2, 64, 16, b.q, b.k_pool, b.v_pool)
    bad_idx = b.kv_indices.copy(); bad_idx[3] = b.num_pages
    with pytest.raises(oracle.OracleError):
        run(kvi=bad_idx)
    bad_last = b.last_page_len.copy(); bad_last[1] = 0
    with pytest.raises(oracle.OracleError):
        run(last=bad_last)
    bad_last[1] = 17
    with pytest.raises(oracle.OracleError):
        run(last=bad_last)
    bad_qo = np.array([0, 1, 2, 3, 305], np.int32)        # 302 rows on a 300-token history
    with pytest.raises(oracle.OracleError):
        run(qo=bad_qo)


def test_generator_is_deterministic_and_poisons_unused_slots():
    a = W.tiny_decode(seed=0)
    b = W.tiny_decode(seed=0)
    assert np.array_equal(a.k_pool.view(np.uint16), b.k_pool.view(np.uint16))
    assert np.array_equal(a.q, b.q)
    used = np.zeros((a.num_pages, a.page_size), bool)
    for r in range(a.batch_size):
        pages = a.kv_indices[a.kv_indptr[r]:a.kv_indptr[r + 1]]
        for t in range(int(a.kv_lens[r])):
            used[pages[t // 16], t % 16] = True
    vals = W.storage_to_f32(a.k_pool, "bf16")
    assert np.isnan(vals[~used]).all() and np.isfinite(vals[used]).all()


# ---------------------------------------------------------------------------------------
# appending a step's new K/V rows to the paged cache
# ---------------------------------------------------------------------------------------
def as_bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


APPEND_CASES = [
    dict(kv=[1, 17, 100, 300], Hkv=2, D=64, P=16, dtype="bf16"),
    dict(kv=[16, 17, 64, 65, 300], Hkv=2, D=128, P=64, dtype="f16"),
    dict(kv=[3, 256, 257, 600], Hkv=1, D=64, P=256, dtype="f32"),
    dict(kv=[80, 17, 33, 5], qo=[37, 1, 0, 5], Hkv=2, D=64, P=16, dtype="bf16"),  # ragged, empty
    dict(kv=[50, 20], qo=[50, 1], Hkv=8, D=64, P=16, dtype="f16"),                # whole history
]


@pytest.mark.parametrize("case", APPEND_CASES,
                         ids=lambda c: f"{c['dtype']}-Hkv{c['Hkv']}-D{c['D']}-P{c['P']}-{'ragged' if 'qo' in c else 'decode'}")
def test_append_restores_the_generator_pools(case):
    """The generator scatters every request's whole history; with the newest qo_len tokens
    taken out (poisoned) and given as new rows, the append must rebuild the same pools, byte
    for byte, NaN slots included."""
    b = W.make_batch(case["kv"], case.get("qo"), num_qo_heads=case["Hkv"] * 2,
                     num_kv_heads=case["Hkv"], head_dim=case["D"], page_size=case["P"],
                     dtype=case["dtype"], num_pages=sum(-(-k // case["P"]) for k in case["kv"]) + 4,
                     seed=21, keep_dense=True)
    st = W.append_step(b)
    assert not np.array_equal(as_bytes(st.k_before), as_bytes(b.k_pool))
    k, v = oracle.kv_append(b, st.k_new, st.v_new, st.k_before, st.v_before)
    assert np.array_equal(as_bytes(k), as_bytes(b.k_pool))
    assert np.array_equal(as_bytes(v), as_bytes(b.v_pool))


def test_append_writes_the_slots_worked_out_by_hand():
    """Three requests on a pool of 4 pages of 16 slots, one kv head, head_dim 64, fp32.
      r0: pages [2, 0], last_page_len 1  -> kv_len 17, its one new token is token 16:
          page 0, slot 0 (the first slot of its second page)
      r1: pages [3],    last_page_len 16 -> kv_len 16, new token 15: page 3, slot 15
      r2: pages [1],    last_page_len 5, 3 new rows -> tokens 2, 3, 4: page 1, slots 2-4
    Every other slot keeps its old value."""
    qo_indptr = np.array([0, 1, 2, 5], np.int32)
    kv_indptr = np.array([0, 2, 3, 4], np.int32)
    kv_indices = np.array([2, 0, 3, 1], np.int32)
    last = np.array([1, 16, 5], np.int32)
    rng = np.random.default_rng(3)
    k_pool = rng.standard_normal((4, 16, 1, 64)).astype(np.float32)
    v_pool = rng.standard_normal((4, 16, 1, 64)).astype(np.float32)
    k_new = (1000 + np.arange(5, dtype=np.float32))[:, None, None] * np.ones((5, 1, 64), np.float32)
    v_new = -k_new
    k, v = oracle.paged_kv_append(4, qo_indptr, kv_indptr, kv_indices, last, 4, 1, 64, 16,
                                  k_new, v_new, k_pool, v_pool)
    expect_k, expect_v = k_pool.copy(), v_pool.copy()
    for row, (page, slot) in enumerate([(0, 0), (3, 15), (1, 2), (1, 3), (1, 4)]):
        expect_k[page, slot] = 1000 + row
        expect_v[page, slot] = -(1000 + row)
    assert np.array_equal(k, expect_k) and np.array_equal(v, expect_v)


def test_append_then_attention_matches_the_full_history():
    b = W.make_batch([80, 17, 33], [37, 1, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="bf16", seed=22, keep_dense=True)
    st = W.append_step(b)
    k, v = oracle.kv_append(b, st.k_new, st.v_new, st.k_before, st.v_before)
    out_full, lse_full = oracle.attention(b)
    out, lse = oracle.attention(dataclasses.replace(b, k_pool=k, v_pool=v))
    assert np.array_equal(out, out_full) and np.array_equal(lse, lse_full)


def test_append_rejects_bad_metadata():
    b = W.tiny_decode(keep_dense=True)
    st = W.append_step(b)

    def run(qo=b.qo_indptr, kvi=b.kv_indices):
        return oracle.paged_kv_append(2, qo, b.kv_indptr, kvi, b.last_page_len, b.num_pages, 2, 64,
                                      16, st.k_new, st.v_new, st.k_before, st.v_before)
    with pytest.raises(oracle.OracleError):
        run(qo=np.array([0, 2, 3, 4, 5], np.int32))      # 2 new rows on a 1-token history
    bad = b.kv_indices.copy(); bad[0] = -1
    with pytest.raises(oracle.OracleError):
        run(kvi=bad)


# ---------------------------------------------------------------------------------------
# freed-page poisoning and the page allocator's reference bookkeeping
# ---------------------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["bf16", "f16", "f32"])
def test_poison_fills_listed_pages_with_nan_only(dtype):
    b = W.make_batch([40, 7], num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype=dtype, num_pages=8, seed=23, poison=False)
    k, v = oracle.paged_kv_poison(b.dtype_code, [5, 1, 5], b.k_pool, b.v_pool)
    kf, vf = W.storage_to_f32(k, dtype), W.storage_to_f32(v, dtype)
    for p in range(8):
        if p in (1, 5):
            assert np.isnan(kf[p]).all() and np.isnan(vf[p]).all()
        else:
            assert np.array_equal(as_bytes(k[p]), as_bytes(b.k_pool[p]))
            assert np.array_equal(as_bytes(v[p]), as_bytes(b.v_pool[p]))
    # the canonical quiet NaN of each type, as numpy / torch spell it
    ref = {"bf16": torch.tensor(float("nan"), dtype=torch.bfloat16).view(torch.int16).item() & 0xFFFF,
           "f16": int(np.float16(np.nan).view(np.uint16)),
           "f32": int(np.float32(np.nan).view(np.uint32))}[dtype]
    assert int(np.ascontiguousarray(k[1]).reshape(-1).view(
        np.uint32 if dtype == "f32" else np.uint16)[0]) == ref


def test_poisoned_page_makes_attention_nan():
    """A request whose page table still names a freed (poisoned) page reads NaN."""
    b = W.make_batch([40, 7], num_qo_heads=4, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype="bf16", num_pages=8, seed=24)
    freed = int(b.kv_indices[b.kv_indptr[1]])   # the page of request 1
    k, v = oracle.paged_kv_poison(b.dtype_code, [freed], b.k_pool, b.v_pool)
    out, _ = oracle.attention(dataclasses.replace(b, k_pool=k, v_pool=v))
    assert np.isfinite(out[0]).all() and np.isnan(out[1]).all()


def test_poison_rejects_pages_outside_the_pool():
    b = W.tiny_decode()
    with pytest.raises(oracle.OracleError):
        oracle.paged_kv_poison(b.dtype_code, [b.num_pages], b.k_pool, b.v_pool)


def test_pool_model_whole_page_reservation():
    from oracle.page_pool import PagePoolModel
    m = PagePoolModel(64, 256)
    # 300 slots on 256-slot pages hold two pages (512 slots); on 64-slot pages five (320)
    assert m.pages_for(300) == 2 and PagePoolModel(64, 64).pages_for(300) == 5
    assert m.pages_for(0) == 0 and m.pages_for(1) == 1 and m.pages_for(256) == 1 and m.pages_for(257) == 2


def test_pool_model_worked_sequence():
    """Four pages. Request A takes pages 0, 1; B adopts A's first page (prefix sharing) and
    takes page 2 of its own; A finishes: only page 1 frees (page 0 is still B's); B finishes:
    pages 0 and 2 free, in list order."""
    from oracle.page_pool import PagePoolModel, PoolModelError
    m = PagePoolModel(4, 16)
    m.alloc([0, 1])
    m.retain([0])
    m.alloc([2])
    assert m.refs == [2, 1, 1, 0] and m.num_free == 1 and m.num_live == 3
    assert m.release([0, 1]) == [1]
    assert m.refs == [1, 0, 1, 0]
    assert m.release([2, 0]) == [2, 0]
    assert m.num_free == 4
    with pytest.raises(PoolModelError):
        m.release([3])                  # never held
    m.alloc([3])
    with pytest.raises(PoolModelError):
        m.release([3, 3])               # released twice, held once: nothing changes
    assert m.refs[3] == 1
    with pytest.raises(PoolModelError):
        m.alloc([3])                    # handed out while held
    with pytest.raises(PoolModelError):
        m.alloc([0, 0])                 # the same page twice
    with pytest.raises(PoolModelError):
        m.retain([1])                   # adopt a free page
    assert not m.can_alloc(4) and m.can_alloc(3)


# ---- rotary embedding (the append fused with RoPE) ---------------------------------------

def _rope_angles(pos, d, theta):
    """The reading's angles: f_i = theta^(-2i/D) in binary32, a_i = binary32(pos) * f_i."""
    f = (float(theta) ** (-2.0 * np.arange(d // 2) / d)).astype(np.float32)
    return (np.asarray(pos, dtype=np.float32)[:, None] * f[None, :]).astype(np.float64)


def test_rope_textbook_values():
    """head_dim 2: one pair, frequency 1, so position 1 turns (1, 0) by one radian onto
    (cos 1, sin 1) = (0.5403023058681398, 0.8414709848078965), and (0, 1) onto (-sin 1, cos 1)."""
    x = np.array([[[1.0, 0.0]], [[0.0, 1.0]]], np.float32)
    y = oracle.rope(3, x, [1, 1], 10000.0)
    assert np.allclose(y[0, 0], [0.5403023058681398, 0.8414709848078965], rtol=0, atol=1e-15)
    assert np.allclose(y[1, 0], [-0.8414709848078965, 0.5403023058681398], rtol=0, atol=1e-15)


@pytest.mark.parametrize("d,theta", [(64, 1e4), (128, 1e6), (8, 500.0)])
def test_rope_is_complex_multiplication(d, theta):
    """Independent form: z_i = x[i] + j x[i + D/2] times e^(j a_i) (numpy complex
    exponential) gives the rotate-half result; positions up to 40k."""
    rng = np.random.default_rng(d)
    x = rng.standard_normal((9, 3, d)).astype(np.float32)
    pos = np.array([0, 1, 2, 17, 300, 1535, 4096, 32767, 40000], np.int32)
    y = oracle.rope(3, x, pos, theta)
    a = _rope_angles(pos, d, theta)
    z = (x[..., : d // 2] + 1j * x[..., d // 2:].astype(np.float64)) * np.exp(1j * a)[:, None, :]
    assert np.abs(y[..., : d // 2] - z.real).max() < 1e-12
    assert np.abs(y[..., d // 2:] - z.imag).max() < 1e-12


def test_rope_position_zero_is_identity_and_pairs_keep_their_norm():
    rng = np.random.default_rng(3)
    x = W.to_storage(rng.standard_normal((5, 2, 64)).astype(np.float32), "bf16")
    xd = W.storage_to_f32(x, "bf16").astype(np.float64)
    y0 = oracle.rope(2, x, [0] * 5, 1e4)
    assert np.array_equal(y0, xd)
    y = oracle.rope(2, x, [3, 70, 511, 2048, 9999], 1e4)
    n_in = xd[..., :32] ** 2 + xd[..., 32:] ** 2
    n_out = y[..., :32] ** 2 + y[..., 32:] ** 2
    assert np.abs(n_out - n_in).max() < 1e-12 * max(1.0, n_in.max())


def test_rope_scores_depend_on_relative_position_only():
    """<R(q, m), R(k, n)> = <R(q, m + s), R(k, n + s)>: with theta = 16 and D = 4 the
    frequencies 1 and 1/4 are exact in binary32, so the angles of integer positions are
    exact and the identity holds to rounding."""
    rng = np.random.default_rng(5)
    q = rng.standard_normal((1, 1, 4)).astype(np.float32)
    k = rng.standard_normal((1, 1, 4)).astype(np.float32)
    for m, n, s in [(5, 2, 7), (100, 0, 33), (1000, 999, 4000)]:
        d0 = np.dot(oracle.rope(3, q, [m], 16.0).ravel(), oracle.rope(3, k, [n], 16.0).ravel())
        d1 = np.dot(oracle.rope(3, q, [m + s], 16.0).ravel(), oracle.rope(3, k, [n + s], 16.0).ravel())
        assert abs(d0 - d1) < 1e-9, (m, n, s)


def test_rope_rejects_bad_arguments():
    x = np.zeros((1, 1, 4), np.float32)
    for kw in (dict(theta=0.0), dict(theta=-1.0)):
        with pytest.raises(oracle.OracleError):
            oracle.rope(3, x, [0], **kw)
    with pytest.raises(oracle.OracleError):
        oracle.rope(3, np.zeros((1, 1, 3), np.float32), [0], 1e4)


def test_append_positions_follow_the_bottom_right_reading():
    """Request 0: 3 new rows over 40 cached tokens -> positions 37, 38, 39; request 1: one
    decode row over 17 tokens -> 16."""
    pos = oracle.append_positions([0, 3, 4], [0, 3, 5], [8, 1], 16)
    assert pos.tolist() == [37, 38, 39, 16]
