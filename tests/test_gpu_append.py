"""GPU parity of the KV append: the HIP kernel against the CPU oracle, through the C interface.

The append is a byte copy, so the bar is bit-exact: after the GPU append, both pools must
equal the oracle's appended pools byte for byte (the NaN poison of unused slots included).
Inputs: a seeded batch's pools with each request's newest qo_len tokens taken out and
poisoned, plus those tokens as the new rows (workloads.append_step).
"""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_plan_amd as fl
import workloads as W
from gpu_helpers import announce, compare, config_for, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


def _device_append(b, st, h=None):
    """Plan b on a device handle, append st's rows into device copies of the before-pools;
    returns (handle, k_pool, v_pool, k_new, v_new) on the device."""
    import torch
    h = h or fl.PagedAttention(config_for(b), device=0)
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
           causal=b.causal, sm_scale=b.sm_scale)
    k = to_device(st.k_before, b.dtype)
    v = to_device(st.v_before, b.dtype)
    kn = to_device(st.k_new, b.dtype)
    vn = to_device(st.v_new, b.dtype)
    h.append(kn, vn, k, v)
    torch.cuda.synchronize()
    return h, k, v, kn, vn


def _check_append(b, what=""):
    announce(f"append {what or b.name}: dtype={b.dtype} B={b.batch_size} rows={b.rows} "
             f"Hkv={b.num_kv_heads} D={b.head_dim} P={b.page_size}")
    st = W.append_step(b)
    ref_k, ref_v = oracle.kv_append(b, st.k_new, st.v_new, st.k_before, st.v_before)
    h, k, v, _, _ = _device_append(b, st)
    assert np.array_equal(_bytes(to_host_bits(k, b.dtype)), _bytes(ref_k)), f"{what}: K pool"
    assert np.array_equal(_bytes(to_host_bits(v, b.dtype)), _bytes(ref_v)), f"{what}: V pool"
    return h, k, v


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_append_workloads_full_size(name):
    _check_append(W.WORKLOADS[name](keep_dense=True))


APPEND_VARIANTS = [
    dict(kv=[16, 17, 64, 65, 300], Hq=12, Hkv=2, D=128, P=64, dtype="f16"),
    dict(kv=[3, 256, 257, 600], Hq=4, Hkv=1, D=64, P=256, dtype="f32"),
    dict(kv=[33, 1, 900], Hq=32, Hkv=8, D=128, P=16, dtype="bf16"),
    dict(kv=[80, 17, 33, 5, 1], qo=[37, 1, 0, 5, 1], Hq=14, Hkv=2, D=64, P=16, dtype="bf16"),
    dict(kv=[50, 20, 256], qo=[50, 1, 256], Hq=8, Hkv=1, D=128, P=256, dtype="f32"),
]


@pytest.mark.parametrize("case", APPEND_VARIANTS,
                         ids=lambda c: f"{c['dtype']}-Hkv{c['Hkv']}-D{c['D']}-P{c['P']}-{'ragged' if 'qo' in c else 'decode'}")
def test_append_variants(case):
    b = W.make_batch(case["kv"], case.get("qo"), num_qo_heads=case["Hq"], num_kv_heads=case["Hkv"],
                     head_dim=case["D"], page_size=case["P"], dtype=case["dtype"],
                     num_pages=sum(-(-k // case["P"]) for k in case["kv"]) + 6, seed=31,
                     keep_dense=True)
    _check_append(b, what=str(case))


def test_append_then_attention_matches_oracle_on_two_layers():
    """One plan per step serves every layer: append layer l's new rows into layer l's pools,
    then run attention on them; each layer matches the oracle on its full history."""
    import torch

    def layer(l):
        return W.make_batch([300, 17, 1536, 100], [1, 1, 512, 1], num_qo_heads=14, num_kv_heads=2,
                            head_dim=64, page_size=16, dtype="bf16", seed=50 + l, num_pages=200,
                            keep_dense=True)
    b0 = layer(0)
    # layer 1 has its own values; its pages are relabelled onto layer 0's page table
    b1 = layer(1)
    perm = np.full(b1.num_pages, -1, np.int64)
    perm[b1.kv_indices] = b0.kv_indices
    perm[np.setdiff1d(np.arange(b1.num_pages), b1.kv_indices)] = np.setdiff1d(
        np.arange(b0.num_pages), b0.kv_indices)
    layers = [b0, W.relabel_pages(b1, perm)]
    h = fl.PagedAttention(config_for(b0), device=0)
    h.plan(b0.qo_indptr, b0.kv_indptr, b0.kv_indices, b0.last_page_len, b0.num_pages,
           causal=True, sm_scale=b0.sm_scale)
    for l, b in enumerate(layers):
        announce(f"append + attention, layer {l}")
        assert np.array_equal(b.kv_indices, b0.kv_indices)
        st = W.append_step(b)
        k, v = to_device(st.k_before, b.dtype), to_device(st.v_before, b.dtype)
        kn, vn = to_device(st.k_new, b.dtype), to_device(st.v_new, b.dtype)
        q = to_device(b.q, b.dtype)
        out = torch.full(q.shape, float("nan"), dtype=torch_dtype(b.dtype), device="cuda:0")
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda:0")
        h.append(kn, vn, k, v)
        h.run(q, k, v, out, lse)
        torch.cuda.synchronize()
        ref_out, ref_lse = oracle.attention(b)
        compare(b, out, lse, ref_out, ref_lse, f"layer {l}")


def test_append_graph_replay_across_replans():
    """append + run captured once in a HIP graph; each replay after a new plan (other page
    ids, same lengths) writes the new rows to the new slots."""
    import torch
    b1 = W.make_batch([40, 300, 17, 1], [1, 1, 9, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                      page_size=16, dtype="bf16", seed=61, num_pages=64, keep_dense=True)
    b2 = W.relabel_pages(b1, W.rng_for(62, 0, 0).permutation(b1.num_pages))
    st1 = W.append_step(b1)
    st2 = W.append_step(b2)
    announce("append graph replay across re-plans")
    h, k, v, kn, vn = _device_append(b1, st1)
    q = to_device(b1.q, b1.dtype)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda:0")
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.append(kn, vn, k, v)
        h.run(q, k, v, out)
    ref = oracle.attention(b1)
    for rep in range(4):
        bb, st = (b2, st2) if rep % 2 else (b1, st1)
        h.plan(bb.qo_indptr, bb.kv_indptr, bb.kv_indices, bb.last_page_len, bb.num_pages,
               causal=True, sm_scale=bb.sm_scale)
        k.copy_(to_device(st.k_before, bb.dtype))
        v.copy_(to_device(st.v_before, bb.dtype))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_k, ref_v = oracle.kv_append(bb, st.k_new, st.v_new, st.k_before, st.v_before)
        assert np.array_equal(_bytes(to_host_bits(k, bb.dtype)), _bytes(ref_k)), f"replay {rep}"
        assert np.array_equal(_bytes(to_host_bits(v, bb.dtype)), _bytes(ref_v)), f"replay {rep}"
        compare(bb, out, None, ref[0], None, f"replay {rep}")
        x = torch.randn(1 << 20, device="cuda:0")  # unrelated eager work between replays
        float(x.sum())
        torch.cuda.synchronize()


def test_append_errors_and_empty_plan():
    import torch
    b = W.tiny_decode(keep_dense=True)
    st = W.append_step(b)
    h = fl.PagedAttention(config_for(b), device=0)
    k, v = to_device(st.k_before, b.dtype), to_device(st.v_before, b.dtype)
    kn, vn = to_device(st.k_new, b.dtype), to_device(st.v_new, b.dtype)
    with pytest.raises(fl.FlError) as e:
        h.append(kn, vn, k, v)
    assert e.value.status == fl.FL_ERR_NOT_PLANNED
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages)
    with pytest.raises(fl.FlError) as e:
        fl.fl_paged_kv_append(h.handle, kn.data_ptr() + 2, vn.data_ptr(), k.data_ptr(), v.data_ptr())
    assert e.value.status == fl.FL_ERR_INVALID_ARG
    with pytest.raises(fl.FlError) as e:
        fl.fl_paged_kv_append(h.handle, 0, vn.data_ptr(), k.data_ptr(), v.data_ptr())
    assert e.value.status == fl.FL_ERR_INVALID_ARG
    # a plan whose newest tokens share a slot: refused, pools untouched
    before = to_host_bits(k, b.dtype).copy()
    h.plan(None, np.array([0, 1, 2]), np.array([5, 5]), np.array([7, 7]), b.num_pages)
    with pytest.raises(fl.FlError) as e:
        h.append(kn, vn, k, v)
    assert e.value.status == fl.FL_ERR_INVALID_ARG
    # empty plan: a no-op
    h.plan(np.zeros(1, np.int32), np.zeros(1, np.int32), np.zeros(0, np.int32), np.zeros(0, np.int32),
           b.num_pages)
    h.append(kn, vn, k, v)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(to_host_bits(k, b.dtype)), _bytes(before))


# ---- append + attention in one call ----------------------------------------------------------
def _run_append_check(b, what, num_splits=0, **cfg_kw):
    """fl_paged_attn_run_append on the before-pools must give the oracle's attention over the
    full history and leave the oracle's appended pools."""
    import torch
    announce(f"run_append {what}: dtype={b.dtype} B={b.batch_size} rows={b.rows} "
             f"D={b.head_dim} P={b.page_size} splits={num_splits} {cfg_kw}")
    st = W.append_step(b)
    ref_out, ref_lse = oracle.attention(b)
    ref_k, ref_v = oracle.kv_append(b, st.k_new, st.v_new, st.k_before, st.v_before)
    h = fl.PagedAttention(config_for(b, **cfg_kw), device=0)
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
           causal=b.causal, sm_scale=b.sm_scale, num_splits=num_splits)
    k, v = to_device(st.k_before, b.dtype), to_device(st.v_before, b.dtype)
    kn, vn = to_device(st.k_new, b.dtype), to_device(st.v_new, b.dtype)
    q = to_device(b.q, b.dtype)
    out = torch.full(q.shape, float("nan"), dtype=torch_dtype(b.dtype), device="cuda:0")
    lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda:0")
    h.run_append(q, kn, vn, k, v, out, lse)
    torch.cuda.synchronize()
    compare(b, out, lse, ref_out, ref_lse, what)
    assert np.array_equal(_bytes(to_host_bits(k, b.dtype)), _bytes(ref_k)), f"{what}: K pool"
    assert np.array_equal(_bytes(to_host_bits(v, b.dtype)), _bytes(ref_v)), f"{what}: V pool"
    return h


@pytest.mark.parametrize("name", ["tiny_decode", "saturated_decode", "mixed_length_decode",
                                  "long_context_skew"])
def test_run_append_decode_workloads(name):
    _run_append_check(W.WORKLOADS[name](keep_dense=True), name)


@pytest.mark.parametrize("whole_rows", [1, -1])
@pytest.mark.parametrize("splits", [0, 1, 3])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_run_append_modes_and_pieces(whole_rows, splits, dtype):
    b = W.make_batch([1, 15, 16, 17, 300, 1000, 257], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype=dtype, seed=91, num_pages=120, keep_dense=True)
    _run_append_check(b, f"modes wr{whole_rows} s{splits} {dtype}", num_splits=splits,
                      whole_rows=whole_rows)


@pytest.mark.parametrize("case", ["ragged", "f32", "d128-p256", "g32"])
def test_run_append_other_plans(case):
    kw = dict(num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16, dtype="bf16")
    kv, qo = [80, 17, 300, 33], None
    if case == "ragged":      # a prefill chunk: append first, then attend (two launches)
        qo = [37, 1, 1, 5]
    elif case == "f32":
        kw["dtype"] = "f32"
    elif case == "g32":       # decode rows of 32 heads per kv head run as prefill units
        kw.update(num_qo_heads=32, num_kv_heads=1)
    else:                     # fused at head_dim 128, 256-slot pages
        kw.update(num_qo_heads=12, head_dim=128, page_size=256, dtype="f16")
        kv = [1, 256, 257, 700]
    b = W.make_batch(kv, qo, seed=92, num_pages=40, keep_dense=True, **kw)
    h = _run_append_check(b, f"run_append {case}")
    assert (h.launch()[1] != 0) == (case == "d128-p256")  # the one-launch form


@pytest.mark.parametrize("whole_rows", [1, -1])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_run_append_needle_in_the_new_token_bit_exact(whole_rows, dtype):
    """The new token's K is a needle (its score beats every other key by > 100 in log2
    units), so each head's output is exactly the new token's V row: checks that the
    fused kernel takes both K and V of the newest key from the new rows, at every position
    in its tile (first slot of a page, last slot, middle)."""
    import torch
    kv = [1, 16, 17, 31, 300, 1000, 513]
    b = W.make_batch(kv, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16, dtype=dtype,
                     seed=93, num_pages=140, keep_dense=True)
    st = W.append_step(b)
    zero = W.to_storage(np.zeros(1, np.float32), dtype)[0]
    big = W.to_storage(np.array([256.0], np.float32), dtype)[0]
    for r in range(len(kv)):            # history keys 0, new key a needle on dim 0
        pages = b.kv_indices[b.kv_indptr[r]:b.kv_indptr[r + 1]]
        for t in range(kv[r] - 1):
            st.k_before[pages[t // 16], t % 16] = zero
    st.k_new[:] = zero
    st.k_new[:, :, 0] = big
    b.q[:] = zero
    b.q[:, :, 0] = W.to_storage(np.array([32.0], np.float32), dtype)[0]
    announce(f"run_append needle {dtype} whole_rows={whole_rows}")
    h = fl.PagedAttention(config_for(b, whole_rows=whole_rows), device=0)
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages)
    k, v = to_device(st.k_before, dtype), to_device(st.v_before, dtype)
    kn, vn = to_device(st.k_new, dtype), to_device(st.v_new, dtype)
    q = to_device(b.q, dtype)
    out = torch.full(q.shape, float("nan"), dtype=torch_dtype(dtype), device="cuda:0")
    h.run_append(q, kn, vn, k, v, out)
    torch.cuda.synchronize()
    got = to_host_bits(out, dtype)
    for r in range(len(kv)):
        for hq in range(14):
            assert np.array_equal(np.ascontiguousarray(got[r, hq]).view(np.uint8),
                                  np.ascontiguousarray(st.v_new[r, hq // 7]).view(np.uint8)), (r, hq)


def test_run_append_graph_replay_across_replans():
    import torch
    b1 = W.make_batch([40, 300, 17, 1, 64], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                      page_size=16, dtype="bf16", seed=94, num_pages=64, keep_dense=True)
    b2 = W.relabel_pages(b1, W.rng_for(95, 0, 0).permutation(b1.num_pages))
    sts = [W.append_step(b1), W.append_step(b2)]
    announce("run_append graph replay across re-plans")
    h = fl.PagedAttention(config_for(b1), device=0)
    h.plan(b1.qo_indptr, b1.kv_indptr, b1.kv_indices, b1.last_page_len, b1.num_pages)
    k, v = to_device(sts[0].k_before, "bf16"), to_device(sts[0].v_before, "bf16")
    kn, vn = to_device(sts[0].k_new, "bf16"), to_device(sts[0].v_new, "bf16")
    q = to_device(b1.q, "bf16")
    out = torch.empty(q.shape, dtype=torch.bfloat16, device="cuda:0")
    h.run_append(q, kn, vn, k, v, out)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.run_append(q, kn, vn, k, v, out)
    ref = oracle.attention(b1)
    for rep in range(4):
        bb, st = (b2, sts[1]) if rep % 2 else (b1, sts[0])
        h.plan(bb.qo_indptr, bb.kv_indptr, bb.kv_indices, bb.last_page_len, bb.num_pages)
        k.copy_(to_device(st.k_before, "bf16"))
        v.copy_(to_device(st.v_before, "bf16"))
        out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref_k, ref_v = oracle.kv_append(bb, st.k_new, st.v_new, st.k_before, st.v_before)
        assert np.array_equal(_bytes(to_host_bits(k, "bf16")), _bytes(ref_k)), f"replay {rep}"
        assert np.array_equal(_bytes(to_host_bits(v, "bf16")), _bytes(ref_v)), f"replay {rep}"
        compare(bb, out, None, ref[0], None, f"replay {rep}")
        x = torch.randn(1 << 20, device="cuda:0")
        float(x.sum())
        torch.cuda.synchronize()


# ---- the append fused with the rotary embedding (fl_paged_kv_append_rope) ----------------
# The rotation is floating-point work: rotated K rows in the pool and rotated query heads
# must be within one unit in the last place of the storage type of the oracle's double
# result (the device rotates in fp32 and rounds once; the oracle's value, rounded once, may
# sit across a rounding boundary), plus 1e-6 of fp32 arithmetic (4e-6 for fp32 storage).
# V rows and every untouched slot must match the oracle's append byte for byte.

_MANT = {"bf16": 7, "f16": 10, "f32": 23}
_EMIN = {"bf16": -126, "f16": -14, "f32": -126}


def _ulp(v, dtype):
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** _EMIN[dtype])))
    return 2.0 ** (e - _MANT[dtype])


def _rope_tol(ref, dtype):
    if dtype == "f32":
        return 4e-6 * (1.0 + np.abs(ref))
    return _ulp(ref, dtype) + 1e-6 * (1.0 + np.abs(ref))


def _bits(a, dtype):
    a = np.ascontiguousarray(a)
    return a.view(np.uint32 if dtype == "f32" else np.uint16)


def _check_rope(b, theta, with_q=True, what=""):
    import torch
    announce(f"append+rope {what or b.name}: dtype={b.dtype} rows={b.rows} Hq={b.num_qo_heads} "
             f"Hkv={b.num_kv_heads} D={b.head_dim} P={b.page_size} theta={theta} q={with_q}")
    st = W.append_step(b)
    code = W.DTYPE_CODES[b.dtype]
    pos = oracle.append_positions(b.qo_indptr, b.kv_indptr, b.last_page_len, b.page_size)
    k_rot = oracle.rope(code, st.k_new, pos, theta)
    q_rot = oracle.rope(code, b.q, pos, theta)
    ref_k, ref_v = oracle.kv_append(b, W.to_storage(k_rot.astype(np.float32), b.dtype), st.v_new,
                                    st.k_before, st.v_before)
    h = fl.PagedAttention(config_for(b), device=0)
    h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
           causal=b.causal, sm_scale=b.sm_scale)
    k, v = to_device(st.k_before, b.dtype), to_device(st.v_before, b.dtype)
    kn, vn = to_device(st.k_new, b.dtype), to_device(st.v_new, b.dtype)
    q = to_device(b.q, b.dtype)
    h.append_rope(q if with_q else None, kn, vn, k, v, theta)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(to_host_bits(v, b.dtype)), _bytes(ref_v)), f"{what}: V pool"
    got_k = to_host_bits(k, b.dtype)
    changed = _bits(ref_k, b.dtype) != _bits(st.k_before, b.dtype)
    assert changed.sum() == k_rot.size, "every new K value lands in a poisoned slot"
    assert np.array_equal(_bits(got_k, b.dtype)[~changed], _bits(ref_k, b.dtype)[~changed]), \
        f"{what}: K pool outside the new slots"
    gk = W.storage_to_f32(got_k, b.dtype).astype(np.float64)[changed]
    rk = W.storage_to_f32(ref_k, b.dtype).astype(np.float64)[changed]
    assert (np.abs(gk - rk) <= _rope_tol(rk, b.dtype) + _ulp(rk, b.dtype) * (b.dtype != "f32")).all(), \
        f"{what}: rotated K, max err {np.abs(gk - rk).max()}"
    gq = W.storage_to_f32(to_host_bits(q, b.dtype), b.dtype).astype(np.float64)
    if with_q:
        err = np.abs(gq - q_rot)
        assert (err <= _rope_tol(q_rot, b.dtype)).all(), f"{what}: rotated Q, max err {err.max()}"
    else:
        assert np.array_equal(_bits(to_host_bits(q, b.dtype), b.dtype), _bits(b.q, b.dtype))
    return h, q, k, v, ref_k, ref_v, q_rot


ROPE_CASES = [
    dict(kv=[80, 17, 33, 5, 1], qo=[37, 1, 0, 5, 1], Hq=14, Hkv=2, D=64, P=16, dtype="bf16", theta=1e4),
    dict(kv=[16, 17, 64, 65, 300], Hq=12, Hkv=2, D=128, P=64, dtype="f16", theta=1e6),
    dict(kv=[50, 20, 256], qo=[50, 1, 256], Hq=8, Hkv=1, D=64, P=256, dtype="f32", theta=500.0),
    dict(kv=[32773, 40000, 7], Hq=8, Hkv=1, D=128, P=256, dtype="bf16", theta=1e6),
]


@pytest.mark.parametrize("case", ROPE_CASES,
                         ids=lambda c: f"{c['dtype']}-D{c['D']}-P{c['P']}-theta{c['theta']:g}-{'ragged' if 'qo' in c else 'decode'}")
def test_append_rope_variants(case):
    b = W.make_batch(case["kv"], case.get("qo"), num_qo_heads=case["Hq"], num_kv_heads=case["Hkv"],
                     head_dim=case["D"], page_size=case["P"], dtype=case["dtype"],
                     num_pages=sum(-(-k // case["P"]) for k in case["kv"]) + 6, seed=37,
                     keep_dense=True)
    _check_rope(b, case["theta"], what=str(case))


@pytest.mark.parametrize("name", sorted(W.WORKLOADS))
def test_append_rope_workloads_full_size(name):
    _check_rope(W.WORKLOADS[name](keep_dense=True), 1e4)


def test_append_rope_without_q_leaves_q_alone():
    b = W.make_batch([40, 3, 300], [4, 1, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                     page_size=16, dtype="bf16", seed=38, keep_dense=True)
    _check_rope(b, 1e4, with_q=False, what="q=NULL")


def test_attention_after_append_rope_matches_oracle():
    """The attention call that follows reads the rotated rows: against the oracle's
    attention over its own rotated (and rounded) queries and pools."""
    import dataclasses
    import torch
    b = W.make_batch([300, 17, 1536, 100], [1, 1, 512, 1], num_qo_heads=14, num_kv_heads=2,
                     head_dim=64, page_size=16, dtype="bf16", seed=39, num_pages=200, keep_dense=True)
    h, q, k, v, ref_k, ref_v, q_rot = _check_rope(b, 1e6, what="then attention")
    out = torch.full(q.shape, float("nan"), dtype=torch_dtype(b.dtype), device="cuda:0")
    h.run(q, k, v, out)
    torch.cuda.synchronize()
    bb = dataclasses.replace(b, q=W.to_storage(q_rot.astype(np.float32), b.dtype), k_pool=ref_k, v_pool=ref_v)
    ref_out, _ = oracle.attention(bb)
    compare(bb, out, None, ref_out, None, "attention after append+rope")


def test_append_rope_graph_replay_across_replans():
    """append_rope captured once in a HIP graph; each replay after a new plan (other page ids
    and lengths of the same shape) rotates by the new positions into the new slots."""
    import torch
    b1 = W.make_batch([40, 300, 17, 2], [1, 1, 9, 1], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                      page_size=16, dtype="bf16", seed=63, num_pages=64, keep_dense=True)
    b2 = W.relabel_pages(b1, W.rng_for(64, 0, 0).permutation(b1.num_pages))
    theta = 1e4
    announce("append+rope graph replay across re-plans")
    h = fl.PagedAttention(config_for(b1), device=0)
    h.plan(b1.qo_indptr, b1.kv_indptr, b1.kv_indices, b1.last_page_len, b1.num_pages,
           causal=True, sm_scale=b1.sm_scale)
    st1, st2 = W.append_step(b1), W.append_step(b2)
    k, v = to_device(st1.k_before, "bf16"), to_device(st1.v_before, "bf16")
    kn, vn = to_device(st1.k_new, "bf16"), to_device(st1.v_new, "bf16")
    q = to_device(b1.q, "bf16")
    h.append_rope(q, kn, vn, k, v, theta)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        h.append_rope(q, kn, vn, k, v, theta)
    pos = oracle.append_positions(b1.qo_indptr, b1.kv_indptr, b1.last_page_len, b1.page_size)
    q_rot = oracle.rope(2, b1.q, pos, theta)
    k_rot = W.to_storage(oracle.rope(2, st1.k_new, pos, theta).astype(np.float32), "bf16")
    for rep in range(4):
        bb, st = (b2, st2) if rep % 2 else (b1, st1)
        h.plan(bb.qo_indptr, bb.kv_indptr, bb.kv_indices, bb.last_page_len, bb.num_pages,
               causal=True, sm_scale=bb.sm_scale)
        k.copy_(to_device(st.k_before, "bf16"))
        v.copy_(to_device(st.v_before, "bf16"))
        q.copy_(to_device(bb.q, "bf16"))
        g.replay()
        torch.cuda.synchronize()
        # same lengths, so the same positions; only the slots differ
        ref_k, ref_v = oracle.kv_append(bb, k_rot, st.v_new, st.k_before, st.v_before)
        assert np.array_equal(_bytes(to_host_bits(v, "bf16")), _bytes(ref_v)), f"replay {rep}: V"
        gk = W.storage_to_f32(to_host_bits(k, "bf16"), "bf16").astype(np.float64)
        rk = W.storage_to_f32(ref_k, "bf16").astype(np.float64)
        both_nan = np.isnan(gk) & np.isnan(rk)   # unused slots hold the poison in both
        with np.errstate(invalid="ignore"):
            ok = np.abs(gk - rk) <= 2 * _ulp(rk, "bf16") + 1e-6 * (1 + np.abs(rk))
        assert (both_nan | ok).all(), f"replay {rep}: K"
        gq = W.storage_to_f32(to_host_bits(q, "bf16"), "bf16").astype(np.float64)
        assert (np.abs(gq - q_rot) <= _rope_tol(q_rot, "bf16")).all(), f"replay {rep}: Q"
