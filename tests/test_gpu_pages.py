"""GPU parity of freed-page poisoning, and a serving loop over the page allocator.

Poisoning is checked bit-exactly against the oracle (every element of a listed page
becomes the type's quiet NaN, nothing else changes). The serving loop drives the library's
allocator (whole-page reservation, prefix pages shared by reference count, a page per
decode request crossing a page boundary, release and poisoning of finished requests'
pages), and each step appends the step's new K/V rows and runs attention on the GPU; the
outputs are compared with the oracle on a host mirror of the pools (same appends, same
poisoning), and the pools themselves are compared byte for byte at the end.
"""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_plan_amd as fl
import workloads as W
from gpu_helpers import announce, compare, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu


def _bytes(a):
    return np.ascontiguousarray(a).view(np.uint8)


@pytest.mark.parametrize("dtype,P,Hkv,D", [("bf16", 16, 2, 64), ("f16", 256, 2, 128),
                                           ("f32", 64, 1, 64), ("bf16", 16, 8, 128)])
def test_poison_matches_oracle(dtype, P, Hkv, D):
    import torch
    announce(f"poison {dtype} P={P} Hkv={Hkv} D={D}")
    b = W.make_batch([5 * P, 3], num_qo_heads=Hkv, num_kv_heads=Hkv, head_dim=D, page_size=P,
                     dtype=dtype, num_pages=12, seed=71, poison=False)
    ids = np.array([3, 11, 0, 3, 7], np.int32)    # a duplicate, both ends of the pool
    ref_k, ref_v = oracle.paged_kv_poison(b.dtype_code, ids, b.k_pool, b.v_pool)
    k, v = to_device(b.k_pool, dtype), to_device(b.v_pool, dtype)
    fl.fl_paged_kv_poison(dtype, P, Hkv, D, b.num_pages, ids, k.data_ptr(), v.data_ptr(),
                          torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(to_host_bits(k, dtype)), _bytes(ref_k))
    assert np.array_equal(_bytes(to_host_bits(v, dtype)), _bytes(ref_v))


def test_poison_many_pages_k_only_and_errors():
    import torch
    announce("poison: 700 ids over several launches, K pool only, error paths")
    b = W.make_batch([16] * 900, num_qo_heads=2, num_kv_heads=2, head_dim=64, page_size=16,
                     dtype="bf16", num_pages=1000, seed=72, poison=False)
    ids = W.rng_for(72, 0, 9).permutation(1000)[:700].astype(np.int32)
    ref_k, _ = oracle.paged_kv_poison(b.dtype_code, ids, b.k_pool)
    k, v = to_device(b.k_pool, "bf16"), to_device(b.v_pool, "bf16")
    fl.fl_paged_kv_poison("bf16", 16, 2, 64, 1000, ids, k.data_ptr(), None)
    torch.cuda.synchronize()
    assert np.array_equal(_bytes(to_host_bits(k, "bf16")), _bytes(ref_k))
    assert np.array_equal(_bytes(to_host_bits(v, "bf16")), _bytes(b.v_pool))
    for bad in (dict(ids=[1000]), dict(ids=[-1]), dict(ptr=2)):
        with pytest.raises(fl.FlError) as e:
            fl.fl_paged_kv_poison("bf16", 16, 2, 64, 1000, bad.get("ids", [1]),
                                  k.data_ptr() + bad.get("ptr", 0), None)
        assert e.value.status == fl.FL_ERR_INVALID_ARG
    assert np.array_equal(_bytes(to_host_bits(k, "bf16")), _bytes(ref_k))


def test_serving_loop_over_the_allocator():
    import torch
    Hq, Hkv, D, P, N, dtype = 14, 2, 64, 16, 160, "bf16"
    rng = np.random.default_rng(81)
    vals = W.rng_for(81, 0, 3)
    sd = W.storage_np_dtype(dtype)
    pool = fl.PagePool(N, P)
    host_k = np.full((N, P, Hkv, D), W.poison_value(dtype), dtype=sd)
    host_v = host_k.copy()
    dev_k, dev_v = to_device(host_k, dtype), to_device(host_v, dtype)
    # page-table entries can exceed the pool: shared prefix pages appear once per holder
    h = fl.PagedAttention(fl.make_config(Hq, Hkv, D, P, dtype, 64, 4096, 4 * N), device=0)
    stream = torch.cuda.current_stream().cuda_stream
    reqs = {}       # id -> {"pages": [...], "kv": tokens written, "left": decode steps left}
    nxt, shared_seen, freed_total = 0, 0, 0
    for step in range(40):
        # ---- finish some requests: release, poison what became free ----------------
        for r in [r for r in reqs if reqs[r]["left"] == 0]:
            freed = pool.release(reqs.pop(r)["pages"])
            if freed.size:
                freed_total += freed.size
                fl.fl_paged_kv_poison(dtype, P, Hkv, D, N, freed, dev_k.data_ptr(), dev_v.data_ptr(), stream)
                host_k, host_v = oracle.paged_kv_poison(W.DTYPE_CODES[dtype], freed, host_k, host_v)
        # ---- this step's rows: decodes grow by one token, arrivals bring a prompt --------
        batch = []      # (request, qo_len)
        for r, st in reqs.items():
            if st["kv"] % P == 0:
                got = pool.alloc(1) if pool.info()[0] else None
                if got is None:
                    continue        # no room this step
                st["pages"].append(int(got[0]))
            batch.append((r, 1))
        for _ in range(int(rng.integers(0, 3))):
            prompt = int(rng.integers(1, 120))
            prefix = []
            donors = [r for r, s in reqs.items() if s["kv"] >= 2 * P]
            if donors and rng.random() < 0.5:
                d = reqs[donors[int(rng.integers(len(donors)))]]
                full = d["kv"] // P
                k_pages = int(rng.integers(1, full + 1))
                if k_pages * P < prompt:    # adoption never covers the last prompt token
                    prefix = d["pages"][:k_pages]
            if pool.info()[0] < -(-(prompt - len(prefix) * P) // P):
                continue
            if prefix:
                pool.retain(prefix)
                shared_seen += 1
            own = pool.reserve(prompt - len(prefix) * P).tolist()
            reqs[nxt] = {"pages": list(prefix) + own, "kv": len(prefix) * P,
                         "left": int(rng.integers(1, 12)), "prompt": prompt}
            batch.append((nxt, prompt - len(prefix) * P))
            nxt += 1
        if not batch:
            continue
        # ---- plan, append, attend ---------------------------------------------------------
        qo = np.zeros(len(batch) + 1, np.int32)
        kv_indptr = np.zeros(len(batch) + 1, np.int32)
        indices, last = [], []
        for j, (r, ql) in enumerate(batch):
            st = reqs[r]
            kv_len = st["kv"] + ql
            npg = -(-kv_len // P)
            qo[j + 1] = qo[j] + ql
            kv_indptr[j + 1] = kv_indptr[j] + npg
            indices += st["pages"][:npg]
            last.append(kv_len - (npg - 1) * P)
        indices = np.array(indices, np.int32)
        last = np.array(last, np.int32)
        rows = int(qo[-1])
        k_new = W.to_storage(vals.standard_normal((rows, Hkv, D), dtype=np.float32), dtype)
        v_new = W.to_storage(vals.standard_normal((rows, Hkv, D), dtype=np.float32), dtype)
        q = W.to_storage(vals.standard_normal((rows, Hq, D), dtype=np.float32), dtype)
        announce(f"serving step {step}: {len(batch)} requests, {rows} rows, pages held {pool.info()[1]}")
        h.plan(qo, kv_indptr, indices, last, N, causal=True)
        qd, kn, vn = to_device(q, dtype), to_device(k_new, dtype), to_device(v_new, dtype)
        out = torch.full((rows, Hq, D), float("nan"), dtype=torch_dtype(dtype), device="cuda:0")
        h.append(kn, vn, dev_k, dev_v)
        h.run(qd, dev_k, dev_v, out)
        torch.cuda.synchronize()
        host_k, host_v = oracle.paged_kv_append(2, qo, kv_indptr, indices, last, N, Hkv, D, P,
                                                k_new, v_new, host_k, host_v)
        ref, _ = oracle.paged_attention(W.DTYPE_CODES[dtype], qo, kv_indptr, indices, last, N, Hq,
                                        Hkv, D, P, q, host_k, host_v, causal=True)
        bb = W.Batch(name="serving", dtype=dtype, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     page_size=P, num_pages=N, causal=True, sm_scale=D ** -0.5, qo_indptr=qo,
                     kv_indptr=kv_indptr, kv_indices=indices, last_page_len=last, q=q,
                     k_pool=host_k, v_pool=host_v, kv_lens=(np.diff(kv_indptr) - 1) * P + last,
                     qo_lens=np.diff(qo))
        compare(bb, out, None, ref, None, f"serving step {step}")
        for r, ql in batch:
            reqs[r]["kv"] += ql
            reqs[r]["left"] -= 1
    assert shared_seen > 0 and freed_total > 0
    assert np.array_equal(_bytes(to_host_bits(dev_k, dtype)), _bytes(host_k))
    assert np.array_equal(_bytes(to_host_bits(dev_v, dtype)), _bytes(host_v))
