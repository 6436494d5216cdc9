"""HIP-graph capture of run() and the append calls: the plan refreshes the handle's
persistent metadata in place and every plan of one launch class launches identically, so a
graph captured once replays correctly after every later plan of that class (new page ids,
other lengths, requests joining and leaving)."""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_plan_amd as fl
import workloads as W
from gpu_helpers import DeviceBatch, announce, compare, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu


def test_graph_replay_matches_eager_across_replans():
    import torch
    # long and short histories: cut row blocks, merge tickets and whole blocks all appear
    lens = [5000, 37, 300, 2048, 1, 777, 4100, 16]
    b1 = W.make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=128, page_size=64,
                      dtype="f16", seed=41, num_pages=260)
    b2 = W.relabel_pages(b1, W.rng_for(42, 0, 0).permutation(b1.num_pages))
    ref1 = oracle.attention(b1)
    announce("graph replay across re-plans")
    d = DeviceBatch(b1)
    eager, eager_lse = d.run()
    eager_bits = to_host_bits(eager, "f16").copy()
    compare(b1, eager, eager_lse, *ref1, "eager")
    assert d.h.info()[2] > 1  # some row block was cut into pieces

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        d.h.run(d.q, d.k, d.v, d.out, d.lse)
    k1, v1 = d.k.clone(), d.v.clone()
    k2 = torch.from_numpy(b2.k_pool).to("cuda:0")
    v2 = torch.from_numpy(b2.v_pool).to("cuda:0")
    for rep in range(4):
        use2 = rep % 2 == 1
        d.k.copy_(k2 if use2 else k1)
        d.v.copy_(v2 if use2 else v1)
        bb = b2 if use2 else b1
        d.h.plan(bb.qo_indptr, bb.kv_indptr, bb.kv_indices, bb.last_page_len, bb.num_pages,
                 causal=bb.causal, sm_scale=bb.sm_scale)
        d.out.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        # the same lengths give the same plan, so the result is bit-identical to eager
        assert np.array_equal(to_host_bits(d.out, "f16"), eager_bits), f"replay {rep}"
        compare(bb, d.out, d.lse, *ref1, f"replay {rep}")
        x = torch.randn(1 << 20, device="cuda:0")  # unrelated eager work between replays
        float(x.sum())
        torch.cuda.synchronize()


def _serving_graph_case(Hq, Hkv, D, P, dtype, seed, steps=36):
    """One HIP graph captured on the first decode step and replayed on every later decode
    step of an allocator-driven serving loop: histories grow by one token per step,
    requests finish (their pages poisoned) and join (prefilled eagerly between decode steps,
    sometimes adopting a running request's prefix pages). The graph holds, per layer, the
    KV append and attention: layer 0 as two launches, layer 1 as the one-launch
    run_append. Every replay is checked against the oracle on a host mirror of the pools.
    After a prefill plan (another launch class) a replayed attention launch must refuse:
    no output written, one refusal counted."""
    import torch
    N, L = 800, 2
    max_batch, max_rows = 48, 1024
    rng = np.random.default_rng(seed)
    vals = W.rng_for(seed, 0, 3)
    code = W.DTYPE_CODES[dtype]
    elem = 4 if dtype == "f32" else 2
    td = torch_dtype(dtype)
    pool = fl.PagePool(N, P)
    host_k = [np.full((N, P, Hkv, D), W.poison_value(dtype), dtype=W.storage_np_dtype(dtype))
              for _ in range(L)]
    host_v = [x.copy() for x in host_k]
    dev_k = [to_device(x, dtype) for x in host_k]
    dev_v = [to_device(x, dtype) for x in host_v]
    h = fl.PagedAttention(fl.make_config(Hq, Hkv, D, P, dtype, max_batch, max_rows, 4 * N), device=0)
    stream = torch.cuda.current_stream().cuda_stream
    # static decode buffers, sized for the largest decode step
    sq = torch.zeros((max_batch, Hq, D), dtype=td, device="cuda:0")
    skn = torch.zeros((max_batch, Hkv, D), dtype=td, device="cuda:0")
    svn = torch.zeros((max_batch, Hkv, D), dtype=td, device="cuda:0")
    sout = [torch.zeros((max_batch, Hq, D), dtype=td, device="cuda:0") for _ in range(L)]
    slse = [torch.zeros((max_batch, Hq), dtype=torch.float32, device="cuda:0") for _ in range(L)]

    def layers():
        h.append(skn, svn, dev_k[0], dev_v[0])
        h.run(sq, dev_k[0], dev_v[0], sout[0], slse[0])
        h.run_append(sq, skn, svn, dev_k[1], dev_v[1], sout[1], slse[1])

    def metadata(batch, reqs):
        qo = np.zeros(len(batch) + 1, np.int32)
        kvp = np.zeros(len(batch) + 1, np.int32)
        ids, last = [], []
        for j, (r, ql) in enumerate(batch):
            kv_len = reqs[r]["kv"] + ql
            npg = -(-kv_len // P)
            qo[j + 1] = qo[j] + ql
            kvp[j + 1] = kvp[j] + npg
            ids += reqs[r]["pages"][:npg]
            last.append(kv_len - (npg - 1) * P)
        return qo, kvp, np.array(ids, np.int32), np.array(last, np.int32)

    def oracle_step(l, qo, kvp, ids, last, q, kn, vn):
        host_k[l], host_v[l] = oracle.paged_kv_append(elem, qo, kvp, ids, last, N, Hkv, D, P, kn, vn,
                                                      host_k[l], host_v[l])
        ref, ref_lse = oracle.paged_attention(code, qo, kvp, ids, last, N, Hq, Hkv, D, P, q, host_k[l],
                                              host_v[l], causal=True)
        bb = W.Batch(name="serving", dtype=dtype, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                     page_size=P, num_pages=N, causal=True, sm_scale=D ** -0.5, qo_indptr=qo,
                     kv_indptr=kvp, kv_indices=ids, last_page_len=last, q=q, k_pool=host_k[l],
                     v_pool=host_v[l], kv_lens=(np.diff(kvp) - 1) * P + last, qo_lens=np.diff(qo))
        return bb, ref, ref_lse

    def rnd(shape):
        return W.to_storage(vals.standard_normal(shape, dtype=np.float32), dtype)

    reqs, nxt = {}, 0
    graph, refusal_checked, replays, joined, shared = None, False, 0, 0, 0
    decode_classes = set()
    for step in range(steps):
        # ---- finish: release, poison what became free --------------------------------
        for r in [r for r in reqs if reqs[r]["left"] == 0]:
            freed = pool.release(reqs.pop(r)["pages"])
            if freed.size:
                for l in range(L):
                    fl.fl_paged_kv_poison(dtype, P, Hkv, D, N, freed, dev_k[l].data_ptr(),
                                          dev_v[l].data_ptr(), stream)
                    host_k[l], host_v[l] = oracle.paged_kv_poison(code, freed, host_k[l], host_v[l])
        # ---- join: prefill the prompts eagerly (a plan of the other kind) -------------------
        pre = []
        for _ in range(int(rng.integers(0, 4)) if step else 6):
            if len(reqs) >= max_batch - 1:
                break
            prompt = int(rng.integers(1, 200))
            prefix = []
            donors = [r for r, s in reqs.items() if s["kv"] >= 2 * P]
            if donors and rng.random() < 0.4:
                d = reqs[donors[int(rng.integers(len(donors)))]]
                k_pages = int(rng.integers(1, d["kv"] // P + 1))
                if k_pages * P < prompt:       # adoption never covers the last prompt token
                    prefix = d["pages"][:k_pages]
            if pool.info()[0] < -(-(prompt - len(prefix) * P) // P) + 8:
                break
            if prefix:
                pool.retain(prefix)
                shared += 1
            own = pool.reserve(prompt - len(prefix) * P).tolist()
            reqs[nxt] = {"pages": list(prefix) + own, "kv": len(prefix) * P,
                         "left": int(rng.integers(4, 30))}
            pre.append((nxt, prompt - len(prefix) * P))
            nxt += 1
            joined += 1
        if pre:
            qo, kvp, ids, last = metadata(pre, reqs)
            rows = int(qo[-1])
            # prompts whose new part is a single row make a decode-shaped step (of the decode
            # class); any longer one makes it a prefill step
            prefill = any(ql > 1 for _, ql in pre)
            announce(f"serving graph {dtype} D{D}: step {step} prefill of {len(pre)} prompts, {rows} rows")
            h.plan(qo, kvp, ids, last, N, causal=True)
            if prefill:
                assert h.launch()[1] == 0      # prefill rows: never the one-launch append class
            else:
                decode_classes.add(h.launch()[:3])   # must be the decode steps' launch
            q = rnd((rows, Hq, D))
            qd = to_device(q, dtype)
            for l in range(L):
                kn, vn = rnd((rows, Hkv, D)), rnd((rows, Hkv, D))
                out = torch.full((rows, Hq, D), float("nan"), dtype=td, device="cuda:0")
                h.run_append(qd, to_device(kn, dtype), to_device(vn, dtype), dev_k[l], dev_v[l], out)
                torch.cuda.synchronize()
                bb, ref, _ = oracle_step(l, qo, kvp, ids, last, q, kn, vn)
                compare(bb, out, None, ref, None, f"prefill step {step} layer {l}")
            for r, ql in pre:
                reqs[r]["kv"] += ql
            if graph is not None and not refusal_checked and prefill and fused_one_launch:
                # decode launches replayed under this prefill plan: the one-launch append +
                # attention belongs to another class here and must refuse (nothing written);
                # so must run() where the prefill class differs from the decode class (at
                # head_dim 64, two workgroups per compute unit). Where the two classes are
                # equal, run() would rightly compute this plan, whose rows the static decode
                # buffers cannot hold, so it is not replayed then. (The append launch follows
                # the current plan, so it is not replayed here either.)
                assert h.refused_launches() == 0
                run_differs = h.launch()[0] != decode_class
                assert run_differs == (D == 64)
                for o in sout:
                    o.fill_(float("nan"))
                g_fused.replay()
                if run_differs:
                    g_run.replay()
                assert h.refused_launches() == 1 + run_differs
                assert torch.isnan(sout[1].float()).all()
                assert torch.isnan(sout[0].float()).all()
                refusal_checked = True
        # ---- decode: every live request grows by one token -------------------------------
        batch = []
        for r, st in reqs.items():
            if st["kv"] % P == 0:
                if not pool.info()[0]:
                    continue                      # no free page: this request waits a step
                st["pages"].append(int(pool.alloc(1)[0]))
            batch.append((r, 1))
        qo, kvp, ids, last = metadata(batch, reqs)
        rows = len(batch)
        announce(f"serving graph {dtype} D{D}: step {step} decode of {rows} requests, "
                 f"pages held {pool.info()[1]}")
        h.plan(qo, kvp, ids, last, N, causal=True)
        decode_classes.add(h.launch()[:3])
        q, kn, vn = rnd((rows, Hq, D)), rnd((rows, Hkv, D)), rnd((rows, Hkv, D))
        sq[:rows].copy_(to_device(q, dtype))
        skn[:rows].copy_(to_device(kn, dtype))
        svn[:rows].copy_(to_device(vn, dtype))
        for l in range(L):
            sout[l].fill_(float("nan"))
        if graph is None:
            decode_class = h.launch()[0]
            # run_append is one launch (which a replay under a prefill plan must refuse) up to
            # 16 query heads per kv head; past that it is an append then an attention launch
            fused_one_launch = h.launch()[1] != 0
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                layers()
            g_run = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_run):
                h.run(sq, dev_k[0], dev_v[0], sout[0], slse[0])
            g_fused = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g_fused):
                h.run_append(sq, skn, svn, dev_k[1], dev_v[1], sout[1], slse[1])
        graph.replay()
        torch.cuda.synchronize()
        replays += 1
        for l in range(L):
            bb, ref, ref_lse = oracle_step(l, qo, kvp, ids, last, q, kn, vn)
            compare(bb, sout[l][:rows], slse[l][:rows], ref, ref_lse, f"decode step {step} layer {l}")
            assert torch.isnan(sout[l][rows:].float()).all()   # rows past the plan untouched
        for r, _ in batch:
            reqs[r]["kv"] += 1
            reqs[r]["left"] -= 1
        x = torch.randn(1 << 16, device="cuda:0")   # unrelated eager work between replays
        float(x.sum())
    assert h.refused_launches() == 0
    # (a prefix adoption needs a prompt longer than a page, and prompts stay under 200 tokens)
    assert replays == steps and (refusal_checked or not fused_one_launch) and joined > 10
    assert shared > 0 or P >= 128
    assert len(decode_classes) == 1, decode_classes
    for l in range(L):
        assert np.array_equal(to_host_bits(dev_k[l], dtype).view(np.uint8), host_k[l].view(np.uint8))
        assert np.array_equal(to_host_bits(dev_v[l], dtype).view(np.uint8), host_v[l].view(np.uint8))


def test_graph_replay_across_serving_steps_d64_bf16():
    _serving_graph_case(14, 2, 64, 16, "bf16", seed=301)


def test_graph_replay_across_serving_steps_d128_f16():
    _serving_graph_case(12, 2, 128, 64, "f16", seed=302)


def test_graph_replay_across_serving_steps_g32_p256():
    """32 query heads per kv head (run_append as an append then an attention launch) and
    pages of 256 tokens."""
    _serving_graph_case(32, 1, 128, 256, "bf16", seed=903, steps=48)
