"""The allocation-free run (fl_paged_attn_run_noalloc) against fl_paged_attn_run.

A host-only handle (created and planned without any HIP call) runs through the library's
fixed device scratch array; a device handle with the same configuration and plan runs the
ordinary entry point. Same plan, same kernel, same launch: the outputs must be identical
bit for bit, and both within the oracle's bar. Two calls in a row, the second on a smaller
batch (the array keeps the first call's contents), then a step with a prefill chunk."""
import numpy as np
import pytest

import oracle
import paged_kv_gqa_plan_amd as fl
import workloads as W
from gpu_helpers import announce, compare, config_for, to_device, to_host_bits, torch_dtype

pytestmark = pytest.mark.gpu


def _run_both(b, cfg_kw):
    import torch
    num_cus = torch.cuda.get_device_properties(0).multi_processor_count
    dev = fl.PagedAttention(config_for(b, num_cus=num_cus, **cfg_kw), device=0)
    host = fl.PagedAttention(config_for(b, num_cus=num_cus, **cfg_kw), device=-1)
    for h in (dev, host):
        h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
               causal=b.causal, sm_scale=b.sm_scale)
    assert dev.launch() == host.launch() and dev.info() == host.info()
    q, k, v = to_device(b.q, b.dtype), to_device(b.k_pool, b.dtype), to_device(b.v_pool, b.dtype)
    outs = []
    for h, fn in ((dev, "run"), (host, "run_noalloc")):
        out = torch.full(q.shape, float("nan"), dtype=torch_dtype(b.dtype), device="cuda:0")
        lse = torch.full(q.shape[:2], float("nan"), dtype=torch.float32, device="cuda:0")
        getattr(h, fn)(q, k, v, out, lse)
        torch.cuda.synchronize()
        outs.append((out, lse))
    ref_out, ref_lse = oracle.attention(b)
    for (out, lse), what in zip(outs, ("run", "run_noalloc")):
        compare(b, out, lse, ref_out, ref_lse, f"{b.name} {what}")
    assert np.array_equal(to_host_bits(outs[0][0], b.dtype), to_host_bits(outs[1][0], b.dtype))
    assert np.array_equal(outs[0][1].cpu().numpy().view(np.uint32), outs[1][1].cpu().numpy().view(np.uint32))
    assert dev.refused_launches() == 0
    return dev.info()


def test_noalloc_matches_run_on_two_calls_then_a_prefill_step():
    announce("allocation-free run: mixed-length decode (cut blocks merged), full size")
    info = _run_both(W.mixed_length_decode(), {})
    assert info[2] > 1 and info[3] > 0          # pieces merged through the scratch partials
    announce("allocation-free run: tiny decode (a smaller second call)")
    _run_both(W.tiny_decode(), {})
    announce("allocation-free run: ragged mixed step (prefill chunk, two workgroups per unit)")
    _run_both(W.ragged_mixed_step(), {})
