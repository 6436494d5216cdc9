"""Benchmark: paged GQA decode attention on one MI355X.

A step is one pass of the whole hot path over one synthetic batch: one plan (host
validation and partitioning plus the metadata copy) and one run per layer, each layer
reading its own K/V pool, so consecutive calls never hit data a previous call left in the
caches. Inputs are resident in device memory before the timed region starts.

Reported (one JSON line):
  value        whole-job KV read rate in GB/s: algorithmic K+V bytes of all timed calls
               divided by the wall time of the timed steps (plans included)
  us_per_call  mean duration of one layer's run() measured with HIP events on the stream
               the kernels are launched on
  roofline     the attention kernel against the 8 TB/s HBM peak
  cpu_baseline the CPU oracle on the host's cores, on the same batch

Usage: python bench.py [--workload saturated_decode] [--steps 20] [--warmup 3]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged GQA decode: µs/call and KV GB/s (% HBM peak), 128 seqs×300 ctx"
LAYERS = {"tiny_decode": 24, "saturated_decode": 24, "ragged_mixed_step": 24,
          "mixed_length_decode": 28, "long_context_skew": 28}
KERNEL_SRC = os.path.join(ROOT, "paged_kv_gqa_plan_amd", "csrc", "attn_kernels.hip")
PLAN_SRC = os.path.join(ROOT, "paged_kv_gqa_plan_amd", "csrc", "plan.cpp")


def source_hash() -> str:
    h = hashlib.sha256()
    for p in (KERNEL_SRC, PLAN_SRC):
        h.update(open(p, "rb").read())
    return h.hexdigest()[:16]


def traffic_from_profile(workload: str):
    """HBM bytes per attention launch from the committed counter summary, if it was taken
    on the current kernel and planner sources; else None."""
    p = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    if not os.path.exists(p):
        return None
    try:
        d = json.loads(open(p).read())
    except ValueError:
        return None
    if d.get("source_hash") != source_hash():
        return None
    return d.get("hbm_bytes_per_launch")


def device_tensor(arr, dtype):
    import numpy as np
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        return torch.from_numpy(a.view(np.int16)).view(torch.bfloat16).to("cuda:0")
    return torch.from_numpy(a).to("cuda:0")


def cpu_baseline(b, gpu_out0, budget_s: float):
    """The oracle as it stands, on all host threads, on the same batch, repeated for about
    budget_s seconds; also compares layer 0's GPU output with it."""
    import numpy as np
    import torch

    import oracle
    oracle.load()
    t0 = time.perf_counter()
    ref, _ = oracle.attention(b)
    first = time.perf_counter() - t0
    calls, t0 = 0, time.perf_counter()
    while True:
        oracle.attention(b)
        calls += 1
        el = time.perf_counter() - t0
        if el >= budget_s or (calls >= 3 and el + el / calls > 1.5 * budget_s):
            break
    per_call = el / calls
    got = gpu_out0.to(torch.float64).cpu().numpy()
    err = float(np.abs(got - ref).max())
    return {"value": round(b.kv_bytes() / per_call / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle",
            "sample": f"the full {b.name} batch (one layer call), {calls} repeats over "
                      f"{el:.1f} s, {per_call * 1e3:.2f} ms per call (first call {first * 1e3:.1f} ms)",
            "ms_per_call": round(per_call * 1e3, 4),
            "gpu_vs_oracle_max_abs": err}


def copy_calibration(mib: int):
    """A plain device copy of known size (for scaling the HBM byte counters)."""
    import torch
    n = mib * (1 << 20) // 4
    x = torch.ones(n, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)
    for _ in range(3):
        y.copy_(x)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calibration_bytes_read": n * 4, "bytes_written": n * 4}), flush=True)


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="saturated_decode", choices=sorted(LAYERS))
    ap.add_argument("--layers", type=int, default=0, help="per-layer pools (0: 24 or 28 by workload)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="planner slice override (0 = automatic)")
    ap.add_argument("--groups-per-cu", type=int, default=0)
    ap.add_argument("--min-group-tokens", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0, help="wavefronts per workgroup (4 or 8; 0 = default)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the attention path runs on a single device; no multi-GPU mode exists)",
              file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return 0

    import numpy as np
    import torch

    import paged_kv_gqa_plan_amd as fl
    import workloads as W

    fl.load_library()
    b = W.WORKLOADS[args.workload](seed=args.seed)
    L = args.layers or LAYERS[args.workload]
    kv_bytes = b.kv_bytes()

    q = device_tensor(b.q, b.dtype)
    k0 = device_tensor(b.k_pool, b.dtype)
    v0 = device_tensor(b.v_pool, b.dtype)
    tdt = k0.dtype
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(1000 + args.seed)
    ks, vs = [k0], [v0]
    for _ in range(1, L):
        ks.append(torch.randn(k0.shape, dtype=tdt, device="cuda:0", generator=gen))
        vs.append(torch.randn(v0.shape, dtype=tdt, device="cuda:0", generator=gen))
    outs = [torch.empty(q.shape, dtype=tdt, device="cuda:0") for _ in range(L)]

    cfg = fl.make_config(b.num_qo_heads, b.num_kv_heads, b.head_dim, b.page_size, b.dtype,
                         b.batch_size, b.rows, int(b.kv_indptr[-1]),
                         groups_per_cu=args.groups_per_cu, min_group_tokens=args.min_group_tokens,
                         waves_per_group=args.waves)
    h = fl.PagedAttention(cfg, device=0)
    stream = torch.cuda.current_stream()

    def plan():
        h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
               causal=b.causal, sm_scale=b.sm_scale, num_splits=args.splits)

    def step(evs=None):
        plan()
        for l in range(L):
            if evs is not None:
                evs[l][0].record(stream)
            h.run(q, ks[l], vs[l], outs[l])
            if evs is not None:
                evs[l][1].record(stream)

    for _ in range(max(args.warmup, 1)):
        step()
    torch.cuda.synchronize()
    n_items, n_groups, max_splits, ws_bytes = h.info()

    evs = [[(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            for _ in range(L)] for _ in range(args.steps)]
    plan_s = 0.0
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for s in range(args.steps):
        step(evs[s])
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    call_ms = [a.elapsed_time(e) for row in evs for (a, e) in row]
    # plan host time, measured on its own after the timed region
    for _ in range(10):
        t1 = time.perf_counter()
        plan()
        plan_s += time.perf_counter() - t1
    torch.cuda.synchronize()
    plan_us = plan_s / 10 * 1e6

    us_call = float(np.mean(call_ms)) * 1e3
    us_call_med = float(np.median(call_ms)) * 1e3
    value = kv_bytes * L * args.steps / wall / 1e9
    achieved = kv_bytes / (us_call * 1e-6) / 1e9
    traffic = traffic_from_profile(args.workload)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall / args.steps * 1e3, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": b.dtype,
        "data": "synthetic",
        "config": {"workload": args.workload, "batch": b.batch_size, "query_rows": b.rows,
                   "kv_tokens": int(b.kv_lens.sum()), "num_qo_heads": b.num_qo_heads,
                   "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
                   "page_size": b.page_size, "pool_pages": b.num_pages, "layers": L,
                   "seed": args.seed, "splits": args.splits, "waves": args.waves,
                   "parallelism": "single GPU"},
        "us_per_call": round(us_call, 3),
        "us_per_call_median": round(us_call_med, 3),
        "kv_bytes_per_call": kv_bytes,
        "hbm_peak_frac_per_call": round(achieved / HBM_PEAK_GBS, 4),
        "attention_us_per_step": round(us_call * L, 2),
        "plan_host_us": round(plan_us, 2),
        "work_items": n_items,
        "workgroups": n_groups,
        "max_splits": max_splits,
        "workspace_bytes": ws_bytes,
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    if not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline(b, outs[0], args.cpu_budget)
    print(json.dumps(res), flush=True)
    h.close()
    return 0


if __name__ == "__main__":
    sys.exit(main())
