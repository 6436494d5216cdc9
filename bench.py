"""Benchmark: paged GQA decode attention on one MI355X.

A step is one pass of the whole hot path over one synthetic batch: one plan (host
validation and partitioning plus the metadata copy) and one run per layer, each layer
reading its own K/V pool, so consecutive calls never hit data a previous call left in the
caches. Inputs are resident in device memory before the timed region starts. The layer
runs of a step are captured once into a HIP graph and replayed after each plan (the plan
refreshes the handle's persistent metadata in place, so the graph stays valid); --eager
launches them one by one from Python instead.

Reported (one JSON line):
  value        whole-job KV read rate in GB/s: algorithmic K+V bytes of all timed calls
               divided by the wall time of the timed steps (plans included)
  us_per_call  HIP-event time of the step's layer runs on the launch stream, divided by
               the number of layers
  roofline     the attention kernel against the 8 TB/s HBM peak
  floors       the same launch pattern's floors: a plain read of exactly the call's K/V tiles
               with the loads in flight at once, and an empty kernel (read_probe.hip)
  workloads    the other workloads (mixed-length decode, long-context skew, the ragged step
               with one prefill chunk, several chunks in one call), each timed the same way
               with its own floors
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
          "mixed_length_decode": 28, "long_context_skew": 28, "multi_chunk_step": 24}
KERNEL_SRC = os.path.join(ROOT, "paged_kv_gqa_plan_amd", "csrc", "attn_kernels.hip")
PLAN_SRC = os.path.join(ROOT, "paged_kv_gqa_plan_amd", "csrc", "plan.cpp")
INTERNAL_H = os.path.join(ROOT, "paged_kv_gqa_plan_amd", "csrc", "fl_internal.h")  # planner costs, layouts


def code_text(path: str) -> str:
    """The source's code without its comments and blank lines (C and C++ comments; string
    and character literals kept as written), so that a comment edit leaves the hash of the
    kernel and planner sources unchanged."""
    src = open(path, encoding="utf-8").read()
    out, i, n = [], 0, len(src)
    while i < n:
        c = src[i]
        if c in "\"'":  # a literal: copy through its closing quote
            j = i + 1
            while j < n and src[j] != c:
                j += 2 if src[j] == "\\" else 1
            out.append(src[i:j + 1])
            i = j + 1
        elif src.startswith("//", i):
            j = src.find("\n", i)
            i = n if j < 0 else j
        elif src.startswith("/*", i):
            j = src.find("*/", i + 2)
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    lines = (l.rstrip() for l in "".join(out).splitlines())
    return "\n".join(l for l in lines if l)


def source_hash() -> str:
    """Hash of the attention kernel's and the planner's code and their shared header
    (comments excluded), and of the compiler flags the library's build gives them."""
    from paged_kv_gqa_plan_amd import _build
    h = hashlib.sha256()
    for p in (KERNEL_SRC, PLAN_SRC, INTERNAL_H):
        h.update(code_text(p).encode())
    h.update(repr((_build.ARCH, _build.OPT, _build.DEVICE_FLAGS,
                   {s: _build.FILE_FLAGS.get(s, []) for s in ("attn_kernels.hip", "plan.cpp")})).encode())
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
    # the same oracle on one host thread, over a few seconds
    calls1, t1 = 0, time.perf_counter()
    while True:
        oracle.attention(b, num_threads=1)
        calls1 += 1
        el1 = time.perf_counter() - t1
        if el1 >= min(3.0, budget_s) or calls1 >= 1000:
            break
    per_call1 = el1 / calls1
    got = gpu_out0.to(torch.float64).cpu().numpy()
    err = float(np.abs(got - ref).max())
    return {"value": round(b.kv_bytes() / per_call / 1e9, 3), "unit": "GB/s",
            "cores": oracle.max_threads(), "kind": "oracle", "cpu_model": cpu_model(),
            "affinity_cpus": len(os.sched_getaffinity(0)),
            "sample": f"the full {b.name} batch (one layer call), {calls} repeats over "
                      f"{el:.1f} s, {per_call * 1e3:.2f} ms per call (first call {first * 1e3:.1f} ms)",
            "ms_per_call": round(per_call * 1e3, 4),
            "one_thread": {"ms_per_call": round(per_call1 * 1e3, 3),
                           "value": round(b.kv_bytes() / per_call1 / 1e9, 3), "calls": calls1},
            "gpu_vs_oracle_max_abs": err}


def cold_call_us(h, q, k, v, out, stream, flush_mib: int = 1024, reps: int = 5):
    """One layer call after the caches were flushed: a 1 GiB buffer is written (more than the
    256 MB Infinity Cache and the L2s hold), then a single eager call is timed with events on
    the launch stream; median of `reps`."""
    import torch
    junk = torch.empty(flush_mib << 18, dtype=torch.float32, device="cuda:0")
    ts = []
    for _ in range(reps):
        junk.fill_(1.0)
        a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        h.run(q, k, v, out)
        e.record(stream)
        torch.cuda.synchronize()
        ts.append(a.elapsed_time(e) * 1e3)
    del junk
    return sorted(ts)[len(ts) // 2]


def stream_probe_gbs(mib: int = 1024, reps: int = 10):
    """The streaming rate this GPU sustains on a plain device copy of `mib` MiB (bytes read
    plus bytes written per second, median of `reps`): a measured ceiling to set beside the
    8 TB/s specification. (torch's sum reads the same buffer slower than the copy moves
    twice the bytes, so it is no read ceiling.)"""
    import torch
    x = torch.ones(mib << 18, dtype=torch.float32, device="cuda:0")
    y = torch.empty_like(x)

    def median_s(fn):
        fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            a, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            e.record()
            torch.cuda.synchronize()
            ts.append(a.elapsed_time(e) * 1e-3)
        return sorted(ts)[len(ts) // 2]
    return 2 * x.numel() * 4 / median_s(lambda: y.copy_(x)) / 1e9


def time_kv_append(h, b, ks, vs, L: int, stream, replays: int = 20, rope_theta=None):
    """The KV append of the same step: each layer's new K/V rows ([rows, Hkv, D], seeded
    device data) written into that layer's pools by one launch, the L launches captured in
    one HIP graph. Timed after the attention measurement (it overwrites the new tokens'
    slots). Bytes: the new rows read plus the same bytes written, for K and V. With
    rope_theta, the append fused with the rotary embedding (fl_paged_kv_append_rope), whose
    query heads are rotated in place too: their bytes are read and written as well."""
    import torch
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(7)
    shape = (b.rows, b.num_kv_heads, b.head_dim)
    kn = [torch.randn(shape, dtype=ks[0].dtype, device="cuda:0", generator=gen) for _ in range(L)]
    vn = [torch.randn(shape, dtype=ks[0].dtype, device="cuda:0", generator=gen) for _ in range(L)]
    qn = [torch.randn((b.rows, b.num_qo_heads, b.head_dim), dtype=ks[0].dtype, device="cuda:0",
                      generator=gen) for _ in range(L)] if rope_theta else None

    def call(l):
        if rope_theta:
            h.append_rope(qn[l], kn[l], vn[l], ks[l], vs[l], rope_theta)
        else:
            h.append(kn[l], vn[l], ks[l], vs[l])
    for l in range(L):
        call(l)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for l in range(L):
            call(l)
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for a, e in ev:
        a.record(stream)
        g.replay()
        e.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(e) / L * 1e3 for a, e in ev)
    us_med = us[len(us) // 2]
    heads = 2 * b.num_kv_heads + (b.num_qo_heads if rope_theta else 0)
    nbytes = b.rows * heads * b.head_dim * b.elem_bytes * 2
    d = {"us_per_call_median": round(us_med, 3), "bytes_per_call": nbytes,
         "GB_per_s": round(nbytes / (us_med * 1e-6) / 1e9, 2), "rows": b.rows,
         "launch": "hip_graph", "layers": L}
    if rope_theta:
        d["rope_theta"] = rope_theta
    return d


def time_append_attention(h, b, q, ks, vs, outs, L: int, stream, replays: int = 20):
    """A layer's KV append plus its attention, per layer: one fl_paged_attn_run_append call
    (one launch on decode-only 16-bit plans) against fl_paged_kv_append then
    fl_paged_attn_run, each as L calls captured in one HIP graph. Timed after the attention
    measurement (both overwrite the new tokens' slots)."""
    import numpy as np
    import torch
    gen = torch.Generator(device="cuda:0")
    gen.manual_seed(8)
    shape = (b.rows, b.num_kv_heads, b.head_dim)
    kn = [torch.randn(shape, dtype=ks[0].dtype, device="cuda:0", generator=gen) for _ in range(L)]
    vn = [torch.randn(shape, dtype=ks[0].dtype, device="cuda:0", generator=gen) for _ in range(L)]

    def graph_us(body):
        body()
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            body()
        g.replay()
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(replays)]
        for a, e in ev:
            a.record(stream)
            g.replay()
            e.record(stream)
        torch.cuda.synchronize()
        us = sorted(a.elapsed_time(e) / L * 1e3 for a, e in ev)
        return us[len(us) // 2]

    def fused():
        for l in range(L):
            h.run_append(q, kn[l], vn[l], ks[l], vs[l], outs[l])

    def separate():
        for l in range(L):
            h.append(kn[l], vn[l], ks[l], vs[l])
            h.run(q, ks[l], vs[l], outs[l])
    f_us, s_us = graph_us(fused), graph_us(separate)
    one_launch = all(x == 1 for x in np.diff(b.qo_indptr)) and b.dtype != "f32"
    return {"fused_us_per_layer": round(f_us, 3), "separate_us_per_layer": round(s_us, 3),
            "fused_launches_per_layer": 1 if one_launch else 2, "launch": "hip_graph", "layers": L}


def _csv_rows(path):
    import csv
    with open(path, newline="") as f:
        return list(csv.DictReader(f))


def _counter_per_dispatch(dir_, name_has: str, counter: str):
    """Mean per-dispatch value of a rocprofv3 counter (KiB) for kernels whose name contains
    name_has, from <dir>/run_counter_collection.csv."""
    import glob
    vals = []
    for path in glob.glob(os.path.join(dir_, "**", "*counter_collection.csv"), recursive=True):
        for r in _csv_rows(path):
            if name_has in r["Kernel_Name"] and r["Counter_Name"] == counter:
                vals.append(float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no {counter} rows for {name_has!r} under {dir_}")
    return sum(vals) / len(vals), len(vals)


def summarize_profiles(workload: str, kt: str, pf: str, pw: str, cf: str, cw: str, calib_mib: int,
                       commands: str, steps: int, layers: int):
    """Write profiles/attn_kernel_<workload>.md and profiles/traffic_<workload>.txt from
    rocprofv3 CSV output: a kernel-trace run (kt) and FETCH_SIZE / WRITE_SIZE passes of the
    benchmark (pf, pw) and of a plain copy of known size (cf, cw). steps: the timed steps of
    the profiled benchmark command; its last steps * layers attention dispatches are also
    averaged on their own (the earlier ones are warmup steps and first, cold launches)."""
    import glob
    stats = None
    others = []
    for path in glob.glob(os.path.join(kt, "**", "*kernel_stats.csv"), recursive=True):
        for r in _csv_rows(path):
            if "attn_kernel" in r["Name"]:
                stats = r
            else:
                others.append(r)
    if stats is None:
        raise SystemExit(f"no attention kernel in the kernel stats under {kt}")
    durs = []
    for path in glob.glob(os.path.join(kt, "**", "*kernel_trace.csv"), recursive=True):
        rows = [r for r in _csv_rows(path) if "attn_kernel" in r["Kernel_Name"]]
        rows.sort(key=lambda r: int(r["Start_Timestamp"]))
        durs += [(int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) / 1e3 for r in rows]
    layers = layers or LAYERS[workload]
    timed = durs[-steps * layers:] if steps > 0 and len(durs) >= steps * layers else []
    fetch, nf = _counter_per_dispatch(pf, "attn_kernel", "FETCH_SIZE")
    write, nw = _counter_per_dispatch(pw, "attn_kernel", "WRITE_SIZE")
    cfetch, _ = _counter_per_dispatch(cf, "copyBuffer", "FETCH_SIZE")
    cwrite, _ = _counter_per_dispatch(cw, "copyBuffer", "WRITE_SIZE")
    known_kib = calib_mib * 1024.0
    fscale, wscale = known_kib / cfetch, known_kib / cwrite
    hbm_bytes = (fetch * fscale + write * wscale) * 1024.0
    import workloads as W
    b = W.WORKLOADS[workload]()
    algo = b.kv_bytes()
    avg_ns = float(stats["AverageNs"])
    d = {"workload": workload, "source_hash": source_hash(),
         "hbm_bytes_per_launch": round(hbm_bytes),
         "fetch_kib_per_dispatch": fetch, "write_kib_per_dispatch": write,
         "fetch_scale": fscale, "write_scale": wscale,
         "calibration": f"plain device copy of {calib_mib} MiB: FETCH_SIZE {cfetch:.1f} KiB, "
                        f"WRITE_SIZE {cwrite:.1f} KiB per dispatch",
         "kernel_avg_us": avg_ns / 1e3, "algorithmic_kv_bytes": algo}
    timed_line = []
    if timed:
        d["kernel_timed_avg_us"] = sum(timed) / len(timed)
        d["kernel_timed_median_us"] = sorted(timed)[len(timed) // 2]
        d["kernel_timed_dispatches"] = len(timed)
        timed_line = [f"The last {len(timed)} attention dispatches ({steps} timed steps x {layers} "
                      f"layers, from the per-dispatch trace): average {d['kernel_timed_avg_us']:.3f} us, "
                      f"median {d['kernel_timed_median_us']:.3f} us. The average in the table also holds "
                      f"the warmup steps and the first, cold launches.", ""]
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    with open(os.path.join(ROOT, "profiles", f"traffic_{workload}.txt"), "w") as f:
        f.write(json.dumps(d, indent=1) + "\n")
    md = [f"# attention kernel, {workload} ({b.batch_size} requests, {int(b.kv_lens.sum())} cached "
          f"tokens, {b.num_qo_heads}/{b.num_kv_heads} heads, d {b.head_dim}, {b.dtype}, "
          f"page size {b.page_size})", "",
          "Commands (from the repository root on the GPU host):", "", "```", commands.strip(), "```", "",
          "## Kernel trace (rocprofv3 --kernel-trace --stats)", "",
          "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|",
          f"| {stats['Name'][:80]} | {stats['Calls']} | {avg_ns / 1e3:.3f} | "
          f"{float(stats['MinNs']) / 1e3:.3f} | {float(stats['MaxNs']) / 1e3:.3f} |"] + [
          f"| {r['Name'][:80]} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.3f} | "
          f"{float(r['MinNs']) / 1e3:.3f} | {float(r['MaxNs']) / 1e3:.3f} |"
          for r in sorted(others, key=lambda r: -float(r["TotalDurationNs"]))[:6]] + ["",
          "The attention kernel is one launch per layer; stage_copy_kernel copies each plan's "
          "metadata (one launch per step); the other rows are torch's input setup.", ""] + timed_line + [
          f"Algorithmic K+V bytes per call: {algo} -> {algo / avg_ns:.1f} GB/s at the average "
          f"duration ({algo / avg_ns / 8000.0 * 100:.1f}% of 8 TB/s).", "",
          "## HBM traffic (rocprofv3 --pmc, one counter per run)", "",
          f"* FETCH_SIZE {fetch:.1f} KiB per dispatch ({nf} dispatches), scale {fscale:.4f}",
          f"* WRITE_SIZE {write:.1f} KiB per dispatch ({nw} dispatches), scale {wscale:.4f}",
          f"* calibration: {d['calibration']} (the copy reads and writes {calib_mib} MiB each)",
          f"* HBM bytes per launch: {hbm_bytes:.0f} ({hbm_bytes / algo:.3f} x the algorithmic "
          f"K+V bytes)", ""]
    with open(os.path.join(ROOT, "profiles", f"attn_kernel_{workload}.md"), "w") as f:
        f.write("\n".join(md))
    print(json.dumps(d))


SQ_PASS_A = ("SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_ACTIVE_INST_VALU", "SQ_ACTIVE_INST_LDS",
             "SQ_WAIT_INST_ANY", "SQ_WAIT_ANY", "SQ_ACTIVE_INST_ANY", "SQ_INSTS_VALU")
SQ_PASS_B = ("SQ_VALU_MFMA_BUSY_CYCLES", "SQ_INSTS_MFMA", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
             "SQ_ACTIVE_INST_VMEM", "SQ_INSTS_SALU", "SQ_ACTIVE_INST_SCA", "SQ_INSTS_VMEM")
# flops per MFMA instruction of the 16-bit decode tiles: per tile NC = D/32 instructions of
# 16x16x32 (16384 flops) and 2 * D/16 of 16x16x16 (8192 flops), the same 1:4 mix at d 64 and
# 128; the prefill units issue only 16x16x32
FLOPS_PER_MFMA_DECODE = (16384 + 4 * 8192) / 5
FLOPS_PER_MFMA_16X16X32 = 16384


def summarize_sq(workload: str, da: str, db: str, commands: str):
    """Write profiles/sq_<workload>.md from two rocprofv3 --pmc passes of SQ counters."""
    import workloads as W
    b = W.WORKLOADS[workload]()
    c = {}
    for d, names in ((da, SQ_PASS_A), (db, SQ_PASS_B)):
        for n in names:
            c[n], nd = _counter_per_dispatch(d, "attn_kernel", n)
    tp = os.path.join(ROOT, "profiles", f"traffic_{workload}.txt")
    tr = json.loads(open(tp).read()) if os.path.exists(tp) else None
    wc = c["SQ_WAVE_CYCLES"]
    frac = lambda n: c[n] / wc
    lines = [f"# attention kernel, {workload}: SQ counters (rocprofv3 --pmc, two passes)", "",
             "Commands (from the repository root on the GPU host):", "", "```", commands.strip(), "```", "",
             "| counter | per dispatch |", "|---|---|"]
    lines += [f"| {n} | {c[n]:.4g} |" for n in SQ_PASS_A + SQ_PASS_B]
    lines += ["", "Fractions of wave time (SQ_WAVE_CYCLES, same units):", "",
              f"* any instruction issuing: {frac('SQ_ACTIVE_INST_ANY'):.1%}",
              f"* VALU issuing: {frac('SQ_ACTIVE_INST_VALU'):.1%}; LDS: {frac('SQ_ACTIVE_INST_LDS'):.1%}; "
              f"scalar: {frac('SQ_ACTIVE_INST_SCA'):.1%}; vector memory: {frac('SQ_ACTIVE_INST_VMEM'):.1%}",
              f"* waiting at s_waitcnt (SQ_WAIT_ANY): {frac('SQ_WAIT_ANY'):.1%}; "
              f"waiting to issue (SQ_WAIT_INST_ANY): {frac('SQ_WAIT_INST_ANY'):.1%}",
              f"* LDS bank-conflict cycles per LDS instruction: "
              f"{c['SQ_LDS_BANK_CONFLICT'] / max(c['SQ_INSTS_LDS'], 1):.2f}"]
    if b.dtype != "f32":
        n = c["SQ_INSTS_MFMA"]
        lo = n * FLOPS_PER_MFMA_DECODE
        # with prefill rows the instructions mix the decode tiles' 1:4 forms and the prefill
        # units' 16x16x32 only: the issued flops lie between the two pricings
        hi = n * FLOPS_PER_MFMA_16X16X32 if b.rows > b.batch_size else lo
        rng = lambda f, p=2: f"{f(lo):.{p}f}" if hi == lo else f"{f(lo):.{p}f}-{f(hi):.{p}f}"
        lines += [f"* MFMA instructions: {n:.4g} per dispatch, {rng(lambda x: x / 1e9)} GFLOP issued"
                  + ("" if hi == lo else " (every instruction priced as a decode tile's mix, or as "
                                         "16x16x32 like the prefill units')")]
        if tr is not None:
            us = tr.get("kernel_timed_avg_us", tr["kernel_avg_us"])
            lines += [f"* at the timed dispatches' average of {us:.2f} us (profiles/traffic_{workload}.txt): "
                      f"{rng(lambda x: x / us / 1e6, 0)} TFLOP/s issued on MFMA, "
                      f"{rng(lambda x: x / us / 1e6 / 2500 * 100, 1)}% of the 2.5 PFLOP/s dense 16-bit peak"]
    lines.append("")
    with open(os.path.join(ROOT, "profiles", f"sq_{workload}.md"), "w") as f:
        f.write("\n".join(lines))
    print("\n".join(lines[-8:]))


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


def tile_rows(b):
    """Pool row (page * P + slot) * Hkv + kv_head of the first key of every 16-key tile of
    every (request, kv head): the tiles a decode call must read, each once."""
    import numpy as np
    P, Hkv = b.page_size, b.num_kv_heads
    out = []
    for r in range(b.batch_size):
        kl = int(b.kv_lens[r])
        t = np.arange(0, kl, 16)
        pages = b.kv_indices[b.kv_indptr[r] + t // P].astype(np.int64)
        slot_rows = pages * P + t % P
        for h in range(Hkv):
            out.append(slot_rows * Hkv + h)
    return np.concatenate(out).astype(np.int32)


def whole_row_tiles(b):
    """Pool row page * P + slot of the first key of every 16-key tile of every request: the
    same tiles as tile_rows, each read as whole token rows (every kv head at once)."""
    import numpy as np
    P = b.page_size
    out = []
    for r in range(b.batch_size):
        t = np.arange(0, int(b.kv_lens[r]), 16)
        pages = b.kv_indices[b.kv_indptr[r] + t // P].astype(np.int64)
        out.append(pages * P + t % P)
    return np.concatenate(out).astype(np.int32)


def graph_us(body, stream, L: int, replays: int = 20):
    """Median time per layer of `body` (L launches) captured in one HIP graph."""
    import torch
    body()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        body()
    g.replay()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(replays)]
    for a, e in ev:
        a.record(stream)
        g.replay()
        e.record(stream)
    torch.cuda.synchronize()
    us = sorted(a.elapsed_time(e) / L * 1e3 for a, e in ev)
    return us[len(us) // 2]


def floors(b, ks, vs, L: int, stream, grid: int = 256):
    """The read floor of the workload's access pattern and the launch floor, each as a graph
    of L launches over the same per-layer pools the attention reads (the probe kernels of
    paged_kv_gqa_plan_amd/csrc/read_probe.hip): a plain read of exactly the tiles the call
    needs (each (request, kv head)'s keys once, the kv head's slice of every token row),
    every load of a wave's tiles in flight at once where they fit (8 tiles of 128-byte
    slices, 4 of 256-byte ones), and an empty kernel of `grid` workgroups."""
    import ctypes

    import torch

    from paged_kv_gqa_plan_amd._build import PROBE_LIB
    lib = ctypes.CDLL(PROBE_LIB)
    lib.fl_probe_read_tiles.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
                                        ctypes.c_int, ctypes.c_void_p]
    lib.fl_probe_empty.argtypes = [ctypes.c_int, ctypes.c_void_p]
    rows = torch.from_numpy(tile_rows(b)).to("cuda:0")
    sink = torch.zeros(grid * 4, dtype=torch.int32, device="cuda:0")
    slice_bytes = b.head_dim * b.elem_bytes
    nb = 8 if slice_bytes == 128 else 4

    def reads():
        s = torch.cuda.current_stream().cuda_stream  # the capture stream while capturing
        for l in range(L):
            assert lib.fl_probe_read_tiles(rows.data_ptr(), rows.numel(), ks[l].data_ptr(), vs[l].data_ptr(),
                                           b.num_kv_heads, slice_bytes, nb, sink.data_ptr(), grid, s) == 0

    def empties():
        s = torch.cuda.current_stream().cuda_stream
        for _ in range(L):
            assert lib.fl_probe_empty(grid, s) == 0
    read_us, empty_us = graph_us(reads, stream, L), graph_us(empties, stream, L)
    # the same pages read as whole token rows (every kv head's slice at once): the bound of
    # a kernel that streamed whole rows instead of one kv head's slices
    row_bytes = b.num_kv_heads * slice_bytes
    whole = {}
    if b.num_kv_heads > 1 and row_bytes in (256, 512):
        wrows = torch.from_numpy(whole_row_tiles(b)).to("cuda:0")
        wnb = 4 if row_bytes == 256 else 2

        def whole_reads():
            s = torch.cuda.current_stream().cuda_stream
            for l in range(L):
                assert lib.fl_probe_read_tiles(wrows.data_ptr(), wrows.numel(), ks[l].data_ptr(), vs[l].data_ptr(),
                                               1, row_bytes, wnb, sink.data_ptr(), grid, s) == 0
        wus = graph_us(whole_reads, stream, L)
        whole = {"whole_row_read_floor_us": round(wus, 3),
                 "whole_row_read_floor_kind": f"the same pages read as whole {row_bytes}-byte token rows "
                                              f"({wrows.numel()} tiles of 16 rows of K and V), {grid} "
                                              f"workgroups, {wnb} tiles in flight per wave, graph of {L} launches"}
    tile_bytes = rows.numel() * 16 * slice_bytes * 2
    tiles_per_wave = -(-rows.numel() // (grid * 4))
    return {"read_floor_us": round(read_us, 3),
            "read_floor_GB_per_s": round(b.kv_bytes() / (read_us * 1e-6) / 1e9, 1),
            "read_floor_kind": f"plain read of the call's {rows.numel()} tiles ({tile_bytes} bytes, "
                               f"the kv head's slice of 16 token rows of K and V each), {grid} "
                               f"workgroups, up to {nb} tiles in flight per wave "
                               f"({'all of them' if tiles_per_wave <= nb else f'of {tiles_per_wave}'}), "
                               f"graph of {L} launches",
            "launch_floor_us": round(empty_us, 3),
            "launch_floor_kind": f"empty kernel of {grid} workgroups, graph of {L} launches", **whole}


def prefill_flops(b) -> int:
    """Algorithmic flops of the requests with more than one query row (unmasked pairs)."""
    pairs = 0
    for ql, kl in zip(b.qo_lens.tolist(), b.kv_lens.tolist()):
        if ql > 1:
            pairs += sum(kl - ql + i + 1 for i in range(ql)) if b.causal else ql * kl
    return pairs * b.num_qo_heads * 4 * b.head_dim


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


class Leg:
    """One workload on the device: per-layer pools, a handle, the layer runs captured in a
    HIP graph (or eager), timed over `steps` steps of plan + L runs."""

    def __init__(self, name, args, L: int = 0):
        import torch

        import paged_kv_gqa_plan_amd as fl
        import workloads as W
        self.b = b = W.WORKLOADS[name](seed=args.seed)
        self.L = L or args.layers or LAYERS[name]
        self.q = device_tensor(b.q, b.dtype)
        k0, v0 = device_tensor(b.k_pool, b.dtype), device_tensor(b.v_pool, b.dtype)
        gen = torch.Generator(device="cuda:0")
        gen.manual_seed(1000 + args.seed)
        self.ks, self.vs = [k0], [v0]
        for _ in range(1, self.L):
            self.ks.append(torch.randn(k0.shape, dtype=k0.dtype, device="cuda:0", generator=gen))
            self.vs.append(torch.randn(v0.shape, dtype=k0.dtype, device="cuda:0", generator=gen))
        self.outs = [torch.empty(self.q.shape, dtype=k0.dtype, device="cuda:0") for _ in range(self.L)]
        cfg = fl.make_config(b.num_qo_heads, b.num_kv_heads, b.head_dim, b.page_size, b.dtype,
                             b.batch_size, b.rows, int(b.kv_indptr[-1]),
                             groups_per_cu=args.groups_per_cu, min_group_tokens=args.min_group_tokens,
                             waves_per_group=args.waves, whole_rows=args.whole_rows)
        self.h = fl.PagedAttention(cfg, device=0)
        self.stream = torch.cuda.current_stream()
        self.args = args

    def plan(self):
        b = self.b
        self.h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
                    causal=b.causal, sm_scale=b.sm_scale, num_splits=self.args.splits)

    def layers(self):
        for l in range(self.L):
            self.h.run(self.q, self.ks[l], self.vs[l], self.outs[l])

    def time(self, steps: int, warmup: int, eager: bool = False):
        import numpy as np
        import torch
        graph = None
        if not eager:
            self.plan()
            self.layers()  # first launches outside the capture
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph):
                self.layers()

        def step(ev=None):
            self.plan()
            if ev is not None:
                ev[0].record(self.stream)
            if graph is not None:
                graph.replay()
            else:
                self.layers()
            if ev is not None:
                ev[1].record(self.stream)

        for _ in range(max(warmup, 1)):
            step()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for s_ in range(steps):
            step(evs[s_])
        torch.cuda.synchronize()
        self.wall = time.perf_counter() - t0
        call_ms = [a.elapsed_time(e) / self.L for (a, e) in evs]
        plan_s = 0.0
        for _ in range(10):
            t1 = time.perf_counter()
            self.plan()
            plan_s += time.perf_counter() - t1
        torch.cuda.synchronize()
        self.us_call = float(np.mean(call_ms)) * 1e3
        self.us_call_med = float(np.median(call_ms)) * 1e3
        self.plan_us = plan_s / 10 * 1e6
        n_items, n_groups, max_splits, ws_bytes = self.h.info()
        b = self.b
        achieved = b.kv_bytes() / (self.us_call * 1e-6) / 1e9
        d = {"batch": b.batch_size, "query_rows": b.rows, "kv_tokens": int(b.kv_lens.sum()),
             "num_qo_heads": b.num_qo_heads, "num_kv_heads": b.num_kv_heads, "head_dim": b.head_dim,
             "dtype": b.dtype, "page_size": b.page_size, "layers": self.L,
             "us_per_call": round(self.us_call, 3), "us_per_call_median": round(self.us_call_med, 3),
             "kv_bytes_per_call": b.kv_bytes(), "kv_GB_per_s": round(achieved, 1),
             "hbm_peak_frac": round(achieved / HBM_PEAK_GBS, 4),
             "plan_host_us": round(self.plan_us, 2), "work_items": n_items, "workgroups": n_groups,
             "max_splits": max_splits, "workspace_bytes": ws_bytes,
             "launch": "eager" if eager else "hip_graph"}
        pf = prefill_flops(b)
        if pf:
            # the prefill part's algorithmic flops over the whole call's time: a lower bound
            # of its rate (the decode rows share the call)
            d["prefill_flops_per_call"] = pf
            d["prefill_mfma_frac_lower_bound"] = round(pf / (self.us_call * 1e-6) / 1e12 / MFMA_PEAK_TFLOPS, 4)
        self.achieved = achieved
        return d

    def close(self):
        import torch
        self.h.close()
        del self.q, self.ks, self.vs, self.outs
        torch.cuda.synchronize()
        torch.cuda.empty_cache()


MFMA_PEAK_TFLOPS = 2500.0  # dense bf16 / fp16
EXTRA_WORKLOADS = ("mixed_length_decode", "long_context_skew", "ragged_mixed_step", "multi_chunk_step")


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="saturated_decode", choices=sorted(LAYERS))
    ap.add_argument("--layers", type=int, default=0, help="per-layer pools (0: 24 or 28 by workload)")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--splits", type=int, default=0, help="planner slice override (0 = automatic)")
    ap.add_argument("--groups-per-cu", type=int, default=0)
    ap.add_argument("--min-group-tokens", type=int, default=0)
    ap.add_argument("--waves", type=int, default=0, help="wavefronts per workgroup (4; 0 = default)")
    ap.add_argument("--whole-rows", type=int, default=0, choices=[-1, 0, 1],
                    help="whole-row blocks: 0 where they apply and pay off, 1 wherever they "
                         "apply, -1 never (one block per kv head)")
    ap.add_argument("--cpu-budget", type=float, default=10.0, help="seconds of oracle timing")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--extra-workloads", default=",".join(EXTRA_WORKLOADS),
                    help="comma-separated workloads timed after the headline one ('' for none)")
    ap.add_argument("--attention-only", action="store_true",
                    help="time the attention runs of the chosen workload only (no floors, cold "
                         "call, probe, append legs, other workloads or CPU baseline): for "
                         "profiler runs, whose summaries pick the attention kernel")
    ap.add_argument("--eager", action="store_true", help="launch layer runs without a HIP graph")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="only run a plain copy of this many MiB (counter calibration)")
    ap.add_argument("--summarize-profiles", nargs=5, metavar=("KT", "PF", "PW", "CF", "CW"),
                    help="write profiles/ summaries from rocprofv3 CSV directories (kernel "
                         "trace; FETCH_SIZE and WRITE_SIZE of the bench; the same of a copy)")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("A", "B"),
                    help="write profiles/sq_<workload>.md from two rocprofv3 --pmc CSV directories "
                         "holding the SQ counter passes")
    ap.add_argument("--calib-mib", type=int, default=1024)
    ap.add_argument("--commands", default="", help="commands recorded in the summary")
    args = ap.parse_args(argv)

    if args.summarize_sq:
        summarize_sq(args.workload, *args.summarize_sq, args.commands)
        return 0
    if args.summarize_profiles:
        summarize_profiles(args.workload, *args.summarize_profiles, args.calib_mib, args.commands,
                           args.steps, args.layers)
        return 0

    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(the attention path runs on a single device; no multi-GPU mode exists)",
              file=sys.stderr)
        return 2
    if args.copy_calibration_mib:
        copy_calibration(args.copy_calibration_mib)
        return 0

    # torch first: its HIP runtime is the one the library then binds to
    import torch  # noqa: F401

    import paged_kv_gqa_plan_amd as fl

    fl.load_library()
    leg = Leg(args.workload, args)
    b, L = leg.b, leg.L
    d = leg.time(args.steps, args.warmup, eager=args.eager)
    kv_bytes = b.kv_bytes()
    value = kv_bytes * L * args.steps / leg.wall / 1e9
    traffic = traffic_from_profile(args.workload)
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(leg.wall / args.steps * 1e3, 4),
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
                   "whole_rows": args.whole_rows,
                   "parallelism": "single GPU"},
        "us_per_call": d["us_per_call"],
        "us_per_call_median": d["us_per_call_median"],
        "kv_bytes_per_call": kv_bytes,
        "hbm_peak_frac_per_call": d["hbm_peak_frac"],
        "attention_us_per_step": round(leg.us_call * L, 2),
        "launch": d["launch"],
        "plan_host_us": d["plan_host_us"],
        "work_items": d["work_items"],
        "workgroups": d["workgroups"],
        "max_splits": d["max_splits"],
        "workspace_bytes": d["workspace_bytes"],
        "roofline": {"bound": "hbm", "achieved": round(leg.achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(leg.achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic},
    }
    out0 = leg.outs[0].clone()  # layer 0's result, before the extra legs below overwrite it
    if not args.attention_only:
        fl_ = floors(b, leg.ks, leg.vs, L, leg.stream)
        fl_["achieved_frac_of_read_floor"] = round(fl_["read_floor_us"] / leg.us_call, 4)
        res["floors"] = fl_
        cold = cold_call_us(leg.h, leg.q, leg.ks[0], leg.vs[0], leg.outs[0], leg.stream)
        probe = stream_probe_gbs()
        res["cold_call_us"] = round(cold, 3)
        res["stream_probe"] = {"GB_per_s": round(probe, 1),
                               "kind": "device copy of 1 GiB, bytes read + written per second",
                               "achieved_frac_of_probe": round(leg.achieved / probe, 4)}
        res["kv_append"] = time_kv_append(leg.h, b, leg.ks, leg.vs, L, leg.stream)
        res["kv_append_rope"] = time_kv_append(leg.h, b, leg.ks, leg.vs, L, leg.stream, rope_theta=1e4)
        res["append_attention"] = time_append_attention(leg.h, b, leg.q, leg.ks, leg.vs, leg.outs, L,
                                                        leg.stream)
    leg.close()
    if not args.attention_only and args.extra_workloads:
        # the other workloads, each with its own floors, timed the same way
        res["workloads"] = {}
        for name in [w for w in args.extra_workloads.split(",") if w and w != args.workload]:
            x = Leg(name, args)
            e = x.time(args.steps, args.warmup, eager=args.eager)
            f = floors(x.b, x.ks, x.vs, x.L, x.stream)
            f["achieved_frac_of_read_floor"] = round(f["read_floor_us"] / x.us_call, 4)
            e.update(f)
            res["workloads"][name] = e
            x.close()
            print(f"# {name}: {e['us_per_call']} us per call, {e['hbm_peak_frac']:.3f} of HBM peak, "
                  f"read floor {f['read_floor_us']} us", file=sys.stderr, flush=True)
    if not args.no_cpu_baseline and not args.attention_only:
        res["cpu_baseline"] = cpu_baseline(b, out0, args.cpu_budget)
    print(json.dumps(res), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
