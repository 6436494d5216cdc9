"""Shared helpers for the GPU tests: move a seeded batch to the device, run it through the
C interface, bring the result back. torch provides device memory and the stream only."""
from __future__ import annotations

import sys

import numpy as np

import paged_kv_gqa_plan_amd as fl
import workloads as W

TOL = {"bf16": 4e-3, "f16": 4e-3, "f32": 1e-5}   # max-abs against the unrounded oracle
LSE_TOL = {"bf16": 1e-4, "f16": 1e-4, "f32": 1e-5}


def torch_dtype(dtype):
    import torch
    return {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}[dtype]


def to_device(arr: np.ndarray, dtype: str):
    import torch
    a = np.ascontiguousarray(arr)
    if dtype == "bf16":
        t = torch.from_numpy(a.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(a)
    return t.to("cuda:0")


def to_host_f64(t) -> np.ndarray:
    import torch
    return t.detach().to(torch.float64).cpu().numpy()


def to_host_bits(t, dtype: str) -> np.ndarray:
    import torch
    c = t.detach().cpu()
    if dtype == "bf16":
        return c.view(torch.int16).numpy().view(np.uint16)
    return c.numpy()


def config_for(b: W.Batch, **kw):
    return fl.make_config(b.num_qo_heads, b.num_kv_heads, b.head_dim, b.page_size, b.dtype,
                          max(b.batch_size, 1), max(b.rows, 1), max(int(b.kv_indptr[-1]), 1), **kw)


class DeviceBatch:
    """A batch resident on cuda:0 plus a handle planned for it."""

    def __init__(self, b: W.Batch, num_splits: int = 0, handle: fl.PagedAttention = None, **cfg_kw):
        import torch
        self.b = b
        self.q = to_device(b.q, b.dtype)
        self.k = to_device(b.k_pool, b.dtype)
        self.v = to_device(b.v_pool, b.dtype)
        self.out = torch.full((b.rows, b.num_qo_heads, b.head_dim), float("nan"),
                              dtype=torch_dtype(b.dtype), device="cuda:0")
        self.lse = torch.full((b.rows, b.num_qo_heads), float("nan"), dtype=torch.float32,
                              device="cuda:0")
        self.h = handle or fl.PagedAttention(config_for(b, **cfg_kw), device=0)
        self.plan(num_splits)

    def plan(self, num_splits=0):
        b = self.b
        self.h.plan(b.qo_indptr, b.kv_indptr, b.kv_indices, b.last_page_len, b.num_pages,
                    causal=b.causal, sm_scale=b.sm_scale, num_splits=num_splits)

    def run(self, with_lse=True):
        import torch
        self.h.run(self.q, self.k, self.v, self.out, self.lse if with_lse else None)
        torch.cuda.synchronize()
        return self.out, self.lse


def announce(msg: str):
    print(f"[gpu-case] {msg}", file=sys.stderr, flush=True)


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output type at |x| (normal range)."""
    mant = {"bf16": 7, "f16": 10, "f32": 23}[dtype]
    _, e = np.frexp(np.abs(x))                 # |x| = m * 2^e, m in [0.5, 1)
    return np.ldexp(1.0, e - 2 - mant)


def tolerance(ref: np.ndarray, dtype: str) -> np.ndarray:
    """Max-abs bar per cell: the stated bound (4e-3 for 16-bit outputs, 1e-5 for fp32),
    except where the output type cannot hold a value that close: where its half-ulp at the
    result's magnitude exceeds the bound (bf16 |o| >= 2, fp16 |o| >= 16), half an ulp plus
    1e-4 for the arithmetic."""
    t = TOL[dtype]
    if dtype == "f32":
        return np.full(ref.shape, t)
    hu = half_ulp(ref, dtype)
    return np.where(hu < t, t, hu + 1e-4)


def compare(b: W.Batch, out_dev, lse_dev, ref_out, ref_lse, what: str = ""):
    got = to_host_f64(out_dev)
    assert np.isfinite(got).all(), f"{what}: non-finite output"
    err = np.abs(got - ref_out)
    tol = tolerance(ref_out, b.dtype)
    worst = float(err.max()) if err.size else 0.0
    ratio = err / tol
    assert (ratio <= 1.0).all(), (f"{what}: max-abs {worst:.3e}, worst cell err/tol "
                                  f"{float(ratio.max()):.3f} at {np.unravel_index(np.argmax(ratio), ratio.shape)}")
    if lse_dev is not None:
        gl = to_host_f64(lse_dev)
        lerr = float(np.abs(gl - ref_lse).max()) if gl.size else 0.0
        assert lerr <= LSE_TOL[b.dtype], f"{what}: lse max-abs {lerr:.3e}"
    return worst
