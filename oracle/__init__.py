"""CPU oracle for paged grouped-query attention: loader and build step.

TEST INFRASTRUCTURE ONLY. The test suite, the package smoke check and the benchmark's
CPU-baseline leg are the only callers. The HIP library never imports this package and
this package imports nothing from the HIP library; the two share only the seeded input
arrays from ``workloads``.

The arithmetic lives in ``paged_attn_oracle.c`` (plain C, double precision): a gather of
each request's pages into dense K/V followed by plain softmax attention, plus an optional
split-and-merge mode. ``attention(batch)`` returns unrounded fp64 results.
``kv_append(...)`` writes a step's new K/V rows into copies of the pools (a byte copy to
each new token's page slot); ``rope(...)`` rotates head vectors by their positions (the
rotary embedding of the append fused with RoPE); ``paged_kv_poison(...)`` fills freed pages
with NaN.
``page_pool.PagePoolModel`` is the page allocator's reference bookkeeping.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "paged_attn_oracle.c")
LIB = os.path.join(_HERE, "liboracle_paged_attn.so")
# A test may point the loader at another build of the oracle (a planted-mistake copy).
_LIB_OVERRIDE = os.environ.get("FL_ORACLE_LIB")
_lib = None


def build(force: bool = True) -> str:
    """Compile the oracle with gcc (OpenMP, -O2, no fast-math: IEEE double arithmetic)."""
    if force or not os.path.exists(LIB) or os.path.getmtime(LIB) < os.path.getmtime(SRC):
        tmp = LIB + ".tmp"
        subprocess.check_call(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11",
                               "-Wall", "-Wextra", "-o", tmp, SRC, "-lm"])
        os.replace(tmp, LIB)
    return LIB


def load(path: Optional[str] = None):
    global _lib
    if _lib is not None and path is None:
        return _lib
    if path is None and _LIB_OVERRIDE:
        path = _LIB_OVERRIDE
    p = path or LIB
    if p == LIB and (not os.path.exists(p) or os.path.getmtime(p) < os.path.getmtime(SRC)):
        build(force=True)
    lib = ctypes.CDLL(p)
    lib.oracle_paged_attention.restype = ctypes.c_int
    lib.oracle_paged_attention.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_double,
        ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int]
    lib.oracle_decode.restype = ctypes.c_int
    lib.oracle_decode.argtypes = [ctypes.c_int, ctypes.c_void_p, ctypes.c_int64, ctypes.c_void_p]
    lib.oracle_paged_kv_append.restype = ctypes.c_int
    lib.oracle_paged_kv_append.argtypes = [
        ctypes.c_int, ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
        ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int, ctypes.c_int,
        ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]
    lib.oracle_paged_kv_poison.restype = ctypes.c_int
    lib.oracle_paged_kv_poison.argtypes = [ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_int, ctypes.c_int64, ctypes.c_void_p,
                                           ctypes.c_void_p]
    lib.oracle_rope.restype = ctypes.c_int
    lib.oracle_rope.argtypes = [ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                ctypes.c_void_p, ctypes.c_void_p, ctypes.c_double, ctypes.c_void_p]
    lib.oracle_max_threads.restype = ctypes.c_int
    lib.oracle_max_threads.argtypes = []
    if path is None or path == _LIB_OVERRIDE:
        _lib = lib
    return lib


class OracleError(RuntimeError):
    pass


def _ptr(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def paged_attention(dtype_code: int, qo_indptr, kv_indptr, kv_indices, last_page_len,
                    num_pages: int, num_qo_heads: int, num_kv_heads: int, head_dim: int,
                    page_size: int, q, k_pool, v_pool, causal: bool = True,
                    sm_scale: float = 0.0, num_splits: int = 1, num_threads: int = 0,
                    lib=None):
    """Raw entry: returns (out[rows, Hq, D] float64, lse[rows, Hq] float64)."""
    lib = lib or load()
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    last_page_len = np.ascontiguousarray(last_page_len, dtype=np.int32)
    B = int(kv_indptr.shape[0]) - 1
    if qo_indptr is not None:
        qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
        rows = int(qo_indptr[-1])
    else:
        rows = B
    q = np.ascontiguousarray(q)
    k_pool = np.ascontiguousarray(k_pool)
    v_pool = np.ascontiguousarray(v_pool)
    out = np.zeros((rows, num_qo_heads, head_dim), dtype=np.float64)
    lse = np.zeros((rows, num_qo_heads), dtype=np.float64)
    rc = lib.oracle_paged_attention(
        int(dtype_code), B, _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
        _ptr(last_page_len), int(num_pages), int(num_qo_heads), int(num_kv_heads), int(head_dim),
        int(page_size), _ptr(q), _ptr(k_pool), _ptr(v_pool), int(bool(causal)), float(sm_scale),
        int(num_splits), _ptr(out), _ptr(lse), int(num_threads))
    if rc != 0:
        raise OracleError(f"oracle_paged_attention returned {rc}")
    return out, lse


def attention(batch, num_splits: int = 1, num_threads: int = 0, lib=None):
    """Oracle result for a ``workloads.Batch``: (out fp64 [rows, Hq, D], lse fp64 [rows, Hq])."""
    return paged_attention(batch.dtype_code, batch.qo_indptr, batch.kv_indptr, batch.kv_indices,
                           batch.last_page_len, batch.num_pages, batch.num_qo_heads,
                           batch.num_kv_heads, batch.head_dim, batch.page_size, batch.q,
                           batch.k_pool, batch.v_pool, batch.causal, batch.sm_scale, num_splits,
                           num_threads, lib=lib)


def paged_kv_append(elem_bytes: int, qo_indptr, kv_indptr, kv_indices, last_page_len,
                    num_pages: int, num_kv_heads: int, head_dim: int, page_size: int,
                    k_new, v_new, k_pool, v_pool, lib=None):
    """Raw entry: returns new (k_pool, v_pool) arrays with the rows of k_new / v_new
    ``[rows, Hkv, D]`` written to their tokens' page slots; the inputs are not modified."""
    lib = lib or load()
    kv_indptr = np.ascontiguousarray(kv_indptr, dtype=np.int32)
    kv_indices = np.ascontiguousarray(kv_indices, dtype=np.int32)
    last_page_len = np.ascontiguousarray(last_page_len, dtype=np.int32)
    B = int(kv_indptr.shape[0]) - 1
    if qo_indptr is not None:
        qo_indptr = np.ascontiguousarray(qo_indptr, dtype=np.int32)
    k_out = np.array(k_pool, copy=True, order="C")
    v_out = np.array(v_pool, copy=True, order="C")
    k_new = np.ascontiguousarray(k_new)
    v_new = np.ascontiguousarray(v_new)
    rc = lib.oracle_paged_kv_append(
        int(elem_bytes), B, _ptr(qo_indptr), _ptr(kv_indptr), _ptr(kv_indices),
        _ptr(last_page_len), int(num_pages), int(num_kv_heads), int(head_dim), int(page_size),
        _ptr(k_new), _ptr(v_new), _ptr(k_out), _ptr(v_out))
    if rc != 0:
        raise OracleError(f"oracle_paged_kv_append returned {rc}")
    return k_out, v_out


def kv_append(batch, k_new, v_new, k_pool=None, v_pool=None, lib=None):
    """Oracle append for a ``workloads.Batch``'s page table and query rows: the new rows go
    into copies of ``k_pool`` / ``v_pool`` (default: the batch's own pools)."""
    return paged_kv_append(batch.elem_bytes, batch.qo_indptr, batch.kv_indptr, batch.kv_indices,
                           batch.last_page_len, batch.num_pages, batch.num_kv_heads,
                           batch.head_dim, batch.page_size, k_new, v_new,
                           batch.k_pool if k_pool is None else k_pool,
                           batch.v_pool if v_pool is None else v_pool, lib=lib)


def rope(dtype_code: int, x, positions, theta: float, lib=None) -> np.ndarray:
    """Rotary embedding of ``x`` ``[rows, heads, D]`` (storage values) at per-row
    ``positions``; float64 result of the same shape."""
    lib = lib or load()
    a = np.ascontiguousarray(x)
    pos = np.ascontiguousarray(positions, dtype=np.int32)
    rows, heads, d = a.shape
    if pos.shape != (rows,):
        raise OracleError("one position per row")
    y = np.zeros(a.shape, dtype=np.float64)
    rc = lib.oracle_rope(int(dtype_code), rows, heads, d, _ptr(a), _ptr(pos), float(theta), _ptr(y))
    if rc != 0:
        raise OracleError(f"oracle_rope returned {rc}")
    return y


def append_positions(qo_indptr, kv_indptr, last_page_len, page_size: int) -> np.ndarray:
    """Position of every query row: row i of a request with qo_len rows and kv_len cached
    tokens is token kv_len - qo_len + i (the same reading as the append's slots and the
    bottom-right causal mask)."""
    kv_indptr = np.asarray(kv_indptr, dtype=np.int64)
    last = np.asarray(last_page_len, dtype=np.int64)
    B = kv_indptr.shape[0] - 1
    qo = np.arange(B + 1) if qo_indptr is None else np.asarray(qo_indptr, dtype=np.int64)
    kv_len = (np.diff(kv_indptr) - 1) * page_size + last
    out = np.zeros(int(qo[-1]), dtype=np.int32)
    for r in range(B):
        ql = int(qo[r + 1] - qo[r])
        out[qo[r]:qo[r + 1]] = kv_len[r] - ql + np.arange(ql)
    return out


def paged_kv_poison(dtype_code: int, page_ids, k_pool, v_pool=None, lib=None):
    """Copies of the pools ``[num_pages, ...]`` with every element of the listed pages set to
    the storage type's quiet NaN."""
    lib = lib or load()
    ids = np.ascontiguousarray(page_ids, dtype=np.int32)
    k_out = np.array(k_pool, copy=True, order="C")
    v_out = None if v_pool is None else np.array(v_pool, copy=True, order="C")
    page_elems = int(np.prod(k_out.shape[1:]))
    rc = lib.oracle_paged_kv_poison(int(dtype_code), page_elems, _ptr(ids), int(ids.size),
                                    int(k_out.shape[0]), _ptr(k_out), _ptr(v_out))
    if rc != 0:
        raise OracleError(f"oracle_paged_kv_poison returned {rc}")
    return k_out, v_out


def decode(dtype_code: int, values: np.ndarray, lib=None) -> np.ndarray:
    """The oracle's own decoding of stored 16/32-bit values to float64."""
    lib = lib or load()
    a = np.ascontiguousarray(values)
    dst = np.zeros(a.size, dtype=np.float64)
    rc = lib.oracle_decode(int(dtype_code), _ptr(a), int(a.size), _ptr(dst))
    if rc != 0:
        raise OracleError(f"oracle_decode returned {rc}")
    return dst.reshape(a.shape)


def max_threads(lib=None) -> int:
    return int((lib or load()).oracle_max_threads())
