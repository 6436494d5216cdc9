"""Python binding for ``libfl_paged_attn.so``: paged grouped-query attention on gfx950.

Argument marshalling only. Every step of the computation runs in the library's HIP
kernels; the functions below carry the C interface's names and pass plain pointers,
sizes and host arrays through ctypes. torch is used by the optional ``PagedAttention``
helper for device memory and streams only (``tensor.data_ptr()``,
``torch.cuda.current_stream().cuda_stream``).

The library is built in-tree (``paged_kv_gqa_plan_amd/_build.py``); importing the
binding without it raises at once — there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Tuple

import numpy as np

from ._build import LIB as LIB_PATH

FL_OK, FL_ERR_INVALID_ARG, FL_ERR_UNSUPPORTED, FL_ERR_CAPACITY = 0, -1, -2, -3
FL_ERR_NOT_PLANNED, FL_ERR_HIP = -4, -5
FL_F16, FL_BF16, FL_F32 = 1, 2, 3
FL_WORK_ITEM_INTS = 16
WORK_ITEM_FIELDS = ("q_start", "qo_len", "kv_len", "page_base", "kv_head", "row_begin",
                    "num_rows", "tok_begin", "tok_end", "part_row", "request", "split",
                    "num_splits", "merge", "group", "pos_begin")
STATUS_NAMES = {0: "FL_OK", -1: "FL_ERR_INVALID_ARG", -2: "FL_ERR_UNSUPPORTED",
                -3: "FL_ERR_CAPACITY", -4: "FL_ERR_NOT_PLANNED", -5: "FL_ERR_HIP"}
DTYPE_CODES = {"f16": FL_F16, "bf16": FL_BF16, "f32": FL_F32}


class fl_config(ctypes.Structure):
    _fields_ = [("num_qo_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("max_batch", ctypes.c_int32),
                ("max_qo_rows", ctypes.c_int32), ("max_kv_pages", ctypes.c_int64),
                ("num_cus", ctypes.c_int32), ("groups_per_cu", ctypes.c_int32),
                ("min_group_tokens", ctypes.c_int32), ("waves_per_group", ctypes.c_int32),
                ("max_tiles", ctypes.c_int64), ("whole_rows", ctypes.c_int32)]


class FlError(RuntimeError):
    def __init__(self, status: int, where: str, message: str):
        super().__init__(f"{where}: {STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


EXPORTED = ("fl_paged_attn_create", "fl_paged_attn_destroy", "fl_paged_attn_plan",
            "fl_paged_attn_run", "fl_paged_attn_run_noalloc", "fl_paged_kv_append", "fl_paged_attn_run_append",
            "fl_paged_kv_append_slots", "fl_paged_kv_append_rope",
            "fl_paged_attn_plan_info", "fl_paged_attn_plan_launch",
            "fl_paged_attn_refused_launches", "fl_paged_attn_get_work_items", "fl_page_pool_create", "fl_page_pool_destroy",
            "fl_page_pool_alloc", "fl_page_pool_reserve", "fl_page_pool_retain",
            "fl_page_pool_release", "fl_page_pool_refcounts", "fl_page_pool_info",
            "fl_paged_kv_poison", "fl_last_error")

_lib = None


def load_library(path: Optional[str] = None):
    """Load the built library (raises if it is missing): `path`, else the file named by the
    FL_PAGED_ATTN_LIB environment variable (a checking build, say), else the in-tree build."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or os.environ.get("FL_PAGED_ATTN_LIB") or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -c 'import __graft_entry__ as g; "
                          f"g.build()'` (hipcc, gfx950)")
    lib = ctypes.CDLL(p)
    vp, i32, i64 = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64
    lib.fl_paged_attn_create.argtypes = [ctypes.POINTER(fl_config), ctypes.c_int, ctypes.POINTER(vp)]
    lib.fl_paged_attn_destroy.argtypes = [vp]
    lib.fl_paged_attn_plan.argtypes = [vp, i32, vp, vp, vp, vp, i64, i32, ctypes.c_float, i32, vp]
    lib.fl_paged_attn_run.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.fl_paged_attn_run_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, vp]
    lib.fl_paged_kv_append.argtypes = [vp, vp, vp, vp, vp, vp]
    lib.fl_paged_attn_run_append.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp]
    lib.fl_paged_kv_append_slots.argtypes = [vp, vp, i32, ctypes.POINTER(i32)]
    lib.fl_paged_attn_plan_info.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                            ctypes.POINTER(i32), ctypes.POINTER(i64)]
    lib.fl_paged_attn_plan_launch.argtypes = [vp, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                              ctypes.POINTER(i32), ctypes.POINTER(i32)]
    lib.fl_paged_attn_refused_launches.argtypes = [vp, ctypes.POINTER(i32)]
    lib.fl_paged_attn_get_work_items.argtypes = [vp, vp, i32, ctypes.POINTER(i32)]
    lib.fl_page_pool_create.argtypes = [i64, i32, ctypes.POINTER(vp)]
    lib.fl_page_pool_destroy.argtypes = [vp]
    lib.fl_page_pool_alloc.argtypes = [vp, i32, vp]
    lib.fl_page_pool_reserve.argtypes = [vp, i64, vp, i32, ctypes.POINTER(i32)]
    lib.fl_page_pool_retain.argtypes = [vp, vp, i32]
    lib.fl_page_pool_release.argtypes = [vp, vp, i32, vp, ctypes.POINTER(i32)]
    lib.fl_page_pool_refcounts.argtypes = [vp, vp, i32, vp]
    lib.fl_page_pool_info.argtypes = [vp, ctypes.POINTER(i64), ctypes.POINTER(i64)]
    lib.fl_paged_kv_poison.argtypes = [i32, i32, i32, i32, i64, vp, i32, vp, vp, vp]
    for name in EXPORTED[:-1]:
        getattr(lib, name).restype = ctypes.c_int
    lib.fl_last_error.argtypes = []
    lib.fl_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def _check(st: int, where: str):
    if st != FL_OK:
        raise FlError(st, where, fl_last_error())


def _i32(a) -> Optional[np.ndarray]:
    return None if a is None else np.ascontiguousarray(a, dtype=np.int32)


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def fl_last_error() -> str:
    return load_library().fl_last_error().decode()


def fl_paged_attn_create(cfg: fl_config, device: int) -> ctypes.c_void_p:
    h = ctypes.c_void_p()
    _check(load_library().fl_paged_attn_create(ctypes.byref(cfg), int(device), ctypes.byref(h)),
           "fl_paged_attn_create")
    return h


def fl_paged_attn_destroy(h) -> None:
    _check(load_library().fl_paged_attn_destroy(h), "fl_paged_attn_destroy")


def fl_paged_attn_plan(h, batch: int, qo_indptr, kv_indptr, kv_indices, last_page_len,
                       num_pages: int, causal: bool = True, sm_scale: float = 0.0,
                       num_splits: int = 0, stream: int = 0) -> None:
    """Host arrays (anything numpy turns into int32) for the metadata; ``stream`` is a
    hipStream_t as an integer (0 = null stream)."""
    qo, kp, ki, lp = _i32(qo_indptr), _i32(kv_indptr), _i32(kv_indices), _i32(last_page_len)
    _check(load_library().fl_paged_attn_plan(h, int(batch), _p(qo), _p(kp), _p(ki), _p(lp),
                                             int(num_pages), int(bool(causal)), float(sm_scale),
                                             int(num_splits), ctypes.c_void_p(int(stream))),
           "fl_paged_attn_plan")


def fl_paged_attn_run(h, q: int, k_pool: int, v_pool: int, out: int, lse: Optional[int] = None,
                      stream: int = 0) -> None:
    """Device pointers as integers (e.g. ``tensor.data_ptr()``); lse may be None."""
    _check(load_library().fl_paged_attn_run(h, ctypes.c_void_p(q), ctypes.c_void_p(k_pool),
                                            ctypes.c_void_p(v_pool), ctypes.c_void_p(out),
                                            ctypes.c_void_p(lse or 0), ctypes.c_void_p(int(stream))),
           "fl_paged_attn_run")


def fl_paged_attn_run_noalloc(h, q: int, k_pool: int, v_pool: int, out: int,
                              lse: Optional[int] = None, stream: int = 0) -> None:
    """fl_paged_attn_run without device allocation (the library's fixed scratch array);
    the handle may be host-only."""
    _check(load_library().fl_paged_attn_run_noalloc(
        h, ctypes.c_void_p(q), ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool), ctypes.c_void_p(out),
        ctypes.c_void_p(lse or 0), ctypes.c_void_p(int(stream))), "fl_paged_attn_run_noalloc")


def fl_paged_kv_append(h, k_new: int, v_new: int, k_pool: int, v_pool: int,
                       stream: int = 0) -> None:
    """Device pointers as integers: the plan's query rows' new K/V rows go to their tokens'
    page slots of one layer's pools."""
    _check(load_library().fl_paged_kv_append(h, ctypes.c_void_p(k_new), ctypes.c_void_p(v_new),
                                             ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool),
                                             ctypes.c_void_p(int(stream))),
           "fl_paged_kv_append")


def fl_paged_kv_append_rope(h, q: Optional[int], k_new: int, v_new: int, k_pool: int, v_pool: int,
                            rope_theta: float, stream: int = 0) -> None:
    """Device pointers as integers: the append with the rotary embedding of the new rows'
    key heads (written to the pool) and query heads (rotated in place; q may be None)."""
    _check(load_library().fl_paged_kv_append_rope(
        h, ctypes.c_void_p(q) if q else None, ctypes.c_void_p(k_new), ctypes.c_void_p(v_new),
        ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool), ctypes.c_float(rope_theta),
        ctypes.c_void_p(int(stream))), "fl_paged_kv_append_rope")


def fl_paged_attn_run_append(h, q: int, k_new: int, v_new: int, k_pool: int, v_pool: int, out: int,
                             lse: Optional[int] = None, stream: int = 0) -> None:
    """Device pointers as integers: append the new K/V rows and attend, in one launch on
    decode-only 16-bit plans."""
    _check(load_library().fl_paged_attn_run_append(
        h, ctypes.c_void_p(q), ctypes.c_void_p(k_new), ctypes.c_void_p(v_new), ctypes.c_void_p(k_pool),
        ctypes.c_void_p(v_pool), ctypes.c_void_p(out), ctypes.c_void_p(lse or 0),
        ctypes.c_void_p(int(stream))), "fl_paged_attn_run_append")


def fl_paged_kv_append_slots(h) -> np.ndarray:
    """The current plan's append destinations: int32 token row (page * P + slot) per query row."""
    lib = load_library()
    n = ctypes.c_int32()
    _check(lib.fl_paged_kv_append_slots(h, None, 0, ctypes.byref(n)), "fl_paged_kv_append_slots")
    buf = np.zeros(max(n.value, 1), dtype=np.int32)
    _check(lib.fl_paged_kv_append_slots(h, _p(buf), n.value, ctypes.byref(n)),
           "fl_paged_kv_append_slots")
    return buf[:n.value]


def fl_paged_attn_plan_info(h) -> Tuple[int, int, int, int]:
    """(work items, workgroups, largest pieces per row block, workspace bytes)."""
    n, g, s, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int64()
    _check(load_library().fl_paged_attn_plan_info(h, ctypes.byref(n), ctypes.byref(g),
                                                  ctypes.byref(s), ctypes.byref(b)),
           "fl_paged_attn_plan_info")
    return n.value, g.value, s.value, b.value


def fl_paged_attn_plan_launch(h) -> Tuple[int, int, int, int]:
    """(launch class of run, launch class of the one-launch run_append or 0, grid,
    workgroups with work)."""
    c, f, g, b = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
    _check(load_library().fl_paged_attn_plan_launch(h, ctypes.byref(c), ctypes.byref(f),
                                                    ctypes.byref(g), ctypes.byref(b)),
           "fl_paged_attn_plan_launch")
    return c.value, f.value, g.value, b.value


def fl_paged_attn_refused_launches(h) -> int:
    """Launches refused since the last call (waits for the device)."""
    n = ctypes.c_int32()
    _check(load_library().fl_paged_attn_refused_launches(h, ctypes.byref(n)),
           "fl_paged_attn_refused_launches")
    return n.value


def fl_paged_attn_get_work_items(h) -> np.ndarray:
    """The current plan's work list as an int32 array [items, FL_WORK_ITEM_INTS]."""
    lib = load_library()
    n = ctypes.c_int32()
    _check(lib.fl_paged_attn_get_work_items(h, None, 0, ctypes.byref(n)),
           "fl_paged_attn_get_work_items")
    buf = np.zeros((max(n.value, 1), FL_WORK_ITEM_INTS), dtype=np.int32)
    _check(lib.fl_paged_attn_get_work_items(h, _p(buf), n.value, ctypes.byref(n)),
           "fl_paged_attn_get_work_items")
    return buf[:n.value]


def make_config(num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
                dtype: str, max_batch: int, max_qo_rows: int, max_kv_pages: int,
                num_cus: int = 0, groups_per_cu: int = 0, min_group_tokens: int = 0,
                waves_per_group: int = 0, max_tiles: int = 0, whole_rows: int = 0) -> fl_config:
    return fl_config(num_qo_heads, num_kv_heads, head_dim, page_size, DTYPE_CODES[dtype],
                     max_batch, max_qo_rows, max_kv_pages, num_cus, groups_per_cu,
                     min_group_tokens, waves_per_group, max_tiles, whole_rows)


class PagedAttention:
    """A handle plus torch plumbing: tensors in, pointers and the current stream out."""

    def __init__(self, cfg: fl_config, device: int = 0):
        self.cfg = cfg
        self.device = device
        self.handle = fl_paged_attn_create(cfg, device)

    def close(self):
        if self.handle is not None:
            fl_paged_attn_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _stream(self, stream):
        if stream is not None:
            return int(stream)
        if self.device < 0:
            return 0
        import torch
        return torch.cuda.current_stream(self.device).cuda_stream

    def plan(self, qo_indptr, kv_indptr, kv_indices, last_page_len, num_pages: int,
             causal: bool = True, sm_scale: float = 0.0, num_splits: int = 0, stream=None):
        batch = len(kv_indptr) - 1
        fl_paged_attn_plan(self.handle, batch, qo_indptr, kv_indptr, kv_indices, last_page_len,
                           num_pages, causal, sm_scale, num_splits, self._stream(stream))

    def run(self, q, k_pool, v_pool, out, lse=None, stream=None):
        fl_paged_attn_run(self.handle, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                          out.data_ptr(), None if lse is None else lse.data_ptr(),
                          self._stream(stream))

    def run_noalloc(self, q, k_pool, v_pool, out, lse=None, stream=None):
        if stream is None and self.device < 0:
            import torch
            stream = torch.cuda.current_stream().cuda_stream
        fl_paged_attn_run_noalloc(self.handle, q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                  out.data_ptr(), None if lse is None else lse.data_ptr(),
                                  self._stream(stream))

    def append(self, k_new, v_new, k_pool, v_pool, stream=None):
        fl_paged_kv_append(self.handle, k_new.data_ptr(), v_new.data_ptr(), k_pool.data_ptr(),
                           v_pool.data_ptr(), self._stream(stream))

    def append_rope(self, q, k_new, v_new, k_pool, v_pool, rope_theta, stream=None):
        fl_paged_kv_append_rope(self.handle, None if q is None else q.data_ptr(), k_new.data_ptr(),
                                v_new.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                float(rope_theta), self._stream(stream))

    def run_append(self, q, k_new, v_new, k_pool, v_pool, out, lse=None, stream=None):
        fl_paged_attn_run_append(self.handle, q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                 k_pool.data_ptr(), v_pool.data_ptr(), out.data_ptr(),
                                 None if lse is None else lse.data_ptr(), self._stream(stream))

    def append_slots(self) -> np.ndarray:
        return fl_paged_kv_append_slots(self.handle)

    def info(self):
        return fl_paged_attn_plan_info(self.handle)

    def work_items(self) -> np.ndarray:
        return fl_paged_attn_get_work_items(self.handle)

    def launch(self):
        return fl_paged_attn_plan_launch(self.handle)

    def refused_launches(self) -> int:
        return fl_paged_attn_refused_launches(self.handle)


# ---------------------------------------------------------------------------------------
# page allocator and freed-page poisoning (fl_page_pool.h)
# ---------------------------------------------------------------------------------------
def fl_page_pool_create(num_pages: int, page_size: int) -> ctypes.c_void_p:
    p = ctypes.c_void_p()
    _check(load_library().fl_page_pool_create(int(num_pages), int(page_size), ctypes.byref(p)),
           "fl_page_pool_create")
    return p


def fl_page_pool_destroy(p) -> None:
    _check(load_library().fl_page_pool_destroy(p), "fl_page_pool_destroy")


def fl_page_pool_alloc(p, n: int) -> np.ndarray:
    ids = np.zeros(max(int(n), 1), dtype=np.int32)
    _check(load_library().fl_page_pool_alloc(p, int(n), _p(ids)), "fl_page_pool_alloc")
    return ids[:int(n)]


def fl_page_pool_reserve(p, tokens: int, capacity: int = 1 << 20) -> np.ndarray:
    ids = np.zeros(max(int(capacity), 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(load_library().fl_page_pool_reserve(p, int(tokens), _p(ids), int(capacity),
                                               ctypes.byref(n)), "fl_page_pool_reserve")
    return ids[:n.value]


def fl_page_pool_retain(p, page_ids) -> None:
    ids = _i32(page_ids)
    _check(load_library().fl_page_pool_retain(p, _p(ids), int(ids.size)), "fl_page_pool_retain")


def fl_page_pool_release(p, page_ids) -> np.ndarray:
    """Returns the ids that became free, in the order their counts reached zero."""
    ids = _i32(page_ids)
    freed = np.zeros(max(ids.size, 1), dtype=np.int32)
    n = ctypes.c_int32()
    _check(load_library().fl_page_pool_release(p, _p(ids), int(ids.size), _p(freed), ctypes.byref(n)),
           "fl_page_pool_release")
    return freed[:n.value]


def fl_page_pool_refcounts(p, page_ids) -> np.ndarray:
    ids = _i32(page_ids)
    refs = np.zeros(max(ids.size, 1), dtype=np.int32)
    _check(load_library().fl_page_pool_refcounts(p, _p(ids), int(ids.size), _p(refs)),
           "fl_page_pool_refcounts")
    return refs[:ids.size]


def fl_page_pool_info(p) -> Tuple[int, int]:
    """(free pages, held pages)."""
    f, h = ctypes.c_int64(), ctypes.c_int64()
    _check(load_library().fl_page_pool_info(p, ctypes.byref(f), ctypes.byref(h)), "fl_page_pool_info")
    return f.value, h.value


def fl_paged_kv_poison(dtype: str, page_size: int, num_kv_heads: int, head_dim: int,
                       num_pages: int, page_ids, k_pool: int, v_pool: Optional[int] = None,
                       stream: int = 0) -> None:
    """Device pool pointers as integers; page ids a host array."""
    ids = _i32(page_ids)
    _check(load_library().fl_paged_kv_poison(DTYPE_CODES[dtype], int(page_size), int(num_kv_heads),
                                             int(head_dim), int(num_pages), _p(ids), int(ids.size),
                                             ctypes.c_void_p(k_pool), ctypes.c_void_p(v_pool or 0),
                                             ctypes.c_void_p(int(stream))),
           "fl_paged_kv_poison")


class PagePool:
    """The allocator handle with numpy in and out."""

    def __init__(self, num_pages: int, page_size: int):
        self.num_pages, self.page_size = int(num_pages), int(page_size)
        self.handle = fl_page_pool_create(num_pages, page_size)

    def close(self):
        if self.handle is not None:
            fl_page_pool_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def alloc(self, n: int) -> np.ndarray:
        return fl_page_pool_alloc(self.handle, n)

    def reserve(self, tokens: int) -> np.ndarray:
        return fl_page_pool_reserve(self.handle, tokens)

    def retain(self, page_ids) -> None:
        fl_page_pool_retain(self.handle, page_ids)

    def release(self, page_ids) -> np.ndarray:
        return fl_page_pool_release(self.handle, page_ids)

    def refcounts(self, page_ids) -> np.ndarray:
        return fl_page_pool_refcounts(self.handle, page_ids)

    def info(self) -> Tuple[int, int]:
        return fl_page_pool_info(self.handle)
