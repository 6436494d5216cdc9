"""Seeded synthetic batches for paged grouped-query attention (inputs only).

This module draws request lengths, page tables and q/K/V values. It holds none of
the attention arithmetic: the HIP library and the CPU oracle both take its arrays
as plain inputs, and neither imports the other.

Layout of what it produces (the NHD paged pool described in the flashlet README,
design bullets, and the page-table form of a paged KV cache):

* ``q``       ``[rows, num_qo_heads, head_dim]``; rows = ``qo_indptr[-1]``.
* ``k_pool``, ``v_pool``  ``[num_pages, page_size, num_kv_heads, head_dim]``.
* ``qo_indptr[B+1]``   prefix sums of query rows per request (ragged).
* ``kv_indptr[B+1]``   prefix sums of pages per request.
* ``kv_indices[nnz]``  physical page ids, request after request.
* ``last_page_len[B]`` valid slots in each request's last page, in ``[1, page_size]``.

Values are fp32 draws from N(0, 1) rounded to the storage type with
round-to-nearest-even. Half-precision storage is kept as raw 16-bit patterns
(``uint16`` for bf16, ``float16`` for fp16) so no host library reinterprets them.
Unused slots and unused pages hold NaN ("poison"), so any read of a slot outside
a request's history shows up in the result.

Random streams: ``numpy.random.Generator(PCG64(SeedSequence([seed, cfg_id,
stream])))`` with streams 0 lengths, 1 page permutation, 2 q, 3 k, 4 v. The
default seed is 0, the seed the decode write-up ("A library kernel for decode",
Setup paragraph) runs with.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

# Storage type codes shared with the C interfaces (fp16, bf16, fp32).
DTYPE_CODES = {"f16": 1, "bf16": 2, "f32": 3}
STREAM_LENGTHS, STREAM_PAGES, STREAM_Q, STREAM_K, STREAM_V = 0, 1, 2, 3, 4


def rng_for(seed: int, cfg_id: int, stream: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, cfg_id, stream])))


# ---------------------------------------------------------------------------
# storage conversion (input quantisation only)
# ---------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (round-to-nearest-even), return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    nan = np.isnan(np.asarray(x, dtype=np.float32))
    r = ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)
    if nan.any():
        r = np.where(nan, np.uint16(0x7FC0), r)
    return r


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "f16":
        return np.asarray(x, dtype=np.float32).astype(np.float16)
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    raise ValueError(f"unknown dtype {dtype!r}")


def storage_to_f32(a: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_bits_to_f32(a)
    return np.asarray(a).astype(np.float32)


def storage_np_dtype(dtype: str):
    return {"bf16": np.uint16, "f16": np.float16, "f32": np.float32}[dtype]


def poison_value(dtype: str):
    if dtype == "bf16":
        return np.uint16(0x7FC0)
    if dtype == "f16":
        return np.float16(np.nan)
    return np.float32(np.nan)


# ---------------------------------------------------------------------------
# the batch
# ---------------------------------------------------------------------------
@dataclass
class Batch:
    name: str
    dtype: str
    num_qo_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    causal: bool
    sm_scale: float
    qo_indptr: np.ndarray
    kv_indptr: np.ndarray
    kv_indices: np.ndarray
    last_page_len: np.ndarray
    q: np.ndarray
    k_pool: np.ndarray
    v_pool: np.ndarray
    kv_lens: np.ndarray
    qo_lens: np.ndarray
    seed: int = 0
    cfg_id: int = 0
    dense_k: Optional[List[np.ndarray]] = field(default=None, repr=False)
    dense_v: Optional[List[np.ndarray]] = field(default=None, repr=False)

    @property
    def batch_size(self) -> int:
        return int(self.kv_lens.shape[0])

    @property
    def group(self) -> int:
        return self.num_qo_heads // self.num_kv_heads

    @property
    def rows(self) -> int:
        return int(self.qo_indptr[-1])

    @property
    def dtype_code(self) -> int:
        return DTYPE_CODES[self.dtype]

    @property
    def elem_bytes(self) -> int:
        return 4 if self.dtype == "f32" else 2

    def kv_bytes(self) -> int:
        """Algorithmic K+V bytes one call must read: token-granular, every request."""
        return int(self.kv_lens.sum()) * self.num_kv_heads * self.head_dim * 2 * self.elem_bytes

    def attn_flops(self) -> int:
        """Multiply-add flops over unmasked (query, key) pairs: 4*D per pair and head."""
        pairs = 0
        for ql, kl in zip(self.qo_lens.tolist(), self.kv_lens.tolist()):
            if self.causal:
                pairs += sum(kl - ql + i + 1 for i in range(ql))
            else:
                pairs += ql * kl
        return pairs * self.num_qo_heads * 4 * self.head_dim


def page_table(kv_lens: Sequence[int], page_size: int, num_pages: int, rng: np.random.Generator,
               shuffle: bool = True):
    """Pages for each request, taken in order from a seeded permutation of the pool."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    if np.any(kv_lens < 1):
        raise ValueError("every request needs at least one cached token")
    npages = (kv_lens + page_size - 1) // page_size
    need = int(npages.sum())
    if need > num_pages:
        raise ValueError(f"pool of {num_pages} pages cannot hold {need}")
    order = rng.permutation(num_pages) if shuffle else np.arange(num_pages)
    kv_indices = order[:need].astype(np.int32)
    kv_indptr = np.zeros(len(kv_lens) + 1, dtype=np.int32)
    kv_indptr[1:] = np.cumsum(npages)
    last = (kv_lens - (npages - 1) * page_size).astype(np.int32)
    return kv_indptr, kv_indices, last


def scatter_tokens(pool: np.ndarray, dense: np.ndarray, kv_indptr, kv_indices, kv_lens, page_size):
    """Write concatenated per-request rows ``dense[sum(kv_len), Hkv, D]`` into their page slots."""
    kv_lens = np.asarray(kv_lens, dtype=np.int64)
    req = np.repeat(np.arange(len(kv_lens)), kv_lens)
    starts = np.concatenate([[0], np.cumsum(kv_lens)[:-1]])
    t = np.arange(int(kv_lens.sum())) - np.repeat(starts, kv_lens)
    pages = np.asarray(kv_indices)[np.asarray(kv_indptr)[req] + t // page_size]
    pool[pages, t % page_size] = dense


def make_batch(kv_lens: Sequence[int], qo_lens: Optional[Sequence[int]] = None, *,
               num_qo_heads: int, num_kv_heads: int, head_dim: int, page_size: int,
               dtype: str = "bf16", num_pages: Optional[int] = None, seed: int = 0,
               cfg_id: int = 0, causal: bool = True, sm_scale: Optional[float] = None,
               name: str = "custom", keep_dense: bool = False, shuffle_pages: bool = True,
               poison: bool = True) -> Batch:
    kv_lens = np.asarray(kv_lens, dtype=np.int32)
    B = int(kv_lens.shape[0])
    qo_lens = np.ones(B, dtype=np.int32) if qo_lens is None else np.asarray(qo_lens, dtype=np.int32)
    if num_qo_heads % num_kv_heads:
        raise ValueError("num_qo_heads must be a multiple of num_kv_heads")
    npages_needed = int(((kv_lens.astype(np.int64) + page_size - 1) // page_size).sum())
    if num_pages is None:
        num_pages = max(1, npages_needed)
    kv_indptr, kv_indices, last = page_table(kv_lens, page_size, num_pages,
                                             rng_for(seed, cfg_id, STREAM_PAGES), shuffle_pages)
    qo_indptr = np.zeros(B + 1, dtype=np.int32)
    qo_indptr[1:] = np.cumsum(qo_lens)
    rows = int(qo_indptr[-1])
    Hq, Hkv, D = num_qo_heads, num_kv_heads, head_dim
    q = to_storage(rng_for(seed, cfg_id, STREAM_Q).standard_normal((rows, Hq, D), dtype=np.float32), dtype)
    tot = int(kv_lens.sum())
    k_all = to_storage(rng_for(seed, cfg_id, STREAM_K).standard_normal((tot, Hkv, D), dtype=np.float32), dtype)
    v_all = to_storage(rng_for(seed, cfg_id, STREAM_V).standard_normal((tot, Hkv, D), dtype=np.float32), dtype)
    sd = storage_np_dtype(dtype)
    fill = poison_value(dtype) if poison else sd(0)
    k_pool = np.full((num_pages, page_size, Hkv, D), fill, dtype=sd)
    v_pool = np.full((num_pages, page_size, Hkv, D), fill, dtype=sd)
    scatter_tokens(k_pool, k_all, kv_indptr, kv_indices, kv_lens, page_size)
    scatter_tokens(v_pool, v_all, kv_indptr, kv_indices, kv_lens, page_size)
    dk = dv = None
    if keep_dense:
        cuts = np.cumsum(kv_lens)[:-1]
        dk = np.split(k_all, cuts)
        dv = np.split(v_all, cuts)
    scale = float(1.0 / np.sqrt(D)) if sm_scale is None else float(sm_scale)
    return Batch(name=name, dtype=dtype, num_qo_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                 page_size=page_size, num_pages=num_pages, causal=causal, sm_scale=scale,
                 qo_indptr=qo_indptr, kv_indptr=kv_indptr, kv_indices=kv_indices,
                 last_page_len=last, q=q, k_pool=k_pool, v_pool=v_pool, kv_lens=kv_lens,
                 qo_lens=qo_lens, seed=seed, cfg_id=cfg_id, dense_k=dk, dense_v=dv)


@dataclass
class AppendStep:
    """A step's new K/V rows and the pools as they were before the step.

    The batch's pools hold every request's whole history; here the newest qo_len tokens
    of each request (the tokens its query rows stand for) are taken out of them:
    ``k_new`` / ``v_new`` ``[rows, Hkv, D]`` hold those tokens in query-row order and
    ``k_before`` / ``v_before`` are the pools with their slots poisoned. Writing the new
    rows back gives the batch's pools again."""
    k_new: np.ndarray
    v_new: np.ndarray
    k_before: np.ndarray
    v_before: np.ndarray


def append_step(b: Batch) -> AppendStep:
    """Split a batch made with ``keep_dense=True`` into pools before the step and new rows."""
    if b.dense_k is None:
        raise ValueError("append_step needs a batch made with keep_dense=True")
    if np.any(b.qo_lens > b.kv_lens):
        raise ValueError("every request needs qo_len <= kv_len")
    pre = (b.kv_lens - b.qo_lens).astype(np.int64)
    sd = storage_np_dtype(b.dtype)
    fill = poison_value(b.dtype)
    shape = b.k_pool.shape
    k_before = np.full(shape, fill, dtype=sd)
    v_before = np.full(shape, fill, dtype=sd)
    k_old = np.concatenate([k[:n] for k, n in zip(b.dense_k, pre)])
    v_old = np.concatenate([v[:n] for v, n in zip(b.dense_v, pre)])
    scatter_tokens(k_before, k_old, b.kv_indptr, b.kv_indices, pre, b.page_size)
    scatter_tokens(v_before, v_old, b.kv_indptr, b.kv_indices, pre, b.page_size)
    tail = [(k[n:], v[n:]) for k, v, n in zip(b.dense_k, b.dense_v, pre)]
    empty = np.zeros((0, b.num_kv_heads, b.head_dim), dtype=sd)
    k_new = np.concatenate([t[0] for t in tail] + [empty])
    v_new = np.concatenate([t[1] for t in tail] + [empty])
    return AppendStep(k_new=np.ascontiguousarray(k_new), v_new=np.ascontiguousarray(v_new),
                      k_before=k_before, v_before=v_before)


def relabel_pages(b: Batch, perm: np.ndarray) -> Batch:
    """The same logical batch with physical page p moved to ``perm[p]``."""
    perm = np.asarray(perm, dtype=np.int64)
    k = np.empty_like(b.k_pool)
    v = np.empty_like(b.v_pool)
    k[perm] = b.k_pool
    v[perm] = b.v_pool
    out = Batch(**{**b.__dict__})
    out.k_pool, out.v_pool = k, v
    out.kv_indices = perm[b.kv_indices].astype(np.int32)
    return out


# ---------------------------------------------------------------------------
# the five workloads (the pages' shapes; lengths drawn from stream 0)
# ---------------------------------------------------------------------------
def tiny_decode(seed: int = 0, dtype: str = "bf16", page_size: int = 16, keep_dense: bool = False,
                num_pages: Optional[int] = None) -> Batch:
    """4 requests with 1, 17, 100 and 300 cached tokens; 14 q / 2 kv heads, d 64."""
    if num_pages is None:
        num_pages = 64 if page_size == 16 else -(-418 // page_size) + 8
    return make_batch([1, 17, 100, 300], num_qo_heads=14, num_kv_heads=2, head_dim=64,
                      page_size=page_size, dtype=dtype, num_pages=num_pages, seed=seed, cfg_id=1,
                      name="tiny_decode", keep_dense=keep_dense)


def saturated_decode(seed: int = 0, dtype: str = "bf16", keep_dense: bool = False) -> Batch:
    """128 requests x 300 cached tokens, 14 q / 2 kv heads, d 64, 16-slot pages, 8192-page pool."""
    return make_batch([300] * 128, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                      dtype=dtype, num_pages=8192, seed=seed, cfg_id=2, name="saturated_decode",
                      keep_dense=keep_dense)


def mixed_length_lengths(seed: int = 0, n: int = 32) -> np.ndarray:
    rng = rng_for(seed, 3, STREAM_LENGTHS)
    prompts = rng.choice(np.array([16, 64, 256, 1024, 4096]), size=n)
    gen = rng.integers(64, 256, size=n, endpoint=True)
    return (prompts + gen).astype(np.int32)


def mixed_length_decode(seed: int = 0, dtype: str = "f16", keep_dense: bool = False) -> Batch:
    """32 requests, prompt in {16,64,256,1024,4096} plus 64-256 generated tokens; 12 q / 2 kv
    heads, d 128, 256-slot pages, 1024-page pool."""
    return make_batch(mixed_length_lengths(seed), num_qo_heads=12, num_kv_heads=2, head_dim=128,
                      page_size=256, dtype=dtype, num_pages=1024, seed=seed, cfg_id=3,
                      name="mixed_length_decode", keep_dense=keep_dense)


def long_context_lengths(seed: int = 0, long_len: int = 32768, short_len: int = 512,
                         n_long: int = 8, n_short: int = 56) -> np.ndarray:
    lens = np.array([long_len] * n_long + [short_len] * n_short, dtype=np.int32)
    return lens[rng_for(seed, 4, STREAM_LENGTHS).permutation(len(lens))]


def long_context_skew(seed: int = 0, dtype: str = "f16", keep_dense: bool = False,
                      long_len: int = 32768) -> Batch:
    """64 requests: 8 with 32768 cached tokens and 56 with 512 (order shuffled); 12 q / 2 kv
    heads, d 128, 256-slot pages, 2048-page pool."""
    lens = long_context_lengths(seed, long_len=long_len)
    pages = max(2048, int(((lens + 255) // 256).sum()))
    return make_batch(lens, num_qo_heads=12, num_kv_heads=2, head_dim=128, page_size=256,
                      dtype=dtype, num_pages=pages, seed=seed, cfg_id=4, name="long_context_skew",
                      keep_dense=keep_dense)


def ragged_mixed_lengths(seed: int = 0):
    rng = rng_for(seed, 5, STREAM_LENGTHS)
    dec = rng.integers(32, 768, size=127, endpoint=True).astype(np.int32)
    kv = np.concatenate([[1536], dec]).astype(np.int32)
    qo = np.concatenate([[512], np.ones(127, dtype=np.int32)]).astype(np.int32)
    return kv, qo


def ragged_mixed_step(seed: int = 0, dtype: str = "bf16", keep_dense: bool = False) -> Batch:
    """One 512-row causal prefill chunk over 1536 cached tokens (1024 before the chunk) plus 127
    decode rows with contexts uniform in [32, 768]; 14 q / 2 kv heads, d 64, 16-slot pages."""
    kv, qo = ragged_mixed_lengths(seed)
    return make_batch(kv, qo, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                      dtype=dtype, num_pages=8192, seed=seed, cfg_id=5, name="ragged_mixed_step",
                      keep_dense=keep_dense)


def multi_chunk_lengths(seed: int = 0, chunks: int = 4, chunk_rows: int = 128, decodes: int = 124):
    """Several prefill chunks sharing one 512-token budget with decode rows: 4 chunks of 128
    rows, each on top of 256..2048 cached tokens, plus 124 decode rows with contexts uniform
    in [32, 768]; chunk requests first."""
    rng = rng_for(seed, 6, STREAM_LENGTHS)
    cached = rng.integers(256, 2048, size=chunks, endpoint=True).astype(np.int32)
    dec = rng.integers(32, 768, size=decodes, endpoint=True).astype(np.int32)
    kv = np.concatenate([cached + chunk_rows, dec]).astype(np.int32)
    qo = np.concatenate([np.full(chunks, chunk_rows), np.ones(decodes)]).astype(np.int32)
    return kv, qo


def multi_chunk_step(seed: int = 0, dtype: str = "bf16", keep_dense: bool = False) -> Batch:
    """Four 128-row causal prefill chunks (on 256..2048 cached tokens each) plus 124 decode rows
    in one ragged call; 14 q / 2 kv heads, d 64, 16-slot pages, 8192-page pool."""
    kv, qo = multi_chunk_lengths(seed)
    return make_batch(kv, qo, num_qo_heads=14, num_kv_heads=2, head_dim=64, page_size=16,
                      dtype=dtype, num_pages=8192, seed=seed, cfg_id=6, name="multi_chunk_step",
                      keep_dense=keep_dense)


WORKLOADS = {
    "tiny_decode": tiny_decode,
    "saturated_decode": saturated_decode,
    "mixed_length_decode": mixed_length_decode,
    "long_context_skew": long_context_skew,
    "ragged_mixed_step": ragged_mixed_step,
    "multi_chunk_step": multi_chunk_step,
}
