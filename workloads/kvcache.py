"""Seeded synthetic decode steps against a paged KV cache.

A case holds packed queries (the few new tokens of each sequence) and a
paged cache: ``[num_pages, page_size, Hkv, d]`` K and V with a block table
``[B, max_pages_per_seq]`` (int32) and the cached length of each sequence.
The pages of every sequence are a random permutation of the pool, so no
sequence's keys are contiguous; slots no sequence owns (the tail of each
sequence's last page and the spare pages) hold NaN, and block-table entries
past a sequence's last page hold -1, so a kernel that read them would show
it.  Values are N(0, 1) draws rounded to the case's dtype, as in
``generate.py``.  Nothing here computes attention.
"""

from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .generate import _cu, _draw, _rng

STREAM_PAGES = 20


@dataclass
class KVCase:
    name: str
    dtype: str
    causal: bool
    hq: int
    hkv: int
    d: int
    scale: float
    page_size: int
    lens_q: np.ndarray
    lens_k: np.ndarray
    q: np.ndarray            # [total_q, hq, d] float32
    k_cache: np.ndarray      # [num_pages, page_size, hkv, d] float32
    v_cache: np.ndarray
    block_table: np.ndarray  # [batch, max_pages] int32, -1 past each sequence's pages
    seqlens_k: np.ndarray    # [batch] int32

    @property
    def batch(self) -> int:
        return len(self.lens_q)

    @property
    def cu_q(self) -> np.ndarray:
        return _cu(self.lens_q)

    @property
    def total_q(self) -> int:
        return int(self.lens_q.sum())

    @property
    def max_q(self) -> int:
        return int(self.lens_q.max()) if self.batch else 0

    @property
    def max_k(self) -> int:
        return int(self.lens_k.max()) if self.batch else 0

    @property
    def num_pages(self) -> int:
        return self.k_cache.shape[0]

    def kv_bytes(self) -> int:
        """Bytes of K and V the step must read: every cached key of every KV head, once."""
        elt = 4 if self.dtype == "f32" else 2
        return int(self.lens_k.sum()) * self.hkv * self.d * elt * 2


def page_layout(seed: int, lens_k: Sequence[int], page_size: int, spare_pages: int = 3,
                max_pages: Optional[int] = None):
    """Random page assignment: (block_table [B, max_pages] int32 with -1 past each sequence's
    pages, number of pages in the pool).  The pool's pages are handed out in the order of a
    seeded permutation."""
    if page_size <= 0:
        raise ValueError("page_size must be positive")
    need = [int(math.ceil(int(n) / page_size)) for n in lens_k]
    mp = max(need + [1]) if max_pages is None else int(max_pages)
    if mp < max(need + [0]):
        raise ValueError("max_pages smaller than a sequence's page count")
    n_pages = max(sum(need) + int(spare_pages), 1)
    perm = _rng(300, int(seed), STREAM_PAGES).permutation(n_pages).astype(np.int32)
    bt = np.full((len(need), mp), -1, dtype=np.int32)
    p = 0
    for b, n in enumerate(need):
        bt[b, :n] = perm[p:p + n]
        p += n
    return bt, n_pages


def kvcache_case(seed: int, lens_q: Sequence[int], lens_k: Sequence[int], hq: int = 8, hkv: int = 2,
                 d: int = 64, causal: bool = True, dtype: str = "bf16", page_size: int = 16,
                 spare_pages: int = 3, max_pages: Optional[int] = None,
                 scale: Optional[float] = None, name: Optional[str] = None) -> KVCase:
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(dtype)
    lens_q = np.asarray(list(lens_q), dtype=np.int64)
    lens_k = np.asarray(list(lens_k), dtype=np.int64)
    if len(lens_q) != len(lens_k):
        raise ValueError("lens_q and lens_k differ in batch")
    bt, n_pages = page_layout(seed, lens_k, page_size, spare_pages, max_pages)
    base = (300, int(seed))
    q = _draw(_rng(*base, 1), (int(lens_q.sum()), hq, d), dtype)
    kv_rows = int(lens_k.sum())
    k_rows = _draw(_rng(*base, 2), (kv_rows, hkv, d), dtype)
    v_rows = _draw(_rng(*base, 3), (kv_rows, hkv, d), dtype)
    k_cache = np.full((n_pages, page_size, hkv, d), np.nan, dtype=np.float32)
    v_cache = np.full_like(k_cache, np.nan)
    row = 0
    for b in range(len(lens_q)):
        n = int(lens_k[b])
        j = np.arange(n)
        pages = bt[b, j // page_size]
        k_cache[pages, j % page_size] = k_rows[row:row + n]
        v_cache[pages, j % page_size] = v_rows[row:row + n]
        row += n
    sc = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    return KVCase(name=name or f"kvcache seed={seed}", dtype=dtype, causal=causal, hq=hq, hkv=hkv, d=d,
                  scale=sc, page_size=page_size, lens_q=lens_q, lens_k=lens_k, q=q, k_cache=k_cache,
                  v_cache=v_cache, block_table=bt, seqlens_k=lens_k.astype(np.int32))


# The decode-step workload: a serving batch of 128 sequences, one new token each, cached
# lengths uniform in [1, 4096], the 32 query / 8 KV heads of head_dim 128 of the short
# GQA shape on the ASpec pull request 25 page (section "Verification"), bf16, pages of 64
# keys handed out in random order (``page_layout``).  At this size the values are drawn
# on the device by the bench; ``kvcache_case`` draws them on the host for tests.
DECODE_BATCH = 128
DECODE_MAX_K = 4096


def decode_lengths(seed: int = 11, batch: int = DECODE_BATCH, max_k: int = DECODE_MAX_K) -> np.ndarray:
    """Cached lengths of the decode-step workload: uniform integers in [1, max_k]."""
    return _rng(400, int(seed)).integers(1, max_k + 1, size=batch).astype(np.int64)


DECODE_SHAPE = dict(hq=32, hkv=8, d=128, causal=True, page_size=64)


def decode_device_inputs(device, seed: int = 11) -> dict:
    """The decode-step workload on ``device``: lengths and pages from the seeded layout, Q and
    the caches N(0, 1) drawn on the device from a seeded generator and rounded to bf16, the
    slots past each sequence's last key set to NaN.  Keys: lens_k, bt (host), n_pages, q, kc,
    vc, cu, sk, btd (device)."""
    import torch

    lens_k = decode_lengths(seed)
    B = len(lens_k)
    sh = DECODE_SHAPE
    ps = sh["page_size"]
    bt, n_pages = page_layout(seed, lens_k, ps, 0)
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    q = torch.randn((B, sh["hq"], sh["d"]), generator=g, device=device).to(torch.bfloat16)
    caches = [torch.randn((n_pages, ps, sh["hkv"], sh["d"]), generator=g, device=device).to(torch.bfloat16)
              for _ in range(2)]
    for b in range(B):
        n = int(lens_k[b])
        if n % ps:
            for cache in caches:
                cache[int(bt[b, n // ps]), n % ps:] = float("nan")
    return dict(lens_k=lens_k, bt=bt, n_pages=n_pages, q=q, kc=caches[0], vc=caches[1],
                cu=torch.arange(B + 1, dtype=torch.int32, device=device),
                sk=torch.from_numpy(lens_k.astype(np.int32)).to(device),
                btd=torch.from_numpy(bt).to(device))
