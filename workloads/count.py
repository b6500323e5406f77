"""Exact work counts for packed attention: visible pairs, non-padded FLOPs, algorithmic bytes.

The TorchEasyRec pull request 663 page (section "Choosing the kernel") prices
attention in score pairs: the packed stream behind a dense mask costs the
square of the total length, a left-padded batch costs rows times the longest
row squared, and the varlen kernel costs the sum of the per-sequence squares.
Its worked example (8 rows of 128) gives 1,048,576 and 131,072 pairs.  The
counters here count only the pairs the method must evaluate: the visible
(query, key) pairs of each sequence, with causal visibility aligned to the
bottom-right corner (key j visible to query i iff j <= i + Lk - Lq).

FLOPs (non-padded): forward 4*d per visible pair and query head (two
contractions, QK^T and PV), backward 10*d (five contractions).  Softmax,
bias and mask work and any tile padding are not counted.
"""

from __future__ import annotations

import numpy as np


def visible_pairs(lq: int, lk: int, causal: bool) -> int:
    """Number of visible (i, j) with 0 <= i < lq, 0 <= j < lk."""
    lq, lk = int(lq), int(lk)
    if lq <= 0 or lk <= 0:
        return 0
    if not causal:
        return lq * lk
    off = lk - lq
    # n(i) = clamp(i + off + 1, 0, lk); sum over i in [0, lq)
    i = np.arange(lq, dtype=np.int64)
    return int(np.clip(i + off + 1, 0, lk).sum())


def workload_pairs(lens_q, lens_k, causal: bool) -> int:
    """Visible pairs per head, summed over the packed sequences."""
    return int(sum(visible_pairs(a, b, causal) for a, b in zip(lens_q, lens_k)))


def dense_mask_pairs(lens) -> int:
    """Score pairs of the whole stream behind one dense (T, T) mask: (sum L)^2."""
    t = int(np.sum(lens))
    return t * t


def padded_pairs(lens) -> int:
    """Score pairs of a left-padded batch: rows * (max L)^2."""
    lens = list(lens)
    return len(lens) * int(max(lens)) ** 2 if lens else 0


def fwd_flops(w) -> int:
    return 4 * w.d * w.hq * workload_pairs(w.lens_q, w.lens_k, w.causal)


def bwd_flops(w) -> int:
    return 10 * w.d * w.hq * workload_pairs(w.lens_q, w.lens_k, w.causal)


def _elt(dtype: str) -> int:
    return 4 if dtype == "f32" else 2


def _bias_bytes(w) -> int:
    """Valid bias elements (r < Lq_b, c < Lk_b) read once, in the input dtype."""
    if w.bias is None:
        return 0
    s0, s1, s2, s3 = w.bias_strides
    heads = w.hq if s1 != 0 else 1
    n = 0
    for lq, lk in zip(w.lens_q, w.lens_k):
        if lq <= 0 or lk <= 0:
            continue
        rows = 1 if s2 == 0 else int(lq)
        n += heads * rows * int(lk)
    return n * _elt(w.dtype)


def fwd_bytes(w) -> int:
    """Algorithmic HBM bytes of one forward: read Q, K, V, bias once; write O and LSE once."""
    e = _elt(w.dtype)
    tq, tk = w.total_q, w.total_k
    b = (tq * w.hq * w.d + 2 * tk * w.hkv * w.d + tq * w.hq * w.d) * e
    b += tq * w.hq * 4  # LSE
    b += 2 * (w.batch + 1) * 4  # cu_seqlens
    return b + _bias_bytes(w)


def bwd_bytes(w, grad_dtype: str = "f32") -> int:
    """Algorithmic HBM bytes of one backward: read Q, K, V, O, dO, LSE, bias; write dQ, dK, dV."""
    e = _elt(w.dtype)
    g = _elt(grad_dtype)
    tq, tk = w.total_q, w.total_k
    b = (3 * tq * w.hq * w.d + 2 * tk * w.hkv * w.d) * e  # Q, O, dO, K, V
    b += tq * w.hq * 4  # LSE
    b += (tq * w.hq * w.d + 2 * tk * w.hkv * w.d) * g  # dQ, dK, dV
    b += 2 * (w.batch + 1) * 4
    return b + _bias_bytes(w)
