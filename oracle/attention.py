"""CPU fp64 oracle for exact attention over packed variable-length sequences.

TEST INFRASTRUCTURE.  This module is the slow, plainly written definition the
GPU path is checked against.  Only ``tests/``, the smoke check in
``__graft_entry__`` and the CPU-baseline leg of ``bench.py`` may import it.
It shares no code with the HIP library or its Python binding, and neither
side imports the other.

What it computes (the subject the five pages turn on: FlashAttention-2's
varlen kernel on the TorchEasyRec pull request 663 page, intro and section
"Choosing the kernel"; the per-sequence strided bias of the GiGL pull request
858 page, section "Approach"; the cross-length GQA shape of the ASpec pull
request 25 page, section "Verification"):

For every sequence ``b`` of the packed stream (rows ``cu_q[b]:cu_q[b+1]`` of
Q and ``cu_k[b]:cu_k[b+1]`` of K and V) and every query head ``h``, with KV
head ``g = h // (Hq / Hkv)`` (contiguous GQA groups):

    S  = scale * Q_b,h K_b,g^T + Bias_b,h        (Lq x Lk)
    S[i, j] = -inf  where causal and j > i + (Lk - Lq)    (bottom-right aligned)
    P  = row softmax of S;  O = P V_b,g;  LSE_i = log sum_j exp(S[i, j])

A row with no visible key gives O = 0 and LSE = -inf.  The bias element of
(b, h, r, c) lives at flat offset ``b*s0 + h*s1 + r*s2 + c*s3`` with ``r`` and
``c`` local to the sequence (the GiGL page indexes sequence i's bias at
i * stride(0) through a strided view).  Everything runs in float64 on the
stored input values (bf16 inputs upcast exactly).

Gradients (given dO), the analytic chain rule through the softmax:

    dP = dO V^T;  D_i = sum_j P_ij dP_ij;  dS = P * (dP - D)
    dQ = scale * dS K;  dK = scale * dS^T Q;  dV = P^T dO

with dK and dV summed over the query heads that share a KV head.  The bias
is added to the logits, so its gradient is dS itself, summed over every axis
the bias is broadcast along (``bias_grad``).  The GiGL pull request 858 page
(section "Approach") notes that the varlen kernel it calls has no backward for
a per-sequence bias, which sends biased training to the padded path.

Pins: ``tests/test_oracle_pins.py`` checks every function here against brute
force, a library SDPA in float64, closed forms, invariants and finite
differences.
"""

from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=np.float64)


def visible(lq: int, lk: int, causal: bool) -> np.ndarray:
    """Boolean (lq, lk) visibility; causal keeps key j for query i iff j <= i + lk - lq."""
    if not causal:
        return np.ones((lq, lk), dtype=bool)
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return j <= i + (lk - lq)


def bias_tile(bias, strides, b: int, h: int, lq: int, lk: int):
    """The (lq, lk) float64 bias block of sequence b, query head h (None if no bias)."""
    if bias is None:
        return None
    s0, s1, s2, s3 = (int(s) for s in strides)
    r = np.arange(lq, dtype=np.int64)[:, None]
    c = np.arange(lk, dtype=np.int64)[None, :]
    idx = b * s0 + h * s1 + r * s2 + c * s3
    return _f64(np.asarray(bias)[idx])


def head_forward(qb, kb, vb, scale: float, causal: bool, bias_bh=None):
    """One sequence, one query head.  Returns (O [lq, d], LSE [lq])."""
    qb, kb, vb = _f64(qb), _f64(kb), _f64(vb)
    lq, lk = qb.shape[0], kb.shape[0]
    out = np.zeros((lq, vb.shape[1]))
    lse = np.full(lq, -np.inf)
    if lq == 0 or lk == 0:
        return out, lse
    s = float(scale) * (qb @ kb.T)
    if bias_bh is not None:
        s = s + bias_bh
    vis = visible(lq, lk, causal)
    s = np.where(vis, s, -np.inf)
    rows = vis.any(axis=1)
    if rows.any():
        sr = s[rows]
        m = sr.max(axis=1, keepdims=True)
        e = np.exp(sr - m)
        l = e.sum(axis=1, keepdims=True)
        p = e / l
        out[rows] = p @ vb
        lse[rows] = m[:, 0] + np.log(l[:, 0])
    return out, lse


def head_probs(qb, kb, scale: float, causal: bool, bias_bh=None) -> np.ndarray:
    """Softmax matrix P (lq, lk) of one sequence and head; empty rows are all zero."""
    qb, kb = _f64(qb), _f64(kb)
    lq, lk = qb.shape[0], kb.shape[0]
    p = np.zeros((lq, lk))
    if lq == 0 or lk == 0:
        return p
    s = float(scale) * (qb @ kb.T)
    if bias_bh is not None:
        s = s + bias_bh
    vis = visible(lq, lk, causal)
    s = np.where(vis, s, -np.inf)
    rows = vis.any(axis=1)
    if rows.any():
        sr = s[rows]
        e = np.exp(sr - sr.max(axis=1, keepdims=True))
        p[rows] = e / e.sum(axis=1, keepdims=True)
    return p


def head_logit_grad(qb, kb, vb, dob, scale: float, causal: bool, bias_bh=None):
    """dS (lq, lk): the gradient of sum(dO * O) w.r.t. the logits S = scale Q K^T + bias of
    one sequence and head (zero where the mask hides a pair)."""
    qb, kb, vb, dob = _f64(qb), _f64(kb), _f64(vb), _f64(dob)
    p = head_probs(qb, kb, scale, causal, bias_bh)
    dp = dob @ vb.T
    dsum = (p * dp).sum(axis=1, keepdims=True)
    ds = p * (dp - dsum)
    return p, ds


def head_backward(qb, kb, vb, dob, scale: float, causal: bool, bias_bh=None):
    """One sequence, one query head.  Returns (dQ [lq, d], dK [lk, d], dV [lk, d])."""
    qb, kb, vb, dob = _f64(qb), _f64(kb), _f64(vb), _f64(dob)
    p, ds = head_logit_grad(qb, kb, vb, dob, scale, causal, bias_bh)
    dq = float(scale) * (ds @ kb)
    dk = float(scale) * (ds.T @ qb)
    dv = p.T @ dob
    return dq, dk, dv


def _check(q, k, v, cu_q, cu_k):
    q, k, v = np.asarray(q), np.asarray(k), np.asarray(v)
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    hq, hkv = q.shape[1], k.shape[1]
    if hkv == 0 or hq % hkv:
        raise ValueError("query heads must be a multiple of KV heads")
    cu_q = np.asarray(cu_q, dtype=np.int64)
    cu_k = np.asarray(cu_k, dtype=np.int64)
    if len(cu_q) != len(cu_k):
        raise ValueError("cu_seqlens_q and cu_seqlens_k differ in length")
    return q, k, v, cu_q, cu_k, hq // hkv


def sequence_head_forward(q, k, v, cu_q, cu_k, scale, causal, bias, bias_strides, b: int, h: int):
    """(O, LSE) of sequence b, query head h, taken from the packed stream."""
    q, k, v, cu_q, cu_k, n_rep = _check(q, k, v, cu_q, cu_k)
    q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
    g = h // n_rep
    bb = bias_tile(bias, bias_strides, b, h, q1 - q0, k1 - k0)
    return head_forward(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], scale, causal, bb)


def forward(q, k, v, cu_q, cu_k, scale, causal, bias=None, bias_strides=None):
    """Packed forward.  Returns (out [Tq, Hq, d] float64, lse [Hq, Tq] float64)."""
    q, k, v, cu_q, cu_k, n_rep = _check(q, k, v, cu_q, cu_k)
    tq, hq, d = q.shape
    out = np.zeros((tq, hq, v.shape[2]))
    lse = np.full((hq, tq), -np.inf)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        if q1 <= q0:
            continue
        for h in range(hq):
            g = h // n_rep
            bb = bias_tile(bias, bias_strides, b, h, q1 - q0, k1 - k0)
            o, l = head_forward(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], scale, causal, bb)
            out[q0:q1, h] = o
            lse[h, q0:q1] = l
    return out, lse


def sequence_group_backward(dout, q, k, v, cu_q, cu_k, scale, causal, bias, bias_strides,
                            b: int, g: int):
    """Gradients of sequence b for KV head g and its query heads.

    Returns (dq [Lq, n_rep, d], dk [Lk, d], dv [Lk, d]); dq's middle axis is
    the query heads g*n_rep .. g*n_rep + n_rep - 1.
    """
    q, k, v, cu_q, cu_k, n_rep = _check(q, k, v, cu_q, cu_k)
    dout = np.asarray(dout)
    q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
    lq, lk = q1 - q0, k1 - k0
    d = q.shape[2]
    dq = np.zeros((lq, n_rep, d))
    dk = np.zeros((lk, d))
    dv = np.zeros((lk, v.shape[2]))
    for r in range(n_rep):
        h = g * n_rep + r
        bb = bias_tile(bias, bias_strides, b, h, lq, lk)
        a, bk, bv = head_backward(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], dout[q0:q1, h],
                                  scale, causal, bb)
        dq[:, r] = a
        dk += bk
        dv += bv
    return dq, dk, dv


def backward(dout, q, k, v, cu_q, cu_k, scale, causal, bias=None, bias_strides=None):
    """Packed backward.  Returns float64 (dq [Tq, Hq, d], dk [Tk, Hkv, d], dv [Tk, Hkv, d])."""
    q, k, v, cu_q, cu_k, n_rep = _check(q, k, v, cu_q, cu_k)
    tq, hq, d = q.shape
    tk, hkv, dv_ = v.shape
    dq = np.zeros((tq, hq, d))
    dk = np.zeros((tk, hkv, d))
    dv = np.zeros((tk, hkv, dv_))
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        for g in range(hkv):
            a, bk, bv = sequence_group_backward(dout, q, k, v, cu_q, cu_k, scale, causal,
                                                bias, bias_strides, b, g)
            dq[q0:q1, g * n_rep:(g + 1) * n_rep] = a
            dk[k0:k1, g] = bk
            dv[k0:k1, g] = bv
    return dq, dk, dv


def bias_grad(dout, q, k, v, cu_q, cu_k, scale, causal, bias, bias_strides, size: int,
              grad_strides=None):
    """Gradient of sum(dout * out) w.r.t. a bias buffer of `size` elements read through the
    strided view (b, h, r, c) -> b*t0 + h*t1 + r*t2 + c*t3 (t = grad_strides, default the
    bias strides).  The bias enters the logits additively, so its gradient is dS, summed
    into every buffer element that several (b, h, r, c) read (a stride-0 axis, e.g. the
    rows of a per-key bias).  Elements no valid (b, h, r < Lq, c < Lk) reads stay 0."""
    q, k, v, cu_q, cu_k, n_rep = _check(q, k, v, cu_q, cu_k)
    dout = np.asarray(dout)
    t0, t1, t2, t3 = (int(x) for x in (grad_strides if grad_strides is not None else bias_strides))
    grad = np.zeros(size)
    for b in range(len(cu_q) - 1):
        q0, q1, k0, k1 = cu_q[b], cu_q[b + 1], cu_k[b], cu_k[b + 1]
        lq, lk = q1 - q0, k1 - k0
        if lq == 0 or lk == 0:
            continue
        r = np.arange(lq, dtype=np.int64)[:, None]
        c = np.arange(lk, dtype=np.int64)[None, :]
        for h in range(q.shape[1]):
            g = h // n_rep
            bb = bias_tile(bias, bias_strides, b, h, lq, lk)
            _, ds = head_logit_grad(q[q0:q1, h], k[k0:k1, g], v[k0:k1, g], dout[q0:q1, h],
                                    scale, causal, bb)
            idx = b * t0 + h * t1 + r * t2 + c * t3
            np.add.at(grad, idx.ravel(), ds.ravel())
    return grad
