"""Scalar brute-force attention for tiny inputs (pure Python, ``math.fsum``).

TEST INFRASTRUCTURE, like ``oracle.attention``: used only by tests to pin the
vectorised oracle.  It restates the same definition element by element with
no matrix routine at all: for every sequence, query head and query row it
lists the visible keys (bottom-right causal), forms each score as an exactly
rounded sum of products plus the bias element at its strided offset, and
normalises with the row maximum subtracted.  Rows with no visible key give a
zero output and a log-sum-exp of minus infinity.
"""

from __future__ import annotations

import math


def _val(a, *idx):
    return float(a[idx])


def brute_forward(q, k, v, cu_q, cu_k, scale, causal, bias=None, bias_strides=None):
    """Returns (out, lse) as nested Python lists: out[t][h][c], lse[h][t]."""
    tq, hq, d = q.shape
    tk, hkv, dv = v.shape
    n_rep = hq // hkv
    out = [[[0.0] * dv for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * tq for _ in range(hq)]
    nb = len(cu_q) - 1
    for b in range(nb):
        q0, q1 = int(cu_q[b]), int(cu_q[b + 1])
        k0, k1 = int(cu_k[b]), int(cu_k[b + 1])
        lq, lk = q1 - q0, k1 - k0
        for h in range(hq):
            g = h // n_rep
            for i in range(lq):
                scores = []
                for j in range(lk):
                    if causal and j > i + (lk - lq):
                        continue
                    s = scale * math.fsum(_val(q, q0 + i, h, t) * _val(k, k0 + j, g, t)
                                          for t in range(d))
                    if bias is not None:
                        s0, s1, s2, s3 = bias_strides
                        s += float(bias[b * s0 + h * s1 + i * s2 + j * s3])
                    scores.append((j, s))
                if not scores:
                    continue
                m = max(s for _, s in scores)
                e = [(j, math.exp(s - m)) for j, s in scores]
                l = math.fsum(w for _, w in e)
                for c in range(dv):
                    out[q0 + i][h][c] = math.fsum(w * _val(v, k0 + j, g, c) for j, w in e) / l
                lse[h][q0 + i] = m + math.log(l)
    return out, lse
