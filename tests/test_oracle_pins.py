"""Pins for the CPU fp64 oracle: every check compares it with something other than itself.

* brute force: scalar loops with exactly rounded sums (``oracle.brute``);
* a library routine: PyTorch's CPU scaled_dot_product_attention in float64,
  per sequence and as one dense block-diagonal mask over the whole packed
  stream (the dense (1, 1, T, T) formulation the TorchEasyRec pull request
  663 page describes in section "Choosing the kernel");
* closed forms worked by hand (``tests/golden/hand_examples.json``);
* invariants: rows sum to one, constant V, shift invariance, GQA equal to
  MHA on repeated KV heads, causal special cases, packed equal to solo,
  bit-identical isolation of a rewritten sequence (the row-isolation test of
  the TorchEasyRec page, section "Test plan");
* gradients against central finite differences and against float64 autograd.

``test_planted_mistakes_are_caught`` edits the oracle's source on the CPU
(dropped scale, wrong causal offset, wrong GQA mapping, transposed dV, ...)
and shows the pins above fail for each edit.
"""

import json
import math
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from workloads import make_case

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")

# ---------------------------------------------------------------- tiny cases
# B <= 3, L <= 6, d <= 4, Hq <= 4, Hkv <= 2, every mask and bias mode, Lq != Lk both ways.
TINY = [
    dict(seed=1, lens_q=[3, 5, 2], hq=2, hkv=2, d=4, causal=False),
    dict(seed=2, lens_q=[3, 5, 2], hq=2, hkv=2, d=4, causal=True),
    dict(seed=3, lens_q=[4, 6], hq=4, hkv=2, d=3, causal=True),
    dict(seed=4, lens_q=[4, 6], hq=4, hkv=1, d=4, causal=False),
    dict(seed=5, lens_q=[2, 3], lens_k=[5, 6], hq=2, hkv=1, d=4, causal=True),
    dict(seed=6, lens_q=[6, 4], lens_k=[2, 3], hq=2, hkv=2, d=2, causal=True),
    dict(seed=7, lens_q=[1, 6, 3], lens_k=[6, 1, 3], hq=4, hkv=2, d=4, causal=True),
    dict(seed=8, lens_q=[3, 5], hq=2, hkv=2, d=4, causal=False, bias="per_key"),
    dict(seed=9, lens_q=[3, 5], hq=2, hkv=2, d=4, causal=True, bias="per_pair"),
    dict(seed=10, lens_q=[4, 2], lens_k=[6, 3], hq=4, hkv=2, d=4, causal=True, bias="per_pair",
         bias_layout="permuted"),
    dict(seed=11, lens_q=[5, 3], lens_k=[2, 6], hq=2, hkv=1, d=4, causal=True, bias="per_key",
         bias_layout="head_shared"),
    dict(seed=12, lens_q=[3, 0, 4], lens_k=[3, 2, 0], hq=2, hkv=2, d=4, causal=False),
    dict(seed=13, lens_q=[5, 4], hq=2, hkv=2, d=4, causal=False, bias="per_pair", bias_std=3.0),
]


def _case(c, **kw):
    c = dict(c)
    c.update(kw)
    return make_case(**c)


def _fwd(w, mod=oracle):
    return mod.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)


def _bwd(w, mod=oracle):
    return mod.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                        w.bias_strides)


def _sdpa_sequence(w, b, h, bias_tile=None):
    """PyTorch float64 SDPA for one sequence and head, with an explicit additive mask."""
    n_rep = w.hq // w.hkv
    cq, ck = w.cu_q, w.cu_k
    q0, q1, k0, k1 = cq[b], cq[b + 1], ck[b], ck[b + 1]
    lq, lk = q1 - q0, k1 - k0
    q = torch.from_numpy(np.asarray(w.q[q0:q1, h], dtype=np.float64))[None, None]
    k = torch.from_numpy(np.asarray(w.k[k0:k1, h // n_rep], dtype=np.float64))[None, None]
    v = torch.from_numpy(np.asarray(w.v[k0:k1, h // n_rep], dtype=np.float64))[None, None]
    mask = torch.zeros(lq, lk, dtype=torch.float64)
    if w.causal:
        i = torch.arange(lq)[:, None]
        j = torch.arange(lk)[None, :]
        mask = mask.masked_fill(j > i + (lk - lq), -math.inf)
    if w.bias is not None:
        s0, s1, s2, s3 = w.bias_strides
        r = np.arange(lq)[:, None]
        c = np.arange(lk)[None, :]
        mask = mask + torch.from_numpy(w.bias[b * s0 + h * s1 + r * s2 + c * s3].astype(np.float64))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask[None, None],
                                                         scale=w.scale)
    sc = w.scale * (q[0, 0] @ k[0, 0].T) + mask
    lse = torch.logsumexp(sc, dim=-1)
    return o[0, 0].numpy(), lse.numpy()


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("c", TINY, ids=lambda c: f"s{c['seed']}")
def test_brute_force(c):
    w = _case(c)
    out, lse = _fwd(w)
    bo, bl = oracle.brute_forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                                  w.bias_strides)
    bo, bl = np.array(bo), np.array(bl)
    assert np.max(np.abs(out - bo)) <= 1e-12
    fin = np.isfinite(bl)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - bl[fin]), initial=0.0) <= 1e-12


# ---------------------------------------------------------------- library SDPA
@pytest.mark.parametrize("c", TINY, ids=lambda c: f"s{c['seed']}")
def test_library_sdpa_per_sequence(c):
    w = _case(c)
    out, lse = _fwd(w)
    cq = w.cu_q
    for b in range(w.batch):
        for h in range(w.hq):
            lq, lk = w.lens_q[b], w.lens_k[b]
            if lq == 0:
                continue
            rows = oracle.visible(lq, lk, w.causal).any(axis=1)
            if not rows.any():
                continue
            o, l = _sdpa_sequence(w, b, h)
            sl = slice(cq[b], cq[b + 1])
            assert np.max(np.abs(out[sl, h][rows] - o[rows])) <= 1e-12
            assert np.max(np.abs(lse[h, sl][rows] - l[rows])) <= 1e-12


@pytest.mark.parametrize("c", [t for t in TINY if "lens_k" not in t], ids=lambda c: f"s{c['seed']}")
def test_dense_block_diagonal_mask(c):
    """Whole packed stream through one (T, T) mask: block diagonal plus causal inside blocks."""
    w = _case(c)
    out, lse = _fwd(w)
    T = w.total_q
    seg = np.repeat(np.arange(w.batch), w.lens_q)
    pos = np.concatenate([np.arange(n) for n in w.lens_q]) if T else np.zeros(0, int)
    allowed = seg[:, None] == seg[None, :]
    if w.causal:
        allowed &= pos[None, :] <= pos[:, None]
    n_rep = w.hq // w.hkv
    for h in range(w.hq):
        add = np.where(allowed, 0.0, -np.inf)
        if w.bias is not None:
            s0, s1, s2, s3 = w.bias_strides
            bidx = seg[:, None] * s0 + h * s1 + pos[:, None] * s2 + pos[None, :] * s3
            bidx = np.where(allowed, bidx, 0)
            add = add + np.where(allowed, w.bias[bidx].astype(np.float64), 0.0)
        q = torch.from_numpy(w.q[:, h].astype(np.float64))[None, None]
        k = torch.from_numpy(w.k[:, h // n_rep].astype(np.float64))[None, None]
        v = torch.from_numpy(w.v[:, h // n_rep].astype(np.float64))[None, None]
        o = torch.nn.functional.scaled_dot_product_attention(
            q, k, v, attn_mask=torch.from_numpy(add)[None, None], scale=w.scale)[0, 0].numpy()
        assert np.max(np.abs(out[:, h] - o)) <= 1e-12


# ---------------------------------------------------------------- golden closed forms
def _golden_cases():
    with open(os.path.join(GOLDEN, "hand_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("g", _golden_cases(), ids=lambda g: g["name"])
def test_hand_examples(g):
    q = np.array(g["q"], dtype=np.float64)
    k = np.array(g["k"], dtype=np.float64)
    v = np.array(g["v"], dtype=np.float64)
    cu_q = np.concatenate([[0], np.cumsum(g["lens_q"])])
    cu_k = np.concatenate([[0], np.cumsum(g["lens_k"])])
    bias = np.array(g["bias"]) if "bias" in g else None
    out, lse = oracle.forward(q, k, v, cu_q, cu_k, g["scale"], g["causal"], bias,
                              g.get("bias_strides"))
    exp_lse = np.array([[(-math.inf if x == "-inf" else x) for x in row] for row in g["lse"]])
    assert np.max(np.abs(out - np.array(g["out"]))) <= 1e-14
    fin = np.isfinite(exp_lse)
    assert np.array_equal(fin, np.isfinite(lse))
    assert np.max(np.abs(lse[fin] - exp_lse[fin])) <= 1e-14


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("c", TINY, ids=lambda c: f"s{c['seed']}")
def test_softmax_rows(c):
    w = _case(c)
    n_rep = w.hq // w.hkv
    for b in range(w.batch):
        q0, q1, k0, k1 = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
        lq, lk = q1 - q0, k1 - k0
        vis = oracle.visible(lq, lk, w.causal)
        for h in range(w.hq):
            bb = oracle.bias_tile(w.bias, w.bias_strides, b, h, lq, lk)
            p = oracle.head_probs(w.q[q0:q1, h], w.k[k0:k1, h // n_rep], w.scale, w.causal, bb)
            assert np.all(p >= 0)
            assert np.all(p[~vis] == 0.0)
            rows = vis.any(axis=1)
            assert np.max(np.abs(p[rows].sum(axis=1) - 1.0), initial=0.0) <= 1e-13
            assert np.all(p[~rows] == 0.0)


@pytest.mark.parametrize("c", TINY[:7], ids=lambda c: f"s{c['seed']}")
def test_constant_v(c):
    w = _case(c)
    w.v[:] = 0.375
    out, lse = _fwd(w)
    nonempty = np.isfinite(lse.T)  # [Tq, Hq]
    assert np.max(np.abs(out[nonempty] - 0.375)) <= 1e-13
    assert np.all(out[~nonempty] == 0.0)


def test_single_key():
    w = make_case(21, [4, 1, 3], lens_k=[1, 1, 1], hq=2, hkv=1, d=4, causal=False)
    out, lse = _fwd(w)
    for b in range(w.batch):
        for h in range(w.hq):
            for i in range(w.cu_q[b], w.cu_q[b + 1]):
                assert np.allclose(out[i, h], w.v[b, 0], atol=0, rtol=0) or \
                    np.max(np.abs(out[i, h] - w.v[b, 0])) <= 1e-15
                s = w.scale * float(np.dot(w.q[i, h].astype(np.float64), w.k[b, 0].astype(np.float64)))
                assert abs(lse[h, i] - s) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_zero_query_closed_form(causal):
    """Q = 0, no bias: O_i is the mean of the visible V rows and LSE_i = ln n_vis(i)."""
    w = make_case(22, [5, 3], lens_k=[7, 3], hq=2, hkv=2, d=4, causal=causal)
    w.q[:] = 0
    out, lse = _fwd(w)
    for b in range(w.batch):
        lq, lk = w.lens_q[b], w.lens_k[b]
        vis = oracle.visible(lq, lk, causal)
        for h in range(w.hq):
            for i in range(lq):
                n = int(vis[i].sum())
                t = w.cu_q[b] + i
                if n == 0:
                    assert np.all(out[t, h] == 0) and lse[h, t] == -np.inf
                    continue
                keys = w.cu_k[b] + np.nonzero(vis[i])[0]
                mean = w.v[keys, h].astype(np.float64).mean(axis=0)
                assert np.max(np.abs(out[t, h] - mean)) <= 1e-14
                assert abs(lse[h, t] - math.log(n)) <= 1e-14


def test_shift_invariance():
    w = make_case(23, [4, 6], hq=2, hkv=2, d=4, causal=True, bias="per_pair")
    out0, lse0 = _fwd(w)
    # a per-row constant added to every bias element of that row
    s0, s1, s2, s3 = w.bias_strides
    shift = np.zeros_like(w.bias, dtype=np.float64)
    bias2 = w.bias.astype(np.float64).copy()
    rowshift = {}
    for b in range(w.batch):
        for h in range(w.hq):
            for r in range(w.lens_q[b]):
                c = 0.25 * (1 + b + 2 * h + 3 * r)
                rowshift[(b, h, r)] = c
                for col in range(w.lens_k[b]):
                    bias2[b * s0 + h * s1 + r * s2 + col * s3] += c
    out1, lse1 = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True, bias2, w.bias_strides)
    assert np.max(np.abs(out1 - out0)) <= 1e-13
    for (b, h, r), c in rowshift.items():
        t = w.cu_q[b] + r
        assert abs(lse1[h, t] - lse0[h, t] - c) <= 1e-13
    del shift
    # a per-key bias that is the same for every key equals no bias, up to LSE + constant
    wk = make_case(24, [4, 6], hq=2, hkv=2, d=4, causal=False, bias="per_key")
    wk.bias[:] = 1.5
    o1, l1 = _fwd(wk)
    o2, l2 = oracle.forward(wk.q, wk.k, wk.v, wk.cu_q, wk.cu_k, wk.scale, False)
    assert np.max(np.abs(o1 - o2)) <= 1e-13
    assert np.max(np.abs(l1 - l2 - 1.5)) <= 1e-13


@pytest.mark.parametrize("causal", [False, True])
def test_gqa_equals_mha_on_repeated_heads(causal):
    w = make_case(25, [5, 3], lens_k=[6, 3], hq=4, hkv=2, d=4, causal=causal, with_dout=True)
    out, lse = _fwd(w)
    kr = np.repeat(w.k, 2, axis=1)
    vr = np.repeat(w.v, 2, axis=1)
    out2, lse2 = oracle.forward(w.q, kr, vr, w.cu_q, w.cu_k, w.scale, causal)
    assert np.array_equal(out, out2)
    assert np.array_equal(lse, lse2)
    dq, dk, dv = _bwd(w)
    dq2, dk2, dv2 = oracle.backward(w.dout, w.q, kr, vr, w.cu_q, w.cu_k, w.scale, causal)
    assert np.max(np.abs(dq - dq2)) <= 1e-13
    assert np.max(np.abs(dk - (dk2[:, 0::2] + dk2[:, 1::2]))) <= 1e-13
    assert np.max(np.abs(dv - (dv2[:, 0::2] + dv2[:, 1::2]))) <= 1e-13


def test_causal_square_is_lower_triangular():
    w = make_case(26, [6], hq=1, hkv=1, d=4, causal=True)
    out, _ = _fwd(w)
    q = torch.from_numpy(w.q[:, 0].astype(np.float64))[None, None]
    k = torch.from_numpy(w.k[:, 0].astype(np.float64))[None, None]
    v = torch.from_numpy(w.v[:, 0].astype(np.float64))[None, None]
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale)
    assert np.max(np.abs(out[:, 0] - o[0, 0].numpy())) <= 1e-13


def test_causal_single_query_equals_noncausal():
    w = make_case(27, [1, 1], lens_k=[9, 4], hq=2, hkv=1, d=4, causal=True)
    a = _fwd(w)
    b = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, False)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_more_queries_than_keys_gives_empty_leading_rows():
    w = make_case(28, [6], lens_k=[2], hq=1, hkv=1, d=4, causal=True)
    out, lse = _fwd(w)
    assert np.all(out[:4] == 0) and np.all(np.isneginf(lse[0, :4]))
    assert np.all(np.isfinite(lse[0, 4:]))


def test_packed_equals_solo_bitwise():
    w = make_case(29, [5, 1, 6, 3], lens_k=[5, 4, 6, 2], hq=4, hkv=2, d=4, causal=True,
                  bias="per_pair", with_dout=True)
    out, lse = _fwd(w)
    dq, dk, dv = _bwd(w)
    s0, s1, s2, s3 = w.bias_strides
    for b in range(w.batch):
        q0, q1, k0, k1 = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
        cu_q1 = np.array([0, q1 - q0])
        cu_k1 = np.array([0, k1 - k0])
        bias1 = w.bias[b * s0:(b + 1) * s0]
        o1, l1 = oracle.forward(w.q[q0:q1], w.k[k0:k1], w.v[k0:k1], cu_q1, cu_k1, w.scale, True,
                                bias1, w.bias_strides)
        assert np.array_equal(o1, out[q0:q1]) and np.array_equal(l1, lse[:, q0:q1])
        g1 = oracle.backward(w.dout[q0:q1], w.q[q0:q1], w.k[k0:k1], w.v[k0:k1], cu_q1, cu_k1,
                             w.scale, True, bias1, w.bias_strides)
        assert np.array_equal(g1[0], dq[q0:q1])
        assert np.array_equal(g1[1], dk[k0:k1]) and np.array_equal(g1[2], dv[k0:k1])


def test_packed_equals_padded_with_key_padding_mask():
    """A padded batch with a key-padding mask (the layout the varlen path replaces) agrees."""
    w = make_case(30, [5, 2, 6], hq=2, hkv=2, d=4, causal=False)
    out, _ = _fwd(w)
    L = w.max_q
    for h in range(w.hq):
        qp = np.zeros((w.batch, L, w.d))
        kp = np.zeros((w.batch, L, w.d))
        vp = np.zeros((w.batch, L, w.d))
        mask = np.full((w.batch, L, L), -np.inf)
        for b in range(w.batch):
            n = w.lens_q[b]
            sl = slice(w.cu_q[b], w.cu_q[b + 1])
            qp[b, :n], kp[b, :n], vp[b, :n] = w.q[sl, h], w.k[sl, h], w.v[sl, h]
            mask[b, :, :n] = 0.0
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(qp)[:, None], torch.from_numpy(kp)[:, None],
            torch.from_numpy(vp)[:, None], attn_mask=torch.from_numpy(mask)[:, None],
            scale=w.scale)[:, 0].numpy()
        for b in range(w.batch):
            n = w.lens_q[b]
            assert np.max(np.abs(o[b, :n] - out[w.cu_q[b]:w.cu_q[b + 1], h])) <= 1e-12


def test_isolation_bitwise():
    """Rewrite sequence 0 (values, then its length); every other sequence is bit-identical."""
    w = make_case(31, [5, 4, 6], lens_k=[6, 4, 6], hq=4, hkv=2, d=4, causal=True,
                  bias="per_pair", with_dout=True, grid=(8, 8))
    out, lse = _fwd(w)
    g = _bwd(w)
    w2 = make_case(32, [5, 4, 6], lens_k=[6, 4, 6], hq=4, hkv=2, d=4, causal=True,
                   bias="per_pair", with_dout=True, grid=(8, 8))
    for a, b_ in ((w2.q, w.q), (w2.dout, w.dout)):
        a[5:] = b_[5:]
    for a, b_ in ((w2.k, w.k), (w2.v, w.v)):
        a[6:] = b_[6:]
    s0 = w.bias_strides[0]
    w2.bias[s0:] = w.bias[s0:]
    out2, lse2 = _fwd(w2)
    g2 = _bwd(w2)
    assert np.array_equal(out2[5:], out[5:]) and np.array_equal(lse2[:, 5:], lse[:, 5:])
    assert not np.array_equal(out2[:5], out[:5])
    assert np.array_equal(g2[0][5:], g[0][5:])
    assert np.array_equal(g2[1][6:], g[1][6:]) and np.array_equal(g2[2][6:], g[2][6:])
    # change sequence 0's length: every later offset moves
    w3 = make_case(33, [2], lens_k=[3], hq=4, hkv=2, d=4, with_dout=True)
    q3 = np.concatenate([w3.q, w.q[5:]])
    k3 = np.concatenate([w3.k, w.k[6:]])
    v3 = np.concatenate([w3.v, w.v[6:]])
    do3 = np.concatenate([w3.dout, w.dout[5:]])
    cq = np.array([0, 2, 6, 12])
    ck = np.array([0, 3, 7, 13])
    o3, l3 = oracle.forward(q3, k3, v3, cq, ck, w.scale, True, w.bias, w.bias_strides)
    assert np.array_equal(o3[2:], out[5:]) and np.array_equal(l3[:, 2:], lse[:, 5:])
    g3 = oracle.backward(do3, q3, k3, v3, cq, ck, w.scale, True, w.bias, w.bias_strides)
    assert np.array_equal(g3[0][2:], g[0][5:])
    assert np.array_equal(g3[1][3:], g[1][6:]) and np.array_equal(g3[2][3:], g[2][6:])


# ---------------------------------------------------------------- gradients
GRAD_CASES = [
    dict(seed=41, lens_q=[3, 4], hq=2, hkv=2, d=3, causal=False),
    dict(seed=42, lens_q=[3, 4], hq=4, hkv=2, d=3, causal=True),
    dict(seed=43, lens_q=[2, 4], lens_k=[4, 2], hq=2, hkv=1, d=3, causal=True, bias="per_pair"),
    dict(seed=44, lens_q=[3, 2], hq=2, hkv=2, d=2, causal=False, bias="per_key",
         bias_layout="permuted"),
]


@pytest.mark.parametrize("c", GRAD_CASES, ids=lambda c: f"s{c['seed']}")
def test_gradients_finite_differences(c):
    w = _case(c, with_dout=True)
    dq, dk, dv = _bwd(w)
    q, k, v = (x.astype(np.float64) for x in (w.q, w.k, w.v))
    do = w.dout.astype(np.float64)

    def loss(q_, k_, v_):
        o, _ = oracle.forward(q_, k_, v_, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)
        return float(np.sum(o * do))

    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        it = np.nditer(x, flags=["multi_index"])
        for _ in it:
            i = it.multi_index
            xp = x.copy()
            xp[i] += eps
            xm = x.copy()
            xm[i] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[i] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        err = np.max(np.abs(num - g)) / max(1e-3, np.max(np.abs(g)))
        assert err <= 1e-6, (name, err)


@pytest.mark.parametrize("c", TINY, ids=lambda c: f"s{c['seed']}")
def test_gradients_autograd_float64(c):
    w = _case(c, with_dout=True)
    dq, dk, dv = _bwd(w)
    n_rep = w.hq // w.hkv
    for b in range(w.batch):
        q0, q1, k0, k1 = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
        lq, lk = q1 - q0, k1 - k0
        if lq == 0 or lk == 0:
            assert np.all(dq[q0:q1] == 0)
            assert np.all(dk[k0:k1] == 0) and np.all(dv[k0:k1] == 0)
            continue
        vis = torch.from_numpy(oracle.visible(lq, lk, w.causal))
        q = torch.tensor(w.q[q0:q1].astype(np.float64), requires_grad=True)
        k = torch.tensor(w.k[k0:k1].astype(np.float64), requires_grad=True)
        v = torch.tensor(w.v[k0:k1].astype(np.float64), requires_grad=True)
        total = 0
        for h in range(w.hq):
            g = h // n_rep
            s = w.scale * (q[:, h] @ k[:, g].T)
            if w.bias is not None:
                s = s + torch.from_numpy(oracle.bias_tile(w.bias, w.bias_strides, b, h, lq, lk))
            s = s.masked_fill(~vis, -math.inf)
            rows = vis.any(dim=1)
            p = torch.softmax(s[rows], dim=-1)
            o = p @ v[:, g]
            total = total + (o * torch.from_numpy(w.dout[q0:q1, h].astype(np.float64))[rows]).sum()
        total.backward()
        assert np.max(np.abs(q.grad.numpy() - dq[q0:q1])) <= 1e-12
        assert np.max(np.abs(k.grad.numpy() - dk[k0:k1])) <= 1e-12
        assert np.max(np.abs(v.grad.numpy() - dv[k0:k1])) <= 1e-12


def test_constant_v_gives_zero_dq_dk():
    w = make_case(45, [4, 5], hq=4, hkv=2, d=4, causal=True, with_dout=True, bias="per_pair")
    w.v[:] = -1.25
    dq, dk, _ = _bwd(w)
    assert np.max(np.abs(dq)) <= 1e-12 and np.max(np.abs(dk)) <= 1e-12


# ---------------------------------------------------------------- planted mistakes
MUTATIONS = [
    ("dropped scale", "s = float(scale) * (qb @ kb.T)", "s = (qb @ kb.T)"),
    ("bias subtracted", "s = s + bias_bh", "s = s - bias_bh"),
    ("top-left causal", "return j <= i + (lk - lq)", "return j <= i"),
    ("strict causal", "return j <= i + (lk - lq)", "return j < i + (lk - lq)"),
    ("wrong GQA map", "g = h // n_rep\n            bb", "g = h % k.shape[1]\n            bb"),
    ("bias row/col swapped", "idx = b * s0 + h * s1 + r * s2 + c * s3",
     "idx = b * s0 + h * s1 + r * s3 + c * s2"),
    ("no max shift in lse", "lse[rows] = m[:, 0] + np.log(l[:, 0])", "lse[rows] = np.log(l[:, 0])"),
    ("dV with rows reversed", "dv = p.T @ dob", "dv = p.T @ dob[::-1]"),
    ("D term dropped", "ds = p * (dp - dsum)", "ds = p * dp"),
    ("dK missing scale", "dk = float(scale) * (ds.T @ qb)", "dk = (ds.T @ qb)"),
    ("dQ sign", "dq = float(scale) * (ds @ kb)", "dq = -float(scale) * (ds @ kb)"),
]


def _mutant(src_old, src_new):
    path = oatt.__file__
    with open(path) as f:
        src = f.read()
    assert src.count(src_old) >= 1, src_old
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(src_old, src_new), path, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    try:
        for c in TINY:
            w = _case(c, with_dout=True)
            out, lse = _fwd(w, mod)
            bo, bl = oracle.brute_forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal,
                                          w.bias, w.bias_strides)
            if np.max(np.abs(out - np.array(bo))) > 1e-12:
                return False
            bl = np.array(bl)
            fin = np.isfinite(bl)
            if not np.array_equal(fin, np.isfinite(lse)) or \
                    np.max(np.abs(lse[fin] - bl[fin]), initial=0) > 1e-12:
                return False
        for c in GRAD_CASES[:3]:
            w = _case(c, with_dout=True)
            g = _bwd(w, mod)
            g0 = _bwd(w)
            # the reference gradient is pinned by finite differences and autograd above;
            # here the mutant must reproduce it
            for a, b in zip(g, g0):
                if np.max(np.abs(a - b)) > 1e-12:
                    return False
    except Exception:
        return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _pins_pass(oatt)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    assert not _pins_pass(_mutant(old, new)), name


# ---------------------------------------------------------------- per-sequence checkers
# ``sequence_head_forward`` computes one (sequence, query head) on its own, apart from
# ``forward()``: it finds the sequence's rows, the KV head of the query head and the
# bias block itself.  It is pinned to the brute force (scalar loops, exactly rounded
# sums) for every (b, h) of every tiny case, and must equal forward()'s slice bitwise.
# ``sequence_group_backward`` is the per-(sequence, KV head) body of ``backward()``,
# whose results the finite-difference and autograd pins above fix.


def _seq_head_pins_pass(mod) -> bool:
    try:
        for c in TINY:
            w = _case(c)
            bo, bl = oracle.brute_forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal,
                                          w.bias, w.bias_strides)
            bo, bl = np.array(bo), np.array(bl)
            for b in range(w.batch):
                q0, q1 = w.cu_q[b], w.cu_q[b + 1]
                for h in range(w.hq):
                    o, l = mod.sequence_head_forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal,
                                                     w.bias, w.bias_strides, b, h)
                    if o.shape != (q1 - q0, w.d) or l.shape != (q1 - q0,):
                        return False
                    if np.max(np.abs(o - bo[q0:q1, h]), initial=0) > 1e-12:
                        return False
                    ref = bl[h, q0:q1]
                    fin = np.isfinite(ref)
                    if not np.array_equal(fin, np.isfinite(l)) or \
                            np.max(np.abs(l[fin] - ref[fin]), initial=0) > 1e-12:
                        return False
    except Exception:
        return False
    return True


def test_sequence_head_forward_matches_brute_force_everywhere():
    assert _seq_head_pins_pass(oatt)


def test_sequence_head_forward_equals_forward_slices_bitwise():
    for c in TINY:
        w = _case(c)
        out, lse = _fwd(w)
        for b in range(w.batch):
            q0, q1 = w.cu_q[b], w.cu_q[b + 1]
            for h in range(w.hq):
                o, l = oracle.sequence_head_forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal,
                                                    w.bias, w.bias_strides, b, h)
                assert np.array_equal(o, out[q0:q1, h])
                assert np.array_equal(l, lse[h, q0:q1])


def test_sequence_group_backward_equals_backward_slices():
    for c in GRAD_CASES + [dict(seed=46, lens_q=[3, 0, 5], lens_k=[2, 4, 5], hq=4, hkv=2, d=3, causal=True,
                                bias="per_pair")]:
        w = _case(c, with_dout=True)
        dq, dk, dv = _bwd(w)
        n_rep = w.hq // w.hkv
        for b in range(w.batch):
            q0, q1, k0, k1 = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
            for g in range(w.hkv):
                a, bk, bv = oracle.sequence_group_backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale,
                                                           w.causal, w.bias, w.bias_strides, b, g)
                assert np.array_equal(a, dq[q0:q1, g * n_rep:(g + 1) * n_rep])
                assert np.array_equal(bk, dk[k0:k1, g]) and np.array_equal(bv, dv[k0:k1, g])


SEQ_HEAD_MUTATIONS = [
    ("wrong GQA map", "g = h // n_rep\n    bb", "g = h % k.shape[1]\n    bb"),
    ("KV head from the group size", "g = h // n_rep\n    bb", "g = min(h, k.shape[1] - 1)\n    bb"),
    ("key rows from the query bounds", "k[k0:k1, g], v[k0:k1, g], scale, causal, bb)\n\n\ndef forward",
     "k[q0:q1, g], v[q0:q1, g], scale, causal, bb)\n\n\ndef forward"),
    ("bias of the KV head", "bb = bias_tile(bias, bias_strides, b, h, q1 - q0, k1 - k0)\n    return",
     "bb = bias_tile(bias, bias_strides, b, g, q1 - q0, k1 - k0)\n    return"),
    ("next sequence's bias", "bb = bias_tile(bias, bias_strides, b, h, q1 - q0, k1 - k0)\n    return",
     "bb = bias_tile(bias, bias_strides, min(b + 1, len(cu_q) - 2), h, q1 - q0, k1 - k0)\n    return"),
]


@pytest.mark.parametrize("name,old,new", SEQ_HEAD_MUTATIONS, ids=[m[0] for m in SEQ_HEAD_MUTATIONS])
def test_sequence_head_forward_mistakes_are_caught(name, old, new):
    assert not _seq_head_pins_pass(_mutant(old, new)), name
