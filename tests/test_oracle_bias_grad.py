"""Pins for the oracle's bias gradient (``oracle.bias_grad``), each against
something other than itself:

* central finite differences of sum(dO * O) in float64, element by element
  of the bias buffer (per-pair, per-key, permuted and head-shared layouts,
  causal and cross-length);
* PyTorch float64 autograd through ``torch.as_strided`` views of the bias
  storage (a library routine summing the gradient of overlapping reads);
* a closed form: every softmax row's logit gradient sums to zero, so each
  (sequence, head, row) of a per-pair gradient and each (sequence, head) of a
  per-key gradient sums to zero.

Planted mistakes in the oracle's source (assignment instead of accumulation
into broadcast elements, P in place of dS, a flipped sign) must fail them.
"""

import math
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import attention as oatt
from workloads import make_case

CASES = [
    dict(seed=61, lens_q=[3, 5], hq=2, hkv=2, d=4, causal=False, bias="per_pair"),
    dict(seed=62, lens_q=[4, 2], lens_k=[6, 3], hq=4, hkv=2, d=4, causal=True, bias="per_pair",
         bias_layout="permuted"),
    dict(seed=63, lens_q=[3, 5], hq=2, hkv=1, d=4, causal=True, bias="per_key"),
    dict(seed=64, lens_q=[5, 3], lens_k=[2, 6], hq=2, hkv=1, d=4, causal=True, bias="per_key",
         bias_layout="head_shared"),
    dict(seed=65, lens_q=[4, 0, 3], lens_k=[4, 2, 0], hq=2, hkv=2, d=3, causal=False, bias="per_pair"),
]


def _case(c):
    return make_case(with_dout=True, **c)


def _loss(w, bias, mod=oatt):
    out, _ = mod.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, bias, w.bias_strides)
    return float(np.sum(out * np.asarray(w.dout, dtype=np.float64)))


def _grad(w, mod=oatt):
    return mod.bias_grad(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                         w.bias_strides, len(w.bias))


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_finite_differences(ci, mod=oatt):
    w = _case(CASES[ci])
    g = _grad(w, mod)
    base = np.asarray(w.bias, dtype=np.float64)
    rng = np.random.default_rng(ci)
    picks = rng.choice(len(base), size=min(12, len(base)), replace=False)
    h = 1e-5
    for e in picks:
        up, dn = base.copy(), base.copy()
        up[e] += h
        dn[e] -= h
        fd = (_loss(w, up) - _loss(w, dn)) / (2 * h)
        assert abs(fd - g[e]) <= 1e-7 * max(1.0, abs(fd)), (e, fd, g[e])


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_torch_autograd(ci):
    w = _case(CASES[ci])
    g = _grad(w)
    store = torch.tensor(np.asarray(w.bias, dtype=np.float64), requires_grad=True)
    s0, s1, s2, s3 = w.bias_strides
    n_rep = w.hq // w.hkv
    total = 0
    for b in range(w.batch):
        q0, q1, k0, k1 = w.cu_q[b], w.cu_q[b + 1], w.cu_k[b], w.cu_k[b + 1]
        lq, lk = int(q1 - q0), int(k1 - k0)
        if lq == 0 or lk == 0:
            continue
        vis = torch.from_numpy(oracle.visible(lq, lk, w.causal))
        rows = vis.any(dim=1)
        for h in range(w.hq):
            gk = h // n_rep
            q = torch.from_numpy(np.asarray(w.q[q0:q1, h], dtype=np.float64))
            k = torch.from_numpy(np.asarray(w.k[k0:k1, gk], dtype=np.float64))
            v = torch.from_numpy(np.asarray(w.v[k0:k1, gk], dtype=np.float64))
            bias = torch.as_strided(store, (lq, lk), (s2, s3), b * s0 + h * s1)
            s = w.scale * (q @ k.T) + bias
            s = s.masked_fill(~vis, -math.inf)
            p = torch.softmax(s[rows], dim=-1)
            o = p @ v
            total = total + (o * torch.from_numpy(np.asarray(w.dout[q0:q1, h], dtype=np.float64))[rows]).sum()
    total.backward()
    assert np.max(np.abs(store.grad.numpy() - g)) <= 1e-12


@pytest.mark.parametrize("ci", [0, 1, 2, 3])
def test_rows_of_the_logit_gradient_sum_to_zero(ci):
    w = _case(CASES[ci])
    g = _grad(w)
    s0, s1, s2, s3 = w.bias_strides
    heads = 1 if s1 == 0 else w.hq
    for b in range(w.batch):
        lq = int(w.cu_q[b + 1] - w.cu_q[b])
        lk = int(w.cu_k[b + 1] - w.cu_k[b])
        for h in range(heads):
            for r in range(lq if s2 != 0 else 1):
                idx = b * s0 + h * s1 + r * s2 + np.arange(lk) * s3
                assert abs(g[idx].sum()) <= 1e-12


MUTATIONS = [
    ("assign instead of accumulate", "np.add.at(grad, idx.ravel(), ds.ravel())",
     "grad[idx.ravel()] = ds.ravel()"),
    ("P in place of dS", "np.add.at(grad, idx.ravel(), ds.ravel())", "np.add.at(grad, idx.ravel(), _.ravel())"),
    ("sign", "np.add.at(grad, idx.ravel(), ds.ravel())", "np.add.at(grad, idx.ravel(), -ds.ravel())"),
]


def _mutant(old, new):
    with open(oatt.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("bias_grad_mutant")
    exec(compile(src.replace(old, new), oatt.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    mod = _mutant(old, new)
    caught = False
    for ci in range(len(CASES)):
        try:
            test_finite_differences(ci, mod)
        except AssertionError:
            caught = True
            break
    assert caught, name
