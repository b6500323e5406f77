"""Pins for the packing oracle (``oracle.packing``): each check compares it with
something other than itself.

* hand-worked examples (``tests/golden/packing_examples.json``);
* library routines: ``numpy.flatnonzero`` for the kept positions and
  ``numpy.cumsum`` for the boundaries;
* invariants: pad(unpad(x)) is x with padding zeroed, unpad(pad(y)) is y,
  position ids count up from 0 inside each row;
* the reason the layout exists: attention over the packed stream, padded
  back, equals dense per-row attention whose padding keys are masked out
  (PyTorch's float64 scaled_dot_product_attention), for right-, left- and
  interior-padded rows (TorchEasyRec pull request 663 page, section
  "Choosing the kernel": the packed and the padded branches must agree).
"""

import json
import os
import types

import numpy as np
import pytest
import torch

import oracle
from oracle import packing as opk

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden():
    with open(os.path.join(GOLDEN, "packing_examples.json")) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _golden(), ids=lambda c: c["name"])
def test_hand_examples(case, mod=opk):
    cu, mx, idx, pos, inv = mod.pack_metadata(np.array(case["mask"], dtype=np.uint8))
    assert cu.tolist() == case["cu_seqlens"]
    assert mx == case["max_seqlen"]
    assert idx.tolist() == case["indices"]
    assert pos.tolist() == case["position_ids"]
    assert inv.tolist() == case["inverse"]


def _masks():
    rng = np.random.default_rng(7)
    out = []
    for b, s, kind in [(5, 9, "random"), (4, 16, "right"), (3, 12, "left"), (6, 1, "random"), (1, 33, "random")]:
        if kind == "random":
            m = (rng.random((b, s)) < 0.6).astype(np.uint8)
        else:
            lens = rng.integers(0, s + 1, size=b)
            m = np.zeros((b, s), dtype=np.uint8)
            for i, L in enumerate(lens):
                if kind == "right":
                    m[i, :L] = 1
                else:
                    m[i, s - L:] = 1
        out.append(m)
    return out


@pytest.mark.parametrize("mi", range(5))
def test_against_numpy_routines(mi):
    m = _masks()[mi]
    cu, mx, idx, pos, inv = opk.pack_metadata(m)
    assert np.array_equal(idx, np.flatnonzero(m.reshape(-1)))
    assert np.array_equal(cu, np.concatenate([[0], np.cumsum(m.sum(axis=1))]).astype(np.int32))
    assert mx == int(m.sum(axis=1).max())
    # position ids: t - cu[row of t]
    rows = idx // m.shape[1]
    assert np.array_equal(pos, np.arange(len(idx)) - cu[rows])
    # inverse is the inverse permutation on kept positions and -1 elsewhere
    assert np.array_equal(inv[idx], np.arange(len(idx)))
    assert np.all(inv[m.reshape(-1) == 0] == -1)


@pytest.mark.parametrize("mi", range(5))
def test_round_trips(mi):
    m = _masks()[mi]
    b, s = m.shape
    cu, _, idx, _, inv = opk.pack_metadata(m)
    rng = np.random.default_rng(mi)
    x = rng.standard_normal((b, s, 3, 2))
    packed = opk.unpad(x, idx)
    assert packed.shape == (int(m.sum()), 3, 2)
    back = opk.pad(packed, inv, b, s)
    assert np.array_equal(back, x * m[:, :, None, None])
    y = rng.standard_normal((int(m.sum()), 5))
    assert np.array_equal(opk.unpad(opk.pad(y, inv, b, s), idx), y)


@pytest.mark.parametrize("kind", ["right", "left", "interior"])
def test_packed_attention_equals_masked_dense(kind):
    """unpad -> varlen attention -> pad equals per-row dense attention over real keys."""
    rng = np.random.default_rng({"right": 1, "left": 2, "interior": 3}[kind])
    b, s, h, d = 3, 7, 2, 4
    m = np.zeros((b, s), dtype=np.uint8)
    for i, L in enumerate([7, 4, 1]):
        if kind == "right":
            m[i, :L] = 1
        elif kind == "left":
            m[i, s - L:] = 1
        else:
            m[i, rng.permutation(s)[:L]] = 1
    x = {n: rng.standard_normal((b, s, h, d)) for n in "qkv"}
    cu, _, idx, _, inv = opk.pack_metadata(m)
    q, k, v = (opk.unpad(x[n], idx) for n in "qkv")
    out, _ = oracle.forward(q, k, v, cu, cu, 0.5, False)
    got = opk.pad(out, inv, b, s)
    for i in range(b):
        keep = torch.from_numpy(m[i] != 0)
        qq, kk, vv = (torch.from_numpy(x[n][i]).transpose(0, 1) for n in "qkv")  # [h, s, d]
        ref = torch.nn.functional.scaled_dot_product_attention(
            qq, kk, vv, attn_mask=keep[None, None, :].expand(h, s, s), scale=0.5).transpose(0, 1).numpy()
        ref[m[i] == 0] = 0.0
        assert np.max(np.abs(got[i] - ref)) <= 1e-12


MUTATIONS = [
    ("positions from 1", "rank = 0\n", "rank = 1\n"),
    ("inverse off by one", "inverse[b * seqlen + s] = len(indices)", "inverse[b * seqlen + s] = len(indices) + 1"),
    ("row-major flat index transposed", "indices.append(b * seqlen + s)", "indices.append(s * batch + b)"),
    ("boundaries not cumulative", "cu[b + 1] = cu[b] + lens[b]", "cu[b + 1] = lens[b]"),
    ("pad keeps padding", "if inv[p] >= 0:", "if inv[p] >= -1:"),
]


def _mutant(old, new):
    path = opk.__file__
    with open(path) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("packing_mutant")
    exec(compile(src.replace(old, new), path, "exec"), mod.__dict__)
    return mod


def _pins_pass(mod) -> bool:
    try:
        for c in _golden():
            test_hand_examples(c, mod)
        m = _masks()[0]
        cu, _, idx, _, inv = mod.pack_metadata(m)
        x = np.random.default_rng(0).standard_normal(m.shape + (2,))
        if not np.array_equal(mod.pad(mod.unpad(x, idx), inv, *m.shape), x * m[:, :, None]):
            return False
    except Exception:
        return False
    return True


def test_pins_pass_on_unmodified_oracle():
    assert _pins_pass(opk)


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    assert not _pins_pass(_mutant(old, new)), name
