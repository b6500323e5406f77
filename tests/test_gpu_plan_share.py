"""A forward that also builds its backward's work plans (va_varlen_fwd_bwdplan) and the
backward that takes them (va_varlen_bwd_planned) against the plain pair.

The plans are a pure function of cu_seqlens and the sizes, and each unit's results depend
neither on its place in the list nor on the workgroup that runs it, so the planned pair
must give bitwise the outputs of va_varlen_fwd / va_varlen_bwd (which the parity tests
compare with the oracle).  Cases: long sequences whose tiles split (merges), GQA, both
head dims, float32 and float16, per-key and per-pair (permuted) biases with their gradients,
and a forward that takes the short-query kernels; one buffer reused over calls, with an
unrelated backward between a forward and its planned backward.
"""

import pytest
import torch

import variable_length_packed_amd as va
from workloads import make_case

from . import _gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("split-bf16-d64-c1", dict(seed=71, lens_q=[3000, 17, 513, 1, 1200], hq=4, hkv=4, d=64,
                               causal=True, dtype="bf16", with_dout=True)),
    ("gqa-bf16-d128-c0", dict(seed=72, lens_q=[700, 129, 2048, 5], hq=8, hkv=2, d=128,
                              causal=False, dtype="bf16", with_dout=True)),
    ("f32-d64-c1", dict(seed=73, lens_q=[1100, 63, 255], hq=2, hkv=1, d=64, causal=True,
                        dtype="f32", with_dout=True)),
    ("f16-d128-c1", dict(seed=74, lens_q=[1500, 31, 1], hq=4, hkv=4, d=128, causal=True,
                         dtype="f16", with_dout=True)),
    ("short-query-bf16", dict(seed=75, lens_q=[1, 2, 1, 3], lens_k=[900, 64, 2500, 7], hq=8, hkv=2,
                              d=64, causal=True, dtype="bf16", with_dout=True)),
    ("bias-per-key-bf16", dict(seed=76, lens_q=[1300, 17, 400], hq=4, hkv=4, d=64, causal=False,
                               dtype="bf16", bias="per_key", with_dout=True)),
    ("bias-per-pair-permuted-bf16", dict(seed=77, lens_q=[700, 33, 260], hq=4, hkv=2, d=64, causal=True,
                                         dtype="bf16", bias="per_pair", bias_layout="permuted",
                                         with_dout=True)),
]


def _bws(w):
    n = va.va_varlen_bwd_workspace_size(w.batch, int(w.cu_q[-1]), int(w.cu_k[-1]), max(1, w.max_q),
                                        max(1, w.max_k), w.hq, w.hkv, w.d, _gpu.tdtype(w), torch.float32)
    return torch.empty(n, dtype=torch.uint8, device=_gpu.DEV)


def _dbias(w):
    if w.bias is None:
        return None
    return torch.zeros((len(w.bias),), dtype=torch.float32, device=_gpu.DEV)


def _run(w, inp, ws=None, between=None):
    """Forward + backward; with ``ws`` the forward plans the backward into it."""
    out, lse = _gpu.run_fwd(w, inp, bwd_workspace=ws)
    if between is not None:
        between()
    db = _dbias(w)
    dq, dk, dv = va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"],
                                  inp["cu_k"], max(1, w.max_q), max(1, w.max_k), w.scale, w.causal,
                                  inp["bias"], w.bias_strides if w.bias is not None else None,
                                  dbias=db, dbias_stride=w.bias_strides if db is not None else None,
                                  workspace=ws, planned=ws is not None)
    torch.cuda.synchronize()
    return [t for t in (out, lse, dq, dk, dv, db) if t is not None]


def _same(a, b):
    for name, x, y in zip(("out", "lse", "dq", "dk", "dv", "dbias"), a, b):
        assert torch.equal(x, y), f"{name} differs"


@pytest.mark.parametrize("name,c", CASES, ids=[c[0] for c in CASES])
def test_planned_backward_is_bitwise_the_plain_one(name, c):
    print(f"[case] plan share {name}", flush=True)
    w = make_case(**c)
    inp = _gpu.device_inputs(w)
    ref = _run(w, inp)
    ws = _bws(w)
    _same(_run(w, inp, ws), ref)
    # the same buffer again: the previous backward consumed the plans, this forward rebuilds them
    _same(_run(w, inp, ws), ref)


def test_other_calls_between_forward_and_planned_backward():
    """Plans live in the caller's buffer: an unrelated backward (its own workspace) between
    the forward and its planned backward leaves them alone."""
    print("[case] plan share with an unrelated backward between", flush=True)
    w = make_case(**CASES[0][1])
    w2 = make_case(**CASES[1][1])
    inp, inp2 = _gpu.device_inputs(w), _gpu.device_inputs(w2)
    ref = _run(w, inp)
    ref2 = _run(w2, inp2)
    got2 = []
    got = _run(w, inp, _bws(w), between=lambda: got2.extend(_run(w2, inp2)))
    _same(got, ref)
    _same(got2, ref2)
