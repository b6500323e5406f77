"""GPU parity of the packed forward's short-query path with the oracle.

With few new tokens per sequence by the
max_seqlen_q hint (at most 16, or 32 with at most 128 (token, query head) rows
per KV head), va_varlen_fwd runs the decode kernels over contiguous (or
strided) K/V read through cu_seqlens_k: decode steps and short drafts without
a page table.  Checked: single-token steps over
ragged caches (empty, short, split over tens of chunks), drafts of up to 8
tokens with 4 heads per KV head (32 rows), non-causal, MQA, float16, float32,
an additive bias per key or per pair (contiguous, permuted, head-shared), K and V
interleaved in one buffer, hints smaller than the true lengths (more row
blocks and longer chunks, same results), bitwise determinism, and the backward
run on the forward's O and LSE.
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_amd as va
from workloads import make_case

from . import _gpu

pytestmark = pytest.mark.gpu

DEV = _gpu.DEV

CASES = [
    ("decode-gqa4-d128", dict(seed=101, lens_q=[1] * 6, lens_k=[1, 17, 300, 3000, 0, 9000], hq=32, hkv=8,
                              d=128, causal=True, dtype="bf16")),
    ("draft8-gqa4-d64", dict(seed=102, lens_q=[8, 3, 8, 1], lens_k=[8, 700, 5000, 2], hq=8, hkv=2, d=64,
                             causal=True, dtype="bf16")),
    ("noncausal-mqa-f16", dict(seed=103, lens_q=[2, 1, 2], lens_k=[64, 1025, 4097], hq=16, hkv=1, d=128,
                               causal=False, dtype="f16")),
    ("mha-tokens-0-and-1", dict(seed=104, lens_q=[1, 0, 1, 1], lens_k=[33, 50, 0, 2], hq=4, hkv=4, d=64,
                                causal=True, dtype="bf16")),
    ("draft5-gqa4-d32", dict(seed=108, lens_q=[5, 1, 2], lens_k=[3000, 64, 9], hq=8, hkv=2, d=32,
                             causal=True, dtype="bf16")),
    ("decode-gqa2-d96-f16", dict(seed=109, lens_q=[1, 3, 1], lens_k=[4500, 35, 1], hq=8, hkv=4, d=96,
                                 causal=True, dtype="f16")),
    # float32: the float32 decode kernel
    ("decode-gqa4-d128-f32", dict(seed=110, lens_q=[1] * 5, lens_k=[1, 17, 3000, 0, 9000], hq=32, hkv=8,
                                  d=128, causal=True, dtype="f32")),
    ("draft6-gqa2-d64-f32-noncausal", dict(seed=111, lens_q=[6, 2, 1], lens_k=[700, 4100, 3], hq=8, hkv=4, d=64,
                                           causal=False, dtype="f32")),
    ("draft4-mqa-d32-f32", dict(seed=112, lens_q=[4, 1], lens_k=[2500, 31], hq=8, hkv=1, d=32,
                                causal=True, dtype="f32")),
    # an additive bias (GiGL "Approach": per sequence, through a strided view) on the decode
    # kernels: per key (row stride 0), per pair, a permuted view (no unit key stride: one
    # element per load) and a head-shared grid
    ("decode-gqa4-d128-bf16-bias-key", dict(seed=113, lens_q=[1] * 4, lens_k=[1, 300, 3000, 9000], hq=32, hkv=8,
                                            d=128, causal=True, dtype="bf16", bias="per_key")),
    ("draft6-gqa2-d64-f16-bias-pair", dict(seed=114, lens_q=[6, 2, 1], lens_k=[700, 4100, 3], hq=8, hkv=4,
                                           d=64, causal=True, dtype="f16", bias="per_pair", bias_std=0.5)),
    ("draft3-mqa-d64-bf16-bias-permuted", dict(seed=115, lens_q=[3, 1], lens_k=[1300, 40], hq=8, hkv=1, d=64,
                                               causal=False, dtype="bf16", bias="per_pair",
                                               bias_layout="permuted")),
    ("draft4-gqa4-d128-f32-bias-pair", dict(seed=116, lens_q=[4, 1, 2], lens_k=[2500, 31, 5000], hq=16, hkv=4,
                                            d=128, causal=True, dtype="f32", bias="per_pair", bias_std=0.5)),
    ("decode-d96-f32-bias-head-shared", dict(seed=117, lens_q=[1, 2], lens_k=[777, 3000], hq=8, hkv=2, d=96,
                                             causal=True, dtype="f32", bias="per_pair",
                                             bias_layout="head_shared")),
]


@pytest.mark.parametrize("name,c", CASES, ids=[x[0] for x in CASES])
def test_short_query_parity(name, c):
    print(f"[case] short query {name}", flush=True)
    w = make_case(with_dout=True, **c)
    assert max(w.lens_q) <= 16  # takes the decode kernels
    _gpu.full_parity(w)


def test_hints_below_the_true_lengths():
    """max_seqlen_q / max_seqlen_k of 1 for sequences of up to 6 tokens and 5000 keys."""
    print("[case] short query, small hints", flush=True)
    w = make_case(105, [6, 1, 3], lens_k=[5000, 40, 1300], hq=16, hkv=4, d=64, causal=True, dtype="bf16")
    inp = _gpu.device_inputs(w)
    o1, l1 = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 1, 1, w.scale, True)
    o2, l2 = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k,
                              w.scale, True)
    torch.cuda.synchronize()
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    for o, l in ((o1, l1), (o2, l2)):
        _gpu.check("out", _gpu.host(o), o_ref, "bf16")
        _gpu.check_lse(_gpu.host(l), l_ref, "bf16")


def test_interleaved_kv_and_determinism():
    print("[case] short query, K/V in one buffer", flush=True)
    w = make_case(106, [1, 2, 1], lens_k=[3000, 77, 1], hq=8, hkv=2, d=128, causal=True, dtype="bf16")
    inp = _gpu.device_inputs(w)
    kv = torch.stack([inp["k"], inp["v"]], dim=1).contiguous()
    k, v = kv[:, 0], kv[:, 1]
    va.va_timing_start(64)
    a = va.va_varlen_fwd(inp["q"], k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    b = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    torch.cuda.synchronize()
    names = set(va.va_timing_stop())
    assert "kvcache_bf16" in names and "fwd_bf16" not in names, names  # the decode kernels ran
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    _gpu.check("out", _gpu.host(a[0]), o_ref, "bf16")
    _gpu.check_lse(_gpu.host(a[1]), l_ref, "bf16")


def test_short_query_lse_feeds_the_backward():
    """The backward recomputes P from the LSE the decode kernels wrote."""
    print("[case] short query backward", flush=True)
    w = make_case(107, [4, 1, 8], lens_k=[300, 2000, 8], hq=8, hkv=2, d=64, causal=True, dtype="bf16",
                  with_dout=True)
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    dq, dk, dv = _gpu.run_bwd(w, out, lse, inp)
    torch.cuda.synchronize()
    g_ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    for nm, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
        _gpu.check(nm, _gpu.host(got), ref, "bf16", grad=True, abs_tol=_gpu.grad_abs_tol("bf16", ref, False))
    np.testing.assert_array_equal(np.isneginf(_gpu.host(lse)), np.zeros_like(_gpu.host(lse), dtype=bool))


@pytest.mark.parametrize("dtype,kernel", [("bf16", "kvcache_bf16"), ("f32", "kvcache_f32")])
def test_bias_calls_take_the_decode_kernels(dtype, kernel):
    """A short-query call with a bias runs the decode kernels (not the 128-row tiles)."""
    print(f"[case] short query with a bias: kernel names ({dtype})", flush=True)
    w = make_case(118, [2, 1], lens_k=[600, 90], hq=8, hkv=2, d=64, causal=True, dtype=dtype,
                  bias="per_pair")
    inp = _gpu.device_inputs(w)
    torch.cuda.synchronize()
    va.va_timing_start(64)
    _gpu.run_fwd(w, inp)
    names = set(va.va_timing_stop())
    assert kernel in names and not any(n.startswith("fwd_") for n in names), names
