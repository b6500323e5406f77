"""GPU parity: the HIP path against the CPU fp64 oracle, element by element.

Unit matrix (full oracle): head dims 64/128; float32 and bf16; causal on/off;
bias none / per-key / per-pair / permuted strides / head stride 0; ragged
lengths spanning several 32/64/128 tiles and a ragged tail; cross-length
sequences with Lq < Lk and Lq > Lk (empty leading rows); empty sequences;
head layouts 1/1, 2/2, 8/8, 14/2, 32/8, 8/1.  The test plan of the FDMA pull
request 118 page (section "Recommended Automated Tests": lengths such as
(2, 37) and (4, 512), ragged [17, 5, 31], head dims 64 and 128, bias on and
off, causal decode with q_len 1) and the CUDA tests listed on the GiGL pull
request 858 page (section "Verification": per-key on and off, max_seq_len
not a multiple of 8, one head with full sequences, permuted-view bias) are
covered by these cases.  Long sequences exercise the split work units and
their merges; a max_seqlen hint below the true length must leave results
oracle-exact (it only makes the split coarser, or turns it off).
"""

import pytest
import torch

from workloads import make_case

from . import _gpu

pytestmark = pytest.mark.gpu

RAGGED = [1, 2, 3, 5, 17, 31, 37, 63, 64, 65, 127, 128, 129, 255, 256, 512]

CASES = []
for dt in ("f32", "bf16"):
    for d in (64, 128):
        for causal in (False, True):
            CASES.append((f"ragged-{dt}-d{d}-c{int(causal)}",
                          dict(seed=10 + d + causal, lens_q=RAGGED, hq=14, hkv=2, d=d,
                               causal=causal, dtype=dt, with_dout=True)))
    for bias, layout, causal in (("per_key", "contiguous", False), ("per_pair", "contiguous", False),
                                 ("per_pair", "permuted", True), ("per_key", "head_shared", True),
                                 ("per_pair", "head_shared", False)):
        CASES.append((f"bias-{bias}-{layout}-{dt}-c{int(causal)}",
                      dict(seed=30, lens_q=[17, 5, 31, 130, 2, 255], hq=8, hkv=8, d=64,
                           causal=causal, dtype=dt, bias=bias, bias_layout=layout, with_dout=True,
                           bias_std=0.5 if bias == "per_pair" else 1.0)))
    CASES.append((f"cross-qlt-{dt}", dict(seed=40, lens_q=[1, 5, 37, 112], lens_k=[7, 40, 37, 262],
                                          hq=32, hkv=8, d=128, causal=True, dtype=dt, with_dout=True)))
    CASES.append((f"cross-qgt-{dt}", dict(seed=41, lens_q=[40, 9, 130, 65], lens_k=[3, 9, 64, 1],
                                          hq=4, hkv=2, d=64, causal=True, dtype=dt, with_dout=True)))
    CASES.append((f"empty-seqs-{dt}", dict(seed=42, lens_q=[0, 5, 7, 0, 33], lens_k=[4, 0, 7, 0, 33],
                                           hq=8, hkv=1, d=64, causal=False, dtype=dt, with_dout=True)))
    CASES.append((f"one-head-full-{dt}", dict(seed=43, lens_q=[700, 256], hq=1, hkv=1, d=64,
                                              causal=True, dtype=dt, with_dout=True)))
    CASES.append((f"decode-q1-{dt}", dict(seed=44, lens_q=[1, 1, 1], lens_k=[37, 512, 1], hq=2, hkv=2,
                                          d=128, causal=True, dtype=dt, with_dout=True)))
    CASES.append((f"fdma-shapes-{dt}", dict(seed=45, lens_q=[37, 37, 512, 512, 512, 512], hq=2,
                                            hkv=2, d=64, causal=False, dtype=dt, with_dout=True,
                                            bias="per_pair", bias_std=0.5)))
    # tiles long enough to be split into several work units (forward and dQ:
    # more than 2048 keys; dK/dV: more than 1536 query-row x head pairs),
    # merged by the chunk that finishes last (forward, dQ) and by the dQ pass (dK/dV)
    CASES.append((f"split-long-{dt}", dict(seed=46, lens_q=[1500, 40, 2100], hq=4, hkv=1, d=64,
                                           causal=True, dtype=dt, with_dout=True)))
    CASES.append((f"split-cross-bias-{dt}", dict(seed=47, lens_q=[300, 1700], lens_k=[1300, 2600],
                                                 hq=2, hkv=2, d=64, causal=False, dtype=dt,
                                                 with_dout=True, bias="per_pair", bias_std=0.5)))
    CASES.append((f"split-decode-d128-{dt}", dict(seed=48, lens_q=[1, 3, 1200], lens_k=[3000, 1500, 2500],
                                                  hq=8, hkv=2, d=128, causal=True, dtype=dt,
                                                  with_dout=True)))


@pytest.mark.parametrize("name,c", CASES, ids=[c[0] for c in CASES])
def test_unit_matrix(name, c):
    print(f"[case] {name}", flush=True)
    w = make_case(**c)
    _gpu.full_parity(w)


def test_bf16_gradients_stored_bf16():
    """bf16 gradient storage: report-level tolerance (half a bf16 ulp of |g| added)."""
    w = make_case(50, [17, 130, 255], hq=14, hkv=2, d=64, causal=True, dtype="bf16", with_dout=True)
    import numpy as np
    import oracle
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    g = _gpu.run_bwd(w, out, lse, inp, grad_dtype=torch.bfloat16)
    ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal)
    for got, r in zip(g, ref):
        assert got.dtype == torch.bfloat16
        mx, rel = _gpu.errors(_gpu.host(got), r)
        assert rel <= 5e-3
        assert mx <= 2e-2 + np.max(np.abs(r)) * 2.0 ** -9


def test_autograd_matches_direct_calls():
    import variable_length_packed_amd as va
    w = make_case(51, [33, 200, 7], hq=4, hkv=2, d=64, causal=True, dtype="bf16", with_dout=True)
    inp = _gpu.device_inputs(w)
    q = inp["q"].clone().requires_grad_(True)
    k = inp["k"].clone().requires_grad_(True)
    v = inp["v"].clone().requires_grad_(True)
    out, lse = va.varlen_attn(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    out.backward(inp["dout"])
    o2, l2 = _gpu.run_fwd(w, inp)
    g2 = _gpu.run_bwd(w, o2, l2, inp)
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    assert torch.equal(q.grad, g2[0].to(q.dtype))
    assert torch.equal(k.grad, g2[1].to(k.dtype)) and torch.equal(v.grad, g2[2].to(v.dtype))


@pytest.mark.parametrize("hint", [64, 600])
def test_small_max_seqlen_hint_only_changes_the_split(hint):
    """max_seqlen is a sizing hint: one below the true maximum sizes fewer partial slots, so
    the planner takes coarser chunks (600) or none (64); results must stay oracle-exact."""
    import variable_length_packed_amd as va
    w = make_case(49, [2100, 33, 1800], hq=4, hkv=2, d=64, causal=True, dtype="bf16",
                  with_dout=True)
    print(f"[case] max_seqlen hint {hint}", flush=True)
    inp = _gpu.device_inputs(w)
    out, lse = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], hint, hint,
                                w.scale, True)
    dq, dk, dv = va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"],
                                  inp["cu_k"], hint, hint, w.scale, True)
    out2, lse2 = _gpu.run_fwd(w, inp)
    g2 = _gpu.run_bwd(w, out2, lse2, inp)
    torch.cuda.synchronize()
    import oracle
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    for got in ((out, lse, dq, dk, dv), (out2, lse2) + tuple(g2)):
        _gpu.check("out", _gpu.host(got[0]), o_ref, w.dtype)
        _gpu.check_lse(_gpu.host(got[1]), l_ref, w.dtype)
        for n, g, r in zip(("dq", "dk", "dv"), got[2:], ref):
            _gpu.check(n, _gpu.host(g), r, w.dtype, grad=True,
                       abs_tol=_gpu.grad_abs_tol(w.dtype, r, False))
