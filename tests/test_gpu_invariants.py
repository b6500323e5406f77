"""GPU invariants: bit-identical row isolation, run-to-run determinism, no out-of-bounds
writes and no unwritten outputs.

Isolation follows the TorchEasyRec pull request 663 page (section "Test plan": rewrite
row 0 and another row's result must stay bit-identical), with a row read as one
packed sequence: redrawing sequence 0 (its Q/K/V/dO and bias slice), or changing its
length (which moves every later offset), leaves every other sequence's O, LSE, dQ, dK
and dV bitwise unchanged.
"""

import numpy as np
import pytest
import torch

import variable_length_packed_amd as va
from workloads import make_case

from . import _gpu

pytestmark = pytest.mark.gpu

LENS = [37, 300, 129, 64, 2600, 5]  # 2600: split work units in every pass


def _run_all(w):
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    dq, dk, dv = _gpu.run_bwd(w, out, lse, inp)
    torch.cuda.synchronize()
    return [x.detach().clone() for x in (out, lse, dq, dk, dv)]


LENS_BIAS = [37, 300, 129, 64, 1000, 5]  # keeps the per-pair bias grid at 1024 x 1024 (dK/dV split)


def _case(seed, lens_q, lens_k=None, bias=False, dtype="bf16"):
    return make_case(seed, lens_q, lens_k=lens_k, hq=14, hkv=2, d=64, causal=True, dtype=dtype,
                     bias="per_pair" if bias else "none", with_dout=True, bias_std=0.5,
                     grid=(1024, 1024) if bias else None)


@pytest.mark.parametrize("bias", [False, True])
def test_isolation_rewrite_values(bias):
    lens = LENS_BIAS if bias else LENS
    w = _case(60, lens, bias=bias)
    base = _run_all(w)
    w2 = _case(61, lens, bias=bias)  # every value differs ...
    n0 = lens[0]
    for a, b in ((w2.q, w.q), (w2.k, w.k), (w2.v, w.v), (w2.dout, w.dout)):
        a[n0:] = b[n0:]  # ... except sequences 1.. are copied back
    if bias:
        s0 = w.bias_strides[0]
        w2.bias[s0:] = w.bias[s0:]
    new = _run_all(w2)
    out, lse, dq, dk, dv = base
    o2, l2, dq2, dk2, dv2 = new
    assert not torch.equal(o2[:n0], out[:n0])
    assert torch.equal(o2[n0:], out[n0:]) and torch.equal(l2[:, n0:], lse[:, n0:])
    assert torch.equal(dq2[n0:], dq[n0:])
    assert torch.equal(dk2[n0:], dk[n0:]) and torch.equal(dv2[n0:], dv[n0:])


def test_isolation_change_length():
    w = _case(62, LENS)
    base = _run_all(w)
    lens2 = [200] + LENS[1:]
    w2 = _case(63, lens2)
    n0, m0 = LENS[0], lens2[0]
    for a, b in ((w2.q, w.q), (w2.k, w.k), (w2.v, w.v), (w2.dout, w.dout)):
        a[m0:] = b[n0:]
    new = _run_all(w2)
    for x, y in zip(base, new):
        if x.dim() == 2:  # lse [H, T]
            assert torch.equal(y[:, m0:], x[:, n0:])
        else:
            assert torch.equal(y[m0:], x[n0:])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_determinism(dtype):
    w = make_case(64, LENS, hq=8, hkv=2, d=128, causal=True, dtype=dtype, with_dout=True)
    a = _run_all(w)
    b = _run_all(w)
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def _guarded(shape, dtype, pad=4096, canary=12345.0):
    n = int(np.prod(shape))
    buf = torch.full((n + 2 * pad,), canary, dtype=dtype, device=_gpu.DEV)
    view = buf[pad:pad + n].view(*shape)
    view.fill_(float("nan"))
    return buf, view


def _canary_intact(buf, n, pad=4096, canary=12345.0):
    return bool((buf[:pad] == canary).all()) and bool((buf[pad + n:] == canary).all())


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", [False, True])
def test_guard_bands_and_full_overwrite(dtype, bias):
    w = make_case(65, [1, 63, 0, 129, 17], lens_k=[40, 63, 3, 100, 1], hq=4, hkv=2, d=64,
                  causal=True, dtype=dtype, with_dout=True,
                  bias="per_pair" if bias else "none")
    inp = _gpu.device_inputs(w)
    tdt = _gpu.tdtype(w)
    ob, out = _guarded(inp["q"].shape, tdt)
    lb, lse = _guarded((w.hq, w.total_q), torch.float32)
    va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k,
                     w.scale, True, inp["bias"], w.bias_strides, out=out, lse=lse)
    qb, dq = _guarded(inp["q"].shape, torch.float32)
    kb, dk = _guarded(inp["k"].shape, torch.float32)
    vb, dv = _guarded(inp["v"].shape, torch.float32)
    va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"],
                     inp["cu_k"], w.max_q, w.max_k, w.scale, True, inp["bias"], w.bias_strides,
                     dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    for buf, view in ((ob, out), (qb, dq), (kb, dk), (vb, dv)):
        assert _canary_intact(buf, view.numel()), "write outside the output"
        assert not torch.isnan(view).any(), "an output element was not written"
    assert _canary_intact(lb, lse.numel())
    # LSE: -inf exactly on rows that see no key, finite elsewhere
    assert not torch.isnan(lse).any()
    _gpu.full_parity(w)


def test_python_errors_on_gpu_tensors():
    w = make_case(66, [5, 7], hq=2, hkv=2, d=64, dtype="bf16", with_dout=True)
    inp = _gpu.device_inputs(w)
    with pytest.raises(ValueError):  # zero-length batch (empty cu_seqlens)
        va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"][:1], inp["cu_k"][:1], 5, 5)
    with pytest.raises(ValueError):  # unsupported head dim
        q = torch.zeros(12, 2, 80, dtype=torch.bfloat16, device=_gpu.DEV)
        va.va_varlen_fwd(q, q, q, inp["cu_q"], inp["cu_k"], 7, 7)
    with pytest.raises(ValueError):  # non-contiguous input
        va.va_varlen_fwd(inp["q"].transpose(0, 1), inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 7, 7)
    b = torch.zeros(2, 2, 7, 7, dtype=torch.bfloat16, device=_gpu.DEV, requires_grad=True)
    with pytest.raises(ValueError):  # a bias that needs a gradient, read through an explicit view
        va.varlen_attn(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 7, 7, bias=b,
                       bias_stride=(98, 49, 7, 1))
    with pytest.raises(ValueError):  # bias view reaching past its storage
        small = torch.zeros(2, 2, 3, 3, dtype=torch.bfloat16, device=_gpu.DEV)
        va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 7, 7, bias=small)
