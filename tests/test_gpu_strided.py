"""GPU parity of strided Q/K/V (token strides other than heads * head_dim).

Q, K and V read in place from one fused projection output [T, Hq + 2 Hkv, d]
(the QKV-packed input of flash_attn_qkvpacked_func, which the noether pull
request 236 page lists), K and V from one [Tk, 2, Hkv, d] buffer, and rows
padded to a larger stride.  The kernels read rows through the token stride
and nothing else changes, so strided inputs must give results bitwise equal to
contiguous copies of the same values; they are also checked against the oracle,
forward and backward (with a bias and its gradient in one case), and through
autograd, where the gradients of the three slices land in one fused gradient.
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


def _fused(w, dt):
    """Q, K, V as slices of one [T, Hq + 2 Hkv, d] buffer (self-attention: Tq = Tk)."""
    qkv = torch.cat([_gpu.to_dev(w.q, dt), _gpu.to_dev(w.k, dt), _gpu.to_dev(w.v, dt)], dim=1).contiguous()
    return qkv, qkv[:, :w.hq], qkv[:, w.hq:w.hq + w.hkv], qkv[:, w.hq + w.hkv:]


def _run(w, q, k, v, inp, dbias=None):
    out, lse = va.va_varlen_fwd(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, w.causal,
                                inp["bias"], w.bias_strides)
    grads = va.va_varlen_bwd(inp["dout"], q, k, v, out, lse, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k,
                             w.scale, w.causal, inp["bias"], w.bias_strides, dbias=dbias,
                             dbias_stride=None if dbias is None else w.bias_strides)
    torch.cuda.synchronize()
    return [out, lse] + list(grads)


FUSED = [
    ("bf16-gqa7-causal-split", dict(seed=91, lens_q=[37, 300, 129, 2600, 5], hq=14, hkv=2, d=64, causal=True,
                                    dtype="bf16")),
    ("f32-d128-noncausal", dict(seed=92, lens_q=[100, 260, 1], hq=4, hkv=4, d=128, causal=False, dtype="f32")),
    ("f16-mqa-per-key-bias", dict(seed=93, lens_q=[64, 200, 17], hq=8, hkv=1, d=64, causal=True, dtype="f16",
                                  bias="per_key", bias_std=0.5)),
]


@pytest.mark.parametrize("name,c", FUSED, ids=[f[0] for f in FUSED])
def test_fused_qkv_matches_contiguous_bitwise_and_the_oracle(name, c):
    print(f"[case] fused qkv {name}", flush=True)
    w = make_case(with_dout=True, **c)
    dt = _gpu.tdtype(w)
    inp = _gpu.device_inputs(w)
    _, q, k, v = _fused(w, dt)
    assert not q.is_contiguous() and q.stride(0) == (w.hq + 2 * w.hkv) * w.d
    has_db = w.bias is not None
    db_s = torch.zeros(len(w.bias), dtype=torch.float32, device=DEV) if has_db else None
    db_c = torch.zeros_like(db_s) if has_db else None
    strided = _run(w, q, k, v, inp, db_s)
    dense = _run(w, inp["q"], inp["k"], inp["v"], inp, db_c)
    for a, b in zip(strided, dense):
        assert torch.equal(a, b)
    if has_db:
        assert torch.equal(db_s, db_c)
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)
    _gpu.check("out", _gpu.host(strided[0]), o_ref, w.dtype)
    _gpu.check_lse(_gpu.host(strided[1]), l_ref, w.dtype)
    g_ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)
    for nm, got, ref in zip(("dq", "dk", "dv"), strided[2:], g_ref):
        _gpu.check(nm, _gpu.host(got), ref, w.dtype, grad=True, abs_tol=_gpu.grad_abs_tol(w.dtype, ref, False))


def test_kv_packed_and_padded_rows():
    """K and V from one [Tk, 2, Hkv, d] buffer, Q with 64 elements of padding per row."""
    print("[case] kv-packed, padded q rows", flush=True)
    w = make_case(94, [50, 112, 3], lens_k=[90, 262, 0], hq=32, hkv=8, d=128, causal=True, dtype="bf16",
                  with_dout=True)
    inp = _gpu.device_inputs(w)
    kv = torch.stack([inp["k"], inp["v"]], dim=1).contiguous()
    k, v = kv[:, 0], kv[:, 1]
    qbuf = torch.zeros(w.total_q, w.hq * w.d + 64, dtype=torch.bfloat16, device=DEV)
    qbuf[:, :w.hq * w.d] = inp["q"].reshape(w.total_q, -1)
    q = qbuf[:, :w.hq * w.d].view(w.total_q, w.hq, w.d)
    assert k.stride(0) == 2 * w.hkv * w.d and q.stride(0) == w.hq * w.d + 64
    strided = _run(w, q, k, v, inp)
    dense = _run(w, inp["q"], inp["k"], inp["v"], inp)
    for a, b in zip(strided, dense):
        assert torch.equal(a, b)
    _gpu.full_parity(w)


def test_autograd_through_a_fused_qkv():
    print("[case] autograd fused qkv", flush=True)
    w = make_case(95, [37, 300, 129], hq=4, hkv=2, d=64, causal=True, dtype="f32", with_dout=True)
    inp = _gpu.device_inputs(w)
    qkv, _, _, _ = _fused(w, torch.float32)
    qkv.requires_grad_(True)
    q, k, v = qkv[:, :w.hq], qkv[:, w.hq:w.hq + w.hkv], qkv[:, w.hq + w.hkv:]
    out, _ = va.varlen_attn(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    (out * inp["dout"]).sum().backward()
    torch.cuda.synchronize()
    dq, dk, dv = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    ref = np.concatenate([dq, dk, dv], axis=1)
    _gpu.check("d(qkv)", _gpu.host(qkv.grad), ref, "f32", grad=True)


def test_strided_errors():
    print("[case] strided errors", flush=True)
    w = make_case(96, [5, 7], hq=2, hkv=2, d=64, dtype="bf16", with_dout=True)
    inp = _gpu.device_inputs(w)
    qt = inp["q"].transpose(1, 2).contiguous().transpose(1, 2)  # heads not dense
    with pytest.raises(ValueError):
        va.va_varlen_fwd(qt, inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 7, 7)
    buf = torch.zeros(w.total_q, w.hq * w.d + 4, dtype=torch.bfloat16, device=DEV)  # 8-byte row padding
    q = buf[:, :w.hq * w.d].view(w.total_q, w.hq, w.d)
    with pytest.raises(ValueError):  # rows not 16-byte aligned: the library refuses
        va.va_varlen_fwd(q, inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], 7, 7)
