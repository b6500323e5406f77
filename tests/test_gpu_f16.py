"""GPU parity of float16 inputs (VA_F16) with the oracle.

The same kernels as bf16, instantiated for the float16 MFMA and float16
rounding of P and dS: causal and non-causal, GQA and MQA, cross-length,
head_dim 64 and 128, sequences long enough to split into several work units
in every pass, per-key and per-pair biases (with their gradient), float32 and
float16 gradients, and the autograd path.  Tolerances (``tests/_gpu.py``):
the bf16 bounds scaled by the ratio of the two formats' unit roundoffs.
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_amd as va
from workloads import make_case

from . import _gpu

pytestmark = pytest.mark.gpu

CASES = [
    ("gqa7-causal-ragged", dict(seed=81, lens_q=[37, 300, 129, 64, 1, 5], hq=14, hkv=2, d=64, causal=True)),
    ("gqa7-causal-split", dict(seed=82, lens_q=[2600, 33, 700], hq=14, hkv=2, d=64, causal=True)),
    ("mqa-noncausal", dict(seed=83, lens_q=[200, 17, 64], hq=8, hkv=1, d=64, causal=False)),
    ("cross-d128", dict(seed=84, lens_q=[112, 50, 0], lens_k=[262, 90, 7], hq=32, hkv=8, d=128, causal=True)),
    ("d128-noncausal-long", dict(seed=85, lens_q=[900, 3], hq=4, hkv=2, d=128, causal=False)),
    ("per-key-bias", dict(seed=86, lens_q=[37, 300, 129], hq=8, hkv=8, d=64, causal=False, bias="per_key")),
    ("per-pair-bias-permuted", dict(seed=87, lens_q=[64, 200, 17], hq=4, hkv=2, d=64, causal=True,
                                    bias="per_pair", bias_layout="permuted", bias_std=0.5)),
]


@pytest.mark.parametrize("name,c", CASES, ids=[c[0] for c in CASES])
def test_f16_parity(name, c):
    print(f"[case] f16 {name}", flush=True)
    w = make_case(dtype="f16", with_dout=True, **c)
    _gpu.full_parity(w)


@pytest.mark.parametrize("name,c", CASES[:4:3], ids=[c[0] for c in CASES[:4:3]])
def test_f16_gradients_stored_f16(name, c):
    print(f"[case] f16 grads {name}", flush=True)
    w = make_case(dtype="f16", with_dout=True, **c)
    _gpu.full_parity(w, grad_dtype=torch.float16)


def _dbias_abs_tol(w, ref):
    """Max-abs bound of a float16 bias gradient.

    Besides the rounding of P and dS (the gradient rule of ``tests/_gpu.py``),
    D_i = rowsum(dO * O) is taken over O as the forward stored it, rounded to
    float16, so every dS_ij of row i moves by at most P_ij * 2^-11 * sum_j |dO_ij O_ij|,
    with P_ij <= 1.  Per-pair gradients hold one dS per element.
    """
    o, _ = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)
    row = float(np.max(np.sum(np.abs(o * w.dout), axis=-1)))
    return max(_gpu.grad_abs_tol("f16", ref, False), 2.0 ** -11 * row)


@pytest.mark.parametrize("bias", ["per_key", "per_pair"])
def test_f16_bias_grad(bias):
    print(f"[case] f16 dbias {bias}", flush=True)
    w = make_case(88, [37, 300, 129, 5], hq=4, hkv=2, d=64, causal=True, dtype="f16", bias=bias,
                  with_dout=True, bias_std=0.5)
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    db = torch.zeros(len(w.bias), dtype=torch.float32, device=_gpu.DEV)
    va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"], inp["cu_k"],
                     w.max_q, w.max_k, w.scale, True, inp["bias"], w.bias_strides, dbias=db,
                     dbias_stride=w.bias_strides)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True, w.bias, w.bias_strides,
                           len(w.bias))
    tol = _dbias_abs_tol(w, ref) if bias == "per_pair" else _gpu.grad_abs_tol("f16", ref, False)
    _gpu.check("dbias", _gpu.host(db), ref, "f16", grad=True, abs_tol=tol)


def test_f16_autograd():
    print("[case] f16 autograd", flush=True)
    w = make_case(89, [37, 300, 129], hq=4, hkv=2, d=64, causal=True, dtype="f16", with_dout=True)
    inp = _gpu.device_inputs(w)
    q, k, v = (inp[n].clone().requires_grad_(True) for n in "qkv")
    out, _ = va.varlen_attn(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    assert out.dtype == torch.float16
    (out.float() * inp["dout"].float()).sum().backward()
    torch.cuda.synchronize()
    g_ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    for name, t, ref in zip(("dq", "dk", "dv"), (q, k, v), g_ref):
        assert t.grad.dtype == torch.float16
        _gpu.check(name, _gpu.host(t.grad), ref, "f16", grad=True, abs_tol=_gpu.grad_abs_tol("f16", ref, False))
