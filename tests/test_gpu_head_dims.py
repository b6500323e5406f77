"""GPU parity with the oracle at head_dim 32, 96 and 256 (the packed forward and backward).

The same kernels as at 64 and 128, instantiated for one, three and eight
32-wide output tiles (at 256 with 32-key blocks in the forward and dQ pass,
and two dK/dV work items per unit, each with half of the dims): float32, bf16
and float16;
causal and not; GQA, MQA and MHA;
cross-length; sequences long enough to split in every pass; per-key and
per-pair biases with their gradients; 16-bit gradients; a fused QKV input.
Tolerances as for the other shapes (``tests/_gpu.py``).
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
    ("d32-bf16-gqa7-causal-split", dict(seed=111, lens_q=[37, 300, 129, 2600, 5], hq=14, hkv=2, d=32,
                                        causal=True, dtype="bf16")),
    ("d96-bf16-gqa4-causal-split", dict(seed=112, lens_q=[2600, 64, 1], hq=8, hkv=2, d=96, causal=True,
                                        dtype="bf16")),
    ("d96-f16-cross-mqa", dict(seed=113, lens_q=[112, 50, 0], lens_k=[262, 90, 7], hq=8, hkv=1, d=96,
                               causal=True, dtype="f16")),
    ("d32-f32-noncausal-mha", dict(seed=114, lens_q=[100, 260, 3], hq=4, hkv=4, d=32, causal=False,
                                   dtype="f32")),
    ("d96-f32-causal-gqa", dict(seed=115, lens_q=[200, 37], hq=4, hkv=2, d=96, causal=True, dtype="f32")),
    ("d32-f16-short-rows", dict(seed=116, lens_q=[1, 4, 2], lens_k=[700, 40, 2000], hq=16, hkv=4, d=32,
                                causal=True, dtype="f16")),
    ("d256-bf16-gqa4-causal-split", dict(seed=120, lens_q=[300, 2200, 17], hq=8, hkv=2, d=256, causal=True,
                                         dtype="bf16")),
    ("d256-f32-noncausal-mqa", dict(seed=121, lens_q=[100, 37, 1], hq=2, hkv=1, d=256, causal=False,
                                    dtype="f32")),
    ("d256-f16-cross-mha", dict(seed=122, lens_q=[112, 5, 0], lens_k=[262, 40, 9], hq=4, hkv=4, d=256,
                                causal=True, dtype="f16")),
]


@pytest.mark.parametrize("name,c", CASES, ids=[x[0] for x in CASES])
def test_head_dim_parity(name, c):
    print(f"[case] head dim {name}", flush=True)
    w = make_case(with_dout=True, **c)
    _gpu.full_parity(w)


@pytest.mark.parametrize("name,c", CASES[:2], ids=[x[0] for x in CASES[:2]])
def test_head_dim_16bit_gradients(name, c):
    print(f"[case] head dim 16-bit grads {name}", flush=True)
    w = make_case(with_dout=True, **c)
    _gpu.full_parity(w, grad_dtype=torch.bfloat16)


BIAS = [
    ("d32-f32-per-key", dict(seed=117, lens_q=[37, 300, 129], hq=4, hkv=2, d=32, causal=True, dtype="f32",
                             bias="per_key")),
    ("d96-bf16-per-pair-permuted", dict(seed=118, lens_q=[64, 200, 17], hq=4, hkv=2, d=96, causal=False,
                                        dtype="bf16", bias="per_pair", bias_layout="permuted")),
    ("d256-bf16-per-key", dict(seed=123, lens_q=[37, 300], hq=8, hkv=2, d=256, causal=True, dtype="bf16",
                               bias="per_key")),
    ("d256-f16-per-pair", dict(seed=124, lens_q=[64, 150], hq=2, hkv=2, d=256, causal=False, dtype="f16",
                               bias="per_pair")),
]


@pytest.mark.parametrize("name,c", BIAS, ids=[x[0] for x in BIAS])
def test_head_dim_bias_and_its_gradient(name, c):
    print(f"[case] head dim bias {name}", flush=True)
    w = make_case(with_dout=True, bias_std=0.5, **c)
    _gpu.full_parity(w)
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    db = torch.zeros(len(w.bias), dtype=torch.float32, device=DEV)
    va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"], inp["cu_k"],
                     w.max_q, w.max_k, w.scale, w.causal, inp["bias"], w.bias_strides, dbias=db,
                     dbias_stride=w.bias_strides)
    torch.cuda.synchronize()
    ref = oracle.bias_grad(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides,
                           len(w.bias))
    _gpu.check("dbias", _gpu.host(db), ref, w.dtype, grad=True, abs_tol=_gpu.grad_abs_tol(w.dtype, ref, False))


def test_head_dim_96_fused_qkv():
    print("[case] head dim 96 fused qkv", flush=True)
    w = make_case(119, [37, 300, 129], hq=6, hkv=2, d=96, causal=True, dtype="bf16", with_dout=True)
    inp = _gpu.device_inputs(w)
    qkv = torch.cat([inp["q"], inp["k"], inp["v"]], dim=1).contiguous()
    q, k, v = qkv[:, :w.hq], qkv[:, w.hq:w.hq + w.hkv], qkv[:, w.hq + w.hkv:]
    out, lse = va.va_varlen_fwd(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True)
    o2, l2 = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k,
                              w.scale, True)
    torch.cuda.synchronize()
    assert torch.equal(out, o2) and torch.equal(lse, l2)
    o_ref, _ = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True)
    _gpu.check("out", _gpu.host(out), o_ref, "bf16")
    assert np.isfinite(_gpu.host(lse)).all()
