"""GPU parity of the bias gradient (va_varlen_bwd with dbias) with the oracle's ``bias_grad``.

Per-pair and per-key biases, contiguous and permuted layouts, a head-shared
per-key bias with one KV head, causal and not, cross-length, float32 and bf16,
head_dim 64 and 128, and sequences long enough that key tiles are split over
several work units (their per-key sums then go through the merge).  The
buffer is filled with NaN first: every element a valid (row, key) pair
addresses must be overwritten -- 0 where the causal mask hides the pair, as
the oracle's gradient is there -- and every other element left untouched.
Tolerances as for the other gradients (``tests/_gpu.py``).  The LDS-staged and
the loaded bias paths are also checked against each other, bitwise.
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
    ("pair-f32-causal", dict(seed=71, lens_q=[37, 300, 129, 5], hq=4, hkv=2, d=64, causal=True,
                             dtype="f32", bias="per_pair")),
    ("pair-bf16-noncausal-permuted", dict(seed=72, lens_q=[64, 200, 17], hq=4, hkv=2, d=64, causal=False,
                                         dtype="bf16", bias="per_pair", bias_layout="permuted")),
    ("pair-bf16-cross-d128", dict(seed=73, lens_q=[50, 112], lens_k=[90, 262], hq=8, hkv=2, d=128,
                                  causal=True, dtype="bf16", bias="per_pair")),
    ("pair-bf16-causal-split", dict(seed=81, lens_q=[700, 33, 450], hq=4, hkv=1, d=64, causal=True,
                                    dtype="bf16", bias="per_pair")),
    ("pair-f32-causal-qgtk", dict(seed=82, lens_q=[90, 20, 300], lens_k=[50, 20, 140], hq=2, hkv=1, d=64,
                                  causal=True, dtype="f32", bias="per_pair")),
    ("key-f32-gqa7", dict(seed=74, lens_q=[37, 300, 129, 64], hq=14, hkv=2, d=64, causal=True,
                          dtype="f32", bias="per_key")),
    ("key-bf16-split-long", dict(seed=75, lens_q=[1500, 33, 700], hq=14, hkv=2, d=64, causal=True,
                                 dtype="bf16", bias="per_key")),
    ("key-bf16-head-shared-mqa", dict(seed=76, lens_q=[300, 1200, 9], hq=8, hkv=1, d=64, causal=True,
                                      dtype="bf16", bias="per_key", bias_layout="head_shared")),
    ("key-f32-noncausal-d128", dict(seed=77, lens_q=[100, 260], lens_k=[180, 40], hq=2, hkv=2, d=128,
                                    causal=False, dtype="f32", bias="per_key")),
]


def _addressed(w):
    """Elements of the bias buffer that some valid (b, h, r < Lq, c < Lk) reads."""
    m = np.zeros(len(w.bias), dtype=bool)
    s0, s1, s2, s3 = (int(x) for x in w.bias_strides)
    for b in range(w.batch):
        lq, lk = int(w.cu_q[b + 1] - w.cu_q[b]), int(w.cu_k[b + 1] - w.cu_k[b])
        r = np.arange(lq, dtype=np.int64)[:, None]
        c = np.arange(lk, dtype=np.int64)[None, :]
        for h in range(w.hq):
            m[(b * s0 + h * s1 + r * s2 + c * s3).ravel()] = True
    return m


def _dbias(w, fill=float("nan")):
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    db = torch.full((len(w.bias),), fill, dtype=torch.float32, device=_gpu.DEV)
    va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"], inp["cu_k"],
                     max(1, w.max_q), max(1, w.max_k), w.scale, w.causal, inp["bias"], w.bias_strides,
                     dbias=db, dbias_stride=w.bias_strides)
    torch.cuda.synchronize()
    return _gpu.host(db)


@pytest.mark.parametrize("name,c", CASES, ids=[c[0] for c in CASES])
def test_bias_grad_parity(name, c):
    print(f"[case] dbias {name}", flush=True)
    w = make_case(with_dout=True, bias_std=0.5, **c)
    got = _dbias(w)
    ref = oracle.bias_grad(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                           w.bias_strides, len(w.bias))
    m = _addressed(w)
    assert np.all(np.isnan(got[~m])), "an element no valid pair addresses was written"
    assert np.all(np.isfinite(got[m])), "an element of a valid pair was not written"
    _gpu.check("dbias", got[m], ref[m], w.dtype, grad=True, abs_tol=_gpu.grad_abs_tol(w.dtype, ref, False))


def test_bias_grad_is_deterministic():
    print("[case] dbias determinism", flush=True)
    w = make_case(78, [1500, 33, 700], hq=14, hkv=2, d=64, causal=True, dtype="bf16", bias="per_key",
                  with_dout=True, bias_std=0.5)
    a, b = _dbias(w, 0.0), _dbias(w, 0.0)
    assert np.array_equal(a, b)


def test_autograd_bias_grad():
    """varlen_attn with a [B, H, 1, C] per-key bias that requires grad."""
    print("[case] dbias autograd", flush=True)
    w = make_case(79, [37, 300, 129], hq=4, hkv=2, d=64, causal=True, dtype="f32", bias="per_key",
                  with_dout=True, bias_std=0.5)
    B, H, C = w.batch, w.hq, w.max_k
    assert w.bias_strides == (H * C, C, 0, 1)
    inp = _gpu.device_inputs(w)
    bias = inp["bias"].view(B, H, 1, C).clone().requires_grad_(True)
    q, k, v = (inp[n].clone().requires_grad_(True) for n in "qkv")
    out, _ = va.varlen_attn(q, k, v, inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale, True, bias=bias)
    (out * inp["dout"]).sum().backward()
    torch.cuda.synchronize()
    ref = oracle.bias_grad(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True, w.bias, w.bias_strides,
                           len(w.bias))
    _gpu.check("dbias (autograd)", _gpu.host(bias.grad).reshape(-1), ref, "f32", grad=True)
    dq_ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, True, w.bias, w.bias_strides)[0]
    _gpu.check("dq (autograd)", _gpu.host(q.grad), dq_ref, "f32", grad=True)


@pytest.mark.parametrize("kind,dtype", [("per_pair", "bf16"), ("per_key", "f16"), ("per_pair", "f32")])
def test_staged_and_loaded_bias_paths_agree_bitwise(kind, dtype):
    """A contiguous-key bias whose base is 16-byte aligned goes through the LDS-staged tiles
    (16-bit forward and dK/dV) or vector loads; the same values one element off that
    alignment are read element by element.  Both must give identical results."""
    print(f"[case] bias paths {kind} {dtype}", flush=True)
    w = make_case(80, [64, 300, 17, 129], hq=4, hkv=2, d=64, causal=kind == "per_key", dtype=dtype,
                  bias=kind, with_dout=True, bias_std=0.5)
    inp = _gpu.device_inputs(w)
    dt = inp["q"].dtype
    buf = torch.zeros(len(w.bias) + 1, dtype=dt, device=_gpu.DEV)
    buf[1:] = inp["bias"]
    shifted = buf[1:]  # same values; base 1 element past 16-byte alignment
    assert inp["bias"].data_ptr() % 16 == 0 and shifted.data_ptr() % 16 != 0
    res = []
    for bias in (inp["bias"], shifted):
        out, lse = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k,
                                    w.scale, w.causal, bias, w.bias_strides)
        db = torch.zeros(len(w.bias), dtype=torch.float32, device=_gpu.DEV)
        grads = va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"], inp["cu_k"],
                                 w.max_q, w.max_k, w.scale, w.causal, bias, w.bias_strides, dbias=db,
                                 dbias_stride=w.bias_strides)
        torch.cuda.synchronize()
        res.append([out, lse, *grads, db])
    for name, a, b in zip(("out", "lse", "dq", "dk", "dv", "dbias"), *res):
        assert torch.equal(a, b), name
    o_ref, _ = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias, w.bias_strides)
    _gpu.check("out", _gpu.host(res[0][0]), o_ref, w.dtype)
