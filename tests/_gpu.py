"""Helpers for GPU tests: run a workload through the C ABI and compare with the oracle.

Tolerances (per output tensor, over all valid elements, computed in float64):
float32 runs: max-abs <= 1e-5 on O and LSE; gradients max-abs <= 1e-5 * max(1, max|ref|):
the absolute 1e-5 while every gradient of the tensor stays within +-1, scaled by the
largest gradient beyond that, because each gradient is a float32 sum over up to thousands
of query rows (or keys) whose rounding error grows with the magnitude of the sum (float32
unit roundoff 6e-8 per addition); measured dK error 2.0e-6 at max|dK| 4.9.  bf16 runs: max-abs <= 2e-2 and
relative L2 <= 5e-3 on every tensor (gradients stored float32).  On shapes other than
the five named workloads, a bf16 gradient's max-abs bound is max(2e-2, 2^-8 * max|ref|):
the kernels round P and dS to bf16 (relative error <= 2^-9 per term) before the
contractions, so the error of the largest gradients grows with their magnitude.
float16 runs take the bf16 bounds scaled by 2^-3, the ratio of the two formats' unit
roundoffs (10 against 7 fraction bits): max-abs <= 2.5e-3, relative L2 <= 6.25e-4, and
max(2.5e-3, 2^-11 * max|ref|) for gradients off the named workloads.
"""

from __future__ import annotations

import numpy as np
import torch

import oracle

DEV = torch.device("cuda:0")
TOL = {"f32": dict(abs=1e-5), "bf16": dict(abs=2e-2, rel=5e-3), "f16": dict(abs=2.5e-3, rel=6.25e-4)}
_TORCH = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
_UNIT = {"bf16": 2.0 ** -8, "f16": 2.0 ** -11}  # unit roundoff of each 16-bit format


def tdtype(w):
    return _TORCH[w.dtype]


def to_dev(x, dt):
    return torch.from_numpy(np.ascontiguousarray(x)).to(DEV).to(dt).contiguous()


def device_inputs(w):
    dt = tdtype(w)
    d = dict(q=to_dev(w.q, dt), k=to_dev(w.k, dt), v=to_dev(w.v, dt),
             cu_q=torch.from_numpy(w.cu_q).to(DEV), cu_k=torch.from_numpy(w.cu_k).to(DEV))
    d["bias"] = to_dev(w.bias, dt) if w.bias is not None else None
    d["dout"] = to_dev(w.dout, dt) if w.dout is not None else None
    return d


def run_fwd(w, inp=None, **kw):
    import variable_length_packed_amd as va
    inp = inp or device_inputs(w)
    out, lse = va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"],
                                max(1, w.max_q), max(1, w.max_k), w.scale, w.causal, inp["bias"],
                                w.bias_strides if w.bias is not None else None, **kw)
    return out, lse


def run_bwd(w, out, lse, inp=None, grad_dtype=torch.float32):
    import variable_length_packed_amd as va
    inp = inp or device_inputs(w)
    return va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], out, lse, inp["cu_q"],
                            inp["cu_k"], max(1, w.max_q), max(1, w.max_k), w.scale, w.causal,
                            inp["bias"], w.bias_strides if w.bias is not None else None,
                            grad_dtype=grad_dtype)


def host(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def errors(got, ref):
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    diff = got - ref
    mx = float(np.max(np.abs(diff))) if diff.size else 0.0
    nr = float(np.linalg.norm(ref))
    rel = float(np.linalg.norm(diff) / nr) if nr > 0 else (0.0 if mx == 0 else np.inf)
    return mx, rel


def check(name, got, ref, dtype, grad=False, abs_tol=None):
    mx, rel = errors(got, ref)
    tol = TOL[dtype]
    big = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    msg = f"{name}: max-abs {mx:.3g} rel-L2 {rel:.3g} max|ref| {big:.3g}"
    print("   ", msg, flush=True)
    if dtype == "f32":
        lim = tol["abs"] * (max(1.0, big) if grad else 1.0)
        assert mx <= lim, f"{msg} (limit {lim:.3g})"
    else:
        lim = tol["abs"] if abs_tol is None else abs_tol
        assert mx <= lim, f"{msg} (limit {lim:.3g})"
        assert rel <= tol["rel"], f"{msg} (rel limit {tol['rel']})"
    return mx, rel


def check_lse(got, ref, dtype):
    fin = np.isfinite(ref)
    assert np.array_equal(np.isfinite(got), fin), "LSE -inf pattern differs"
    assert np.all(np.isneginf(got[~fin])), "empty rows must have LSE = -inf"
    return check("lse", got[fin], ref[fin], dtype)


def grad_abs_tol(dtype, ref, named_workload):
    if dtype == "f32" or named_workload:
        return None
    big = float(np.max(np.abs(ref))) if np.size(ref) else 0.0
    return max(TOL[dtype]["abs"], _UNIT[dtype] * big)


def full_parity(w, backward=None, grad_dtype=torch.float32, named_workload=False):
    """Element-by-element comparison with the full oracle (small problems)."""
    inp = device_inputs(w)
    out, lse = run_fwd(w, inp)
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                                  w.bias_strides)
    torch.cuda.synchronize()
    res = {"out": check("out", host(out), o_ref, w.dtype), "lse": check_lse(host(lse), l_ref, w.dtype)}
    if backward if backward is not None else w.dout is not None:
        dq, dk, dv = run_bwd(w, out, lse, inp, grad_dtype)
        g_ref = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                                w.bias_strides)
        torch.cuda.synchronize()
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), g_ref):
            res[name] = check(name, host(got), ref, w.dtype, grad=True,
                              abs_tol=grad_abs_tol(w.dtype, ref, named_workload))
    return res
