"""GPU parity on the five named workloads at full size, in the launch shape bench.py times.

Every workload is compared with the full oracle, element by element: every
sequence, every head, every output tensor (O, LSE and, where the workload has a
backward, dQ, dK and dV).  Tolerances: float32 max-abs <= 1e-5 on O and LSE;
bf16 max-abs <= 2e-2 and relative L2 <= 5e-3 on every tensor, gradients stored
float32.  Each check prints its max-abs, rel-L2 and the worst sequence.
"""

import numpy as np
import pytest
import torch

import oracle
from workloads import config

from . import _gpu

pytestmark = pytest.mark.gpu


def _worst_sequence(got, ref, cu, axis0=True):
    """Index of the sequence holding the largest absolute difference (rows on axis 0,
    or on the last axis for LSE)."""
    diff = np.abs(np.asarray(got, dtype=np.float64) - ref)
    diff = np.where(np.isfinite(diff), diff, 0.0)
    per_row = diff.reshape(diff.shape[0], -1).max(axis=1) if axis0 else diff.max(axis=0)
    row = int(np.argmax(per_row))
    return int(np.searchsorted(cu, row, side="right") - 1)


def _check_fwd_full(w, out, lse):
    o_ref, l_ref = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                                  w.bias_strides)
    o, l = _gpu.host(out), _gpu.host(lse)
    print(f"    worst sequence: out {_worst_sequence(o, o_ref, w.cu_q)}, "
          f"lse {_worst_sequence(l, l_ref, w.cu_q, axis0=False)}", flush=True)
    _gpu.check("out", o, o_ref, w.dtype)
    _gpu.check_lse(l, l_ref, w.dtype)


def _check_bwd_full(w, grads):
    refs = oracle.backward(w.dout, w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal, w.bias,
                           w.bias_strides)
    for name, g, ref, cu in zip(("dq", "dk", "dv"), grads, refs, (w.cu_q, w.cu_k, w.cu_k)):
        got = _gpu.host(g)
        print(f"    worst sequence: {name} {_worst_sequence(got, ref, cu)}", flush=True)
        _gpu.check(name, got, ref, w.dtype, grad=True)


def test_config1_tiny_fp32_full():
    w = config(1)
    print(f"[config 1] {w.describe()}", flush=True)
    _gpu.full_parity(w, backward=False, named_workload=True)


def test_config2_qwen_shaped_bf16_fwd():
    w = config(2)
    print(f"[config 2] {w.describe()}", flush=True)
    out, lse = _gpu.run_fwd(w)
    torch.cuda.synchronize()
    _check_fwd_full(w, out, lse)


def test_config3_long_rows_bf16_fwd_bwd():
    w = config(3)
    print(f"[config 3] {w.describe()}", flush=True)
    inp = _gpu.device_inputs(w)
    out, lse = _gpu.run_fwd(w, inp)
    grads = _gpu.run_bwd(w, out, lse, inp)
    torch.cuda.synchronize()
    _check_fwd_full(w, out, lse)
    _check_bwd_full(w, grads)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("bias", ["none", "per_key", "per_pair"])
def test_config4_graph_encoder(dtype, bias):
    w = config(4, dtype=dtype, bias=bias)
    print(f"[config 4] {w.describe()}", flush=True)
    out, lse = _gpu.run_fwd(w)
    torch.cuda.synchronize()
    _check_fwd_full(w, out, lse)


def test_config5_short_gqa_cross_length_full():
    w = config(5)
    print(f"[config 5] {w.describe()}", flush=True)
    _gpu.full_parity(w, named_workload=True)
