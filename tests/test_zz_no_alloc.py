"""GPU: the allocation-free forward (va_varlen_fwd_noalloc) against va_varlen_fwd.

Called through the C ABI (ctypes), twice in a row on one device -- a
config-3-shaped batch, then a smaller one -- so the second call runs on the
scratch array the first one left behind.  Each result must equal the
workspace entry point's bitwise (the same plan and split, as both fit their
budgets) and match the oracle within the bf16 bounds.  Sizes past the
array's capacity are refused with VA_ERR_WORKSPACE.
"""

import ctypes

import numpy as np
import pytest
import torch

import oracle
from variable_length_packed_amd import _lib
from workloads import config, make_case

from . import _gpu

pytestmark = pytest.mark.gpu


def _noalloc(lib, w, inp, out, lse):
    st = torch.cuda.current_stream().cuda_stream
    return lib.va_varlen_fwd_noalloc(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                                     inp["cu_q"].data_ptr(), inp["cu_k"].data_ptr(), w.max_q, w.max_k,
                                     w.scale, int(w.causal), None, None, out.data_ptr(), lse.data_ptr(), None,
                                     w.batch, w.total_q, w.total_k, w.hq, w.hkv, w.d, _lib.VA_BF16, st)


def test_noalloc_forward_equals_workspace_forward():
    lib = _lib.load()
    cases = [("config 3 lengths", config(3, with_dout=False)),
             ("smaller batch", make_case(91, [300, 5, 1100, 64], hq=14, hkv=2, d=64, causal=True, dtype="bf16"))]
    for name, w in cases:
        print(f"[case] noalloc {name}: {w.describe() if hasattr(w, 'describe') else ''}", flush=True)
        inp = _gpu.device_inputs(w)
        o_ref, l_ref = _gpu.run_fwd(w, inp)
        out = torch.full_like(o_ref, float("nan"))
        lse = torch.full_like(l_ref, float("nan"))
        rc = _noalloc(lib, w, inp, out, lse)
        assert rc == _lib.VA_OK, lib.va_last_error()
        torch.cuda.synchronize()
        assert torch.equal(out, o_ref), name
        assert torch.equal(lse, l_ref), name
        o_or, l_or = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, w.causal)
        _gpu.check("out", _gpu.host(out), o_or, "bf16")
        _gpu.check_lse(_gpu.host(lse), l_or, "bf16")


def test_noalloc_refuses_sizes_past_its_scratch():
    lib = _lib.load()
    w = make_case(92, [64], hq=2, hkv=2, d=64, causal=True, dtype="bf16")
    inp = _gpu.device_inputs(w)
    out = torch.empty_like(inp["q"])
    lse = torch.empty((w.hq, w.total_q), dtype=torch.float32, device=_gpu.DEV)
    st = torch.cuda.current_stream().cuda_stream
    # a batch whose work plan alone outgrows the array (hints only size the plan)
    big = 1 << 22
    rc = lib.va_varlen_fwd_noalloc(inp["q"].data_ptr(), inp["k"].data_ptr(), inp["v"].data_ptr(),
                                   inp["cu_q"].data_ptr(), inp["cu_k"].data_ptr(), big, big, w.scale, 1, None,
                                   None, out.data_ptr(), lse.data_ptr(), None, 1 << 20, big, big, 64, 8, 64,
                                   _lib.VA_BF16, st)
    assert rc == _lib.VA_ERR_WORKSPACE
    assert b"allocation-free" in lib.va_last_error()
