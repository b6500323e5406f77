"""C ABI on the CPU: the library loads, exports every declared symbol, and its
host-side validation returns the documented status codes (no kernel launch:
every call here is rejected before any device work)."""

import ctypes
import os
import re
import subprocess

import pytest

from variable_length_packed_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "va_varlen.h")

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
F32, BF16 = 0, 1
P = 0x1000  # a non-NULL pointer that validation rejects before any use


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(va_[a-z0-9_]+)\s*\(", src)))


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def test_header_and_binding_agree():
    assert sorted(_lib.EXPORTS) == _declared()


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.LIB_PATH], capture_output=True,
                         text=True, check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if line.strip()}
    for name in _declared():
        assert name in exported, name
        assert hasattr(lib, name)


def test_library_has_gfx950_code():
    # the device code bundle of our own build names its target
    data = open(_lib.LIB_PATH, "rb").read()
    assert b"gfx950" in data


def test_status_strings_and_version(lib):
    for s in range(5):
        assert lib.va_status_string(s)
    assert lib.va_status_string(99) == b"unknown status"
    assert lib.va_version() >= 10000


def _fwd(lib, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, mq=8, mk=8, scale=0.125, causal=1, bias=None,
             bstr=None, out=P, lse=P, batch=2, tq=16, tk=16, hq=4, hkv=2, d=64, dt=BF16)
    a.update(kw)
    bstr = _lib.strides_arg(a["bstr"]) if a["bstr"] is not None else None
    return lib.va_varlen_fwd(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["mq"], a["mk"], a["scale"],
                             a["causal"], a["bias"], bstr, a["out"], a["lse"], a["batch"], a["tq"],
                             a["tk"], a["hq"], a["hkv"], a["d"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(lse=None), INVALID),
    (dict(cq=None), INVALID),
    (dict(batch=0), INVALID),          # zero-sized dimension
    (dict(tq=0), INVALID),
    (dict(tk=0), INVALID),
    (dict(hq=0), INVALID),
    (dict(d=0), INVALID),
    (dict(hq=6, hkv=4), INVALID),      # Hq % Hkv != 0
    (dict(mq=0), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(scale=-1.0), INVALID),
    (dict(scale=float("nan")), INVALID),
    (dict(causal=2), INVALID),
    (dict(bias=P), INVALID),           # bias without strides
    (dict(bstr=(1, 1, 1, 1)), INVALID),  # strides without bias
    (dict(bias=P, bstr=(1, -1, 1, 1)), INVALID),
    (dict(d=96), UNSUPPORTED),
    (dict(d=256), UNSUPPORTED),
    (dict(dt=7), UNSUPPORTED),
])
def test_fwd_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert lib.va_last_error()


def _bwd(lib, **kw):
    a = dict(do=P, q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, mq=8, mk=8, scale=0.125, causal=1,
             bias=None, bstr=None, dq=P, dk=P, dv=P, ws=0x100000, wsb=1 << 30, batch=2, tq=16,
             tk=16, hq=4, hkv=2, d=64, dt=BF16, gdt=F32)
    a.update(kw)
    bstr = _lib.strides_arg(a["bstr"]) if a["bstr"] is not None else None
    return lib.va_varlen_bwd(a["do"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                             a["mq"], a["mk"], a["scale"], a["causal"], a["bias"], bstr, a["dq"],
                             a["dk"], a["dv"], a["ws"], a["wsb"], a["batch"], a["tq"], a["tk"],
                             a["hq"], a["hkv"], a["d"], a["dt"], a["gdt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws=0x100010), INVALID),      # misaligned workspace
    (dict(tq=0), INVALID),
    (dict(hq=3, hkv=2), INVALID),
    (dict(d=32), UNSUPPORTED),
    (dict(dt=F32, gdt=BF16), UNSUPPORTED),
    (dict(gdt=5), UNSUPPORTED),
    (dict(wsb=16), WORKSPACE),
])
def test_bwd_validation(lib, kw, code):
    assert _bwd(lib, **kw) == code


def test_workspace_size(lib):
    f = lib.va_varlen_bwd_workspace_size
    assert f(0, 16, 16, 4, 2, 64, BF16, F32) == 0
    assert f(2, 16, 16, 4, 3, 64, BF16, F32) == 0
    assert f(2, 16, 16, 4, 2, 96, BF16, F32) == 0
    assert f(2, 16, 16, 4, 2, 64, F32, BF16) == 0
    n = f(2, 16, 16, 4, 4, 64, BF16, F32)  # no GQA: only D = rowsum(dO * O)
    assert n == 256  # 4 heads * 16 rows * 4 bytes, rounded up to 256
    g = f(2, 16, 16, 4, 2, 64, BF16, F32)  # GQA on a small problem: per-head partial dK/dV
    assert g == 256 + 2 * 2 * 16 * 2 * 64 * 4


def test_python_layer_rejects_cpu_tensors_and_bias_grad():
    import torch
    import variable_length_packed_amd as va
    q = torch.zeros(4, 2, 64)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        va.va_varlen_fwd(q, q, q, cu, cu, 4, 4)
    b = torch.zeros(1, 2, 4, 4, requires_grad=True)
    with pytest.raises(ValueError):
        va.varlen_attn(q, q, q, cu, cu, 4, 4, bias=b)
