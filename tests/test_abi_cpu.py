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
HEADERS = [os.path.join(ROOT, "include", h) for h in sorted(os.listdir(os.path.join(ROOT, "include")))
           if h.endswith(".h")]

OK, INVALID, UNSUPPORTED, WORKSPACE, HIP = range(5)
F32, BF16, F16 = 0, 1, 2
P = 0x1000  # a non-NULL pointer that validation rejects before any use


def _declared():
    names = set()
    for h in HEADERS:
        src = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(va_[a-z0-9_]+)\s*\(", src))
    return sorted(names)


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
             bstr=None, rs=None, out=P, lse=P, ws=0x100000, wsb=1 << 30, batch=2, tq=16, tk=16, hq=4,
             hkv=2, d=64, dt=BF16)
    a.update(kw)
    bstr = _lib.strides_arg(a["bstr"]) if a["bstr"] is not None else None
    rs = _lib.strides_arg(a["rs"]) if a["rs"] is not None else None
    return lib.va_varlen_fwd(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["mq"], a["mk"], a["scale"],
                             a["causal"], a["bias"], bstr, a["out"], a["lse"], rs, a["ws"], a["wsb"],
                             a["batch"], a["tq"], a["tk"], a["hq"], a["hkv"], a["d"], a["dt"], None)


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
    (dict(ws=None), INVALID),
    (dict(ws=0x100040), INVALID),      # misaligned workspace
    (dict(d=80), UNSUPPORTED),
    (dict(d=512), UNSUPPORTED),
    (dict(d=16), UNSUPPORTED),
    (dict(dt=7), UNSUPPORTED),
    (dict(dt=3), UNSUPPORTED),
    (dict(wsb=16), WORKSPACE),
    # token strides of q, k, v
    (dict(rs=(255, 128, 128)), INVALID),       # q rows overlap (below Hq * d = 256)
    (dict(rs=(256, 128, 100)), INVALID),
    (dict(rs=(260, 128, 128)), INVALID),       # 520-byte rows: not 16-byte aligned
    (dict(rs=(258, 128, 128), dt=F32), INVALID),  # float32: 1032-byte rows
    (dict(k=P + 8), INVALID),                  # misaligned base
    (dict(rs=(1 << 28, 128, 128), mq=8), UNSUPPORTED),  # 8 rows of 2^29 bytes: past 32-bit offsets
])
def test_fwd_validation(lib, kw, code):
    assert _fwd(lib, **kw) == code
    assert lib.va_last_error()


def _fwd_bwdplan(lib, bws, bwsb, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, mq=8, mk=8, scale=0.125, causal=1, bias=None,
             bstr=None, rs=None, out=P, lse=P, ws=0x100000, wsb=1 << 30, batch=2, tq=16, tk=16, hq=4,
             hkv=2, d=64, dt=BF16)
    a.update(kw)
    return lib.va_varlen_fwd_bwdplan(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["mq"], a["mk"],
                                     a["scale"], a["causal"], None, None, a["out"], a["lse"], None,
                                     a["ws"], a["wsb"], bws, bwsb, a["batch"], a["tq"], a["tk"], a["hq"],
                                     a["hkv"], a["d"], a["dt"], None)


@pytest.mark.parametrize("bws,bwsb,kw,code", [
    (None, 1 << 30, {}, INVALID),             # no backward workspace
    (0x200040, 1 << 30, {}, INVALID),         # misaligned
    (0x200000, 16, {}, WORKSPACE),            # too small for the backward's sizes
    (0x200000, 1 << 30, dict(q=None), INVALID),  # the forward's own checks still apply
    (0x200000, 1 << 30, dict(d=80), UNSUPPORTED),
])
def test_fwd_bwdplan_validation(lib, bws, bwsb, kw, code):
    assert _fwd_bwdplan(lib, bws, bwsb, **kw) == code
    assert lib.va_last_error()


def test_bwd_planned_validation(lib):
    """The planned backward runs the backward's argument checks."""
    args = [P, P, P, P, P, P, P, P, 8, 8, 0.125, 1, None, None, P, P, P, None, None, None,
            0x100000, 16, 2, 16, 16, 4, 2, 64, BF16, F32, None]
    assert lib.va_varlen_bwd_planned(*args) == WORKSPACE
    args[20] = None
    assert lib.va_varlen_bwd_planned(*args) == INVALID


def _bwd(lib, **kw):
    a = dict(do=P, q=P, k=P, v=P, o=P, lse=P, cq=P, ck=P, mq=8, mk=8, scale=0.125, causal=1,
             bias=None, bstr=None, rs=None, dq=P, dk=P, dv=P, db=None, dbstr=None, ws=0x100000,
             wsb=1 << 30, batch=2, tq=16, tk=16, hq=4, hkv=2, d=64, dt=BF16, gdt=F32)
    a.update(kw)
    bstr = _lib.strides_arg(a["bstr"]) if a["bstr"] is not None else None
    dbstr = _lib.strides_arg(a["dbstr"]) if a["dbstr"] is not None else None
    rs = _lib.strides_arg(a["rs"]) if a["rs"] is not None else None
    return lib.va_varlen_bwd(a["do"], a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                             a["mq"], a["mk"], a["scale"], a["causal"], a["bias"], bstr, a["dq"],
                             a["dk"], a["dv"], a["db"], dbstr, rs, a["ws"], a["wsb"], a["batch"], a["tq"],
                             a["tk"], a["hq"], a["hkv"], a["d"], a["dt"], a["gdt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(do=None), INVALID),
    (dict(ws=None), INVALID),
    (dict(ws=0x100010), INVALID),      # misaligned workspace
    (dict(tq=0), INVALID),
    (dict(hq=3, hkv=2), INVALID),
    (dict(d=48), UNSUPPORTED),
    (dict(dt=F32, gdt=BF16), UNSUPPORTED),
    (dict(dt=BF16, gdt=F16), UNSUPPORTED),     # 16-bit gradients only in the input's format
    (dict(dt=F16, gdt=BF16), UNSUPPORTED),
    (dict(gdt=5), UNSUPPORTED),
    (dict(wsb=16), WORKSPACE),
    (dict(rs=(256, 64, 128)), INVALID),        # k rows overlap (below Hkv * d = 128)
    (dict(v=P + 4), INVALID),
    # bias gradient
    (dict(db=P), INVALID),                                              # no dbias_stride
    (dict(db=P, dbstr=(64, 16, 4, 1)), INVALID),                        # no bias
    (dict(bias=P, bstr=(64, 16, 4, 1), db=P, dbstr=(64, 16, -4, 1)), INVALID),
    (dict(bias=P, bstr=(64, 16, 4, 1), db=P, dbstr=(0, 16, 4, 1)), UNSUPPORTED),   # summed over sequences
    (dict(bias=P, bstr=(64, 16, 4, 1), db=P, dbstr=(64, 16, 4, 0)), UNSUPPORTED),  # summed over keys
    (dict(bias=P, bstr=(64, 16, 4, 1), db=P, dbstr=(64, 0, 4, 1)), UNSUPPORTED),   # per pair, summed over heads
    (dict(bias=P, bstr=(16, 4, 0, 1), db=P, dbstr=(16, 0, 0, 1)), UNSUPPORTED),    # per key over heads, 2 KV heads
    (dict(bias=P, bstr=(16, 4, 0, 1), db=P, dbstr=(16, 4, 0, 1), hq=66, hkv=2), UNSUPPORTED),  # 33 heads per KV head
    (dict(bias=P, bstr=(16, 4, 0, 1), db=P, dbstr=(16, 4, 0, 1), hq=18, hkv=2, d=256), UNSUPPORTED),  # 9 at d = 256
])
def test_bwd_validation(lib, kw, code):
    assert _bwd(lib, **kw) == code


def _r(x):
    return (x + 255) // 256 * 256


def _plan_bytes(units, splits, heads):
    """Header, units and bounds (16 bytes per unit), slot and split index (4 each),
    split list (16 per split) and per (split, head) counts of chunks left (4 each)."""
    return 256 + 2 * _r(16 * units) + 2 * _r(4 * units) + _r(16 * max(splits, 1)) + \
        _r(4 * max(splits, 1) * heads)


def test_fwd_workspace_size(lib):
    f = lib.va_varlen_fwd_workspace_size
    assert f(0, 16, 16, 8, 8, 4, 2, 64, BF16) == 0
    assert f(2, 16, 16, 0, 8, 4, 2, 64, BF16) == 0
    assert f(2, 16, 16, 8, 8, 4, 3, 64, BF16) == 0
    assert f(2, 16, 16, 8, 8, 4, 2, 80, BF16) == 0
    assert f(2, 16, 16, 8, 8, 4, 2, 96, BF16) > 0 and f(2, 16, 16, 8, 8, 4, 2, 32, F32) > 0
    # no tile sees more than 2048 keys: only the plan (<= total/128 + batch units)
    assert f(2, 16, 16, 8, 8, 4, 2, 64, BF16) == _plan_bytes(2, 0, 4)
    assert f(20, 10459, 10459, 1024, 1024, 14, 2, 64, BF16) == _plan_bytes(10459 // 128 + 20, 0, 14)
    assert f(16, 9687, 9687, 2048, 2048, 14, 2, 64, BF16) == _plan_bytes(9687 // 128 + 16, 0, 14)
    # longer keys (up to 4096: 64 steps, two 2048-key chunks): partial slots of
    # hq * 128 rows * (d + 1) floats, two per tile at most
    tiles = 9687 // 128 + 16
    slot = 14 * 128 * 65 * 4
    slots = min(2 * tiles, (64 << 20) // slot)
    assert f(16, 9687, 9687, 4096, 4096, 14, 2, 64, BF16) == \
        _plan_bytes(tiles + slots, slots // 2, 14) + _r(slots * slot)
    assert f(16, 9687, 9687, 4096, 4096, 14, 2, 64, F16) == f(16, 9687, 9687, 4096, 4096, 14, 2, 64, BF16)
    # float32 steps are 32 keys, so the same 2048-key chunk is 64 steps
    assert f(2, 16, 16, 2048, 2048, 4, 2, 64, F32) == _plan_bytes(2, 0, 4)


def test_bwd_workspace_size(lib):
    f = lib.va_varlen_bwd_workspace_size
    assert f(0, 16, 16, 8, 8, 4, 2, 64, BF16, F32) == 0
    assert f(2, 16, 16, 8, 8, 4, 3, 64, BF16, F32) == 0
    assert f(2, 16, 16, 8, 8, 4, 2, 80, BF16, F32) == 0
    assert f(2, 16, 16, 8, 8, 4, 2, 96, BF16, F32) > 0
    assert f(2, 16, 16, 8, 8, 4, 2, 64, F32, BF16) == 0
    assert f(2, 16, 16, 8, 8, 4, 2, 64, BF16, F16) == 0
    # float16 plans exactly as bf16 (same 64-key steps, same unit sizes)
    assert f(2, 16, 16, 416, 8, 4, 2, 64, F16, F16) == f(2, 16, 16, 416, 8, 4, 2, 64, BF16, BF16)
    # short sequences: D = rowsum(dO * O) and the two plans (dK/dV and dQ)
    n = f(2, 16, 16, 8, 8, 4, 4, 64, BF16, F32)
    # dK/dV plan (its split tiles are merged by the dQ pass: no counts) + dQ plan
    assert n == _r(4 * 16 * 4) + _plan_bytes(2, 0, 0) + _plan_bytes(2, 0, 4)  # no partial slots (per-key bias sums: none)
    # GQA 4/2: a dK/dV unit holds at most 1536 (query row, head) pairs = 24 blocks of 32
    assert f(2, 16, 16, 768, 8, 4, 2, 64, BF16, F32) == n
    big = f(2, 16, 16, 800, 8, 4, 2, 64, BF16, F32)
    slots_k = 2 * 2  # two tiles, ceil(25 / 24) = 2 chunks each
    assert big == _r(4 * 16 * 4) + _plan_bytes(2 + slots_k, slots_k // 2, 0) + _plan_bytes(2, 0, 4) + \
        _r(slots_k * 2 * 2 * 128 * 64 * 4) + _r(slots_k * 4 * 128 * 4)  # + per-key bias sums per slot


def test_python_layer_rejects_cpu_tensors_and_bias_grad():
    import torch
    import variable_length_packed_amd as va
    q = torch.zeros(4, 2, 64)
    cu = torch.tensor([0, 4], dtype=torch.int32)
    with pytest.raises(ValueError):
        va.va_varlen_fwd(q, q, q, cu, cu, 4, 4)
    b = torch.zeros(1, 2, 4, 4, requires_grad=True)
    with pytest.raises(ValueError):  # a bias through an explicit strided view cannot require grad
        va.varlen_attn(q, q, q, cu, cu, 4, 4, bias=b, bias_stride=(32, 16, 4, 1))


# ---------------------------------------------------------------- packing (include/va_pack.h)
def _tensors(n=1, rb=128, padded=P, packed=P):
    arr = (_lib.PackTensor * max(n, 1))()
    for i in range(max(n, 1)):
        arr[i].padded = padded
        arr[i].packed = packed
        arr[i].row_bytes = rb
    return arr


@pytest.mark.parametrize("kw,code", [
    (dict(mask=None), INVALID),
    (dict(cu=None), INVALID),
    (dict(inv=None), INVALID),
    (dict(batch=0), INVALID),
    (dict(seqlen=-1), INVALID),
    (dict(batch=1 << 16, seqlen=1 << 15), INVALID),
])
def test_pack_metadata_validation(lib, kw, code):
    a = dict(mask=P, batch=4, seqlen=8, cu=P, mx=P, idx=P, pos=P, inv=P)
    a.update(kw)
    assert lib.va_pack_metadata(a["mask"], a["batch"], a["seqlen"], a["cu"], a["mx"], a["idx"], a["pos"],
                                a["inv"], None) == code
    assert lib.va_last_error()


@pytest.mark.parametrize("which", ["unpad", "pad"])
@pytest.mark.parametrize("kw,code", [
    (dict(n=0), INVALID),
    (dict(n=5), INVALID),
    (dict(tensors=None), INVALID),
    (dict(rb=0), INVALID),
    (dict(padded=0), INVALID),
    (dict(packed=0), INVALID),
    (dict(batch=0), INVALID),
    (dict(seqlen=0), INVALID),
    (dict(rows=-1), INVALID),
    (dict(index=None), INVALID),
])
def test_unpad_pad_validation(lib, which, kw, code):
    a = dict(n=2, rb=128, padded=P, packed=P, batch=4, seqlen=8, rows=32, index=P, tensors="x")
    a.update(kw)
    arr = None if a["tensors"] is None else _tensors(a["n"], a["rb"], a["padded"], a["packed"])
    if which == "unpad":
        r = lib.va_unpad(arr, a["n"], a["index"], P, a["batch"], a["seqlen"], a["rows"], None)
    else:
        r = lib.va_pad(arr, a["n"], a["index"], a["batch"], a["seqlen"], a["rows"], None)
    assert r == code
    assert lib.va_last_error()


# ---------------------------------------------------------------- decode steps (include/va_kvcache.h)
def _kv(lib, **kw):
    a = dict(q=P, kc=P, vc=P, cq=P, sk=P, bt=P, bts=8, ps=16, np_=64, mq=1, mk=128, scale=0.125, causal=1,
             out=P, lse=P, ws=0x100000, wsb=1 << 30, batch=2, tq=2, hq=8, hkv=2, d=128, dt=BF16)
    a.update(kw)
    return lib.va_kvcache_fwd(a["q"], a["kc"], a["vc"], a["cq"], a["sk"], a["bt"], a["bts"], a["ps"], a["np_"],
                              a["mq"], a["mk"], a["scale"], a["causal"], a["out"], a["lse"], a["ws"], a["wsb"],
                              a["batch"], a["tq"], a["hq"], a["hkv"], a["d"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), INVALID),
    (dict(bt=None), INVALID),
    (dict(sk=None), INVALID),
    (dict(lse=None), INVALID),
    (dict(batch=0), INVALID),
    (dict(tq=0), INVALID),
    (dict(hq=6, hkv=4), INVALID),
    (dict(mq=0), INVALID),
    (dict(mk=-1), INVALID),
    (dict(ps=0), INVALID),
    (dict(ps=24), INVALID),            # not a power of two
    (dict(ps=1 << 21), INVALID),
    (dict(np_=0), INVALID),
    (dict(bts=7), INVALID),            # 7 pages of 16 keys do not reach max_seqlen_k = 128
    (dict(causal=2), INVALID),
    (dict(scale=0.0), INVALID),
    (dict(kc=P + 8), INVALID),         # misaligned cache
    (dict(ws=None), INVALID),
    (dict(ws=P + 64), INVALID),        # misaligned workspace
    (dict(wsb=16), WORKSPACE),
    (dict(dt=7), UNSUPPORTED),
    (dict(d=80), UNSUPPORTED),
    (dict(mq=1 << 20, hq=64, hkv=8), UNSUPPORTED),  # a sequence's queries span 2^31 bytes
    (dict(mq=1 << 16, hq=64, hkv=8, dt=F32), UNSUPPORTED),  # 2^31 bytes in float32 (2^30 in bf16)
])
def test_kvcache_validation(lib, kw, code):
    assert _kv(lib, **kw) == code
    assert lib.va_last_error()


def test_kvcache_workspace_size(lib):
    f = lib.va_kvcache_fwd_workspace_size
    assert f(0, 1, 128, 8, 2, 128, BF16) == 0
    for d in (32, 64, 96, 128):
        assert f(2, 1, 128, 8, 2, d, BF16) > 0
    assert f(2, 1, 128, 8, 2, 80, BF16) == 0 and f(2, 1, 128, 8, 2, 256, BF16) == 0
    # float32 steps use the same work list and float32 partials: the same size
    assert f(2, 1, 128, 8, 2, 128, F32) == f(2, 1, 128, 8, 2, 128, BF16) > 0
    assert f(2, 1, 128, 8, 2, 128, 5) == 0             # not a dtype
    assert f(2, 1 << 16, 128, 64, 8, 128, BF16) > 0 and f(2, 1 << 16, 128, 64, 8, 128, F32) == 0
    assert f(2, 1, 128, 8, 3, 128, BF16) == 0

    def plan(entries, split=False):
        # planner header, a 32-byte entry per (sequence, row block, chunk), and the merge
        # list (an int per row block with several chunks: at most entries / 2)
        return 256 + _r(entries * 32) + _r(max(entries // 2 if split else 0, 1) * 4)
    # chunks of at least 256 keys: a cache that fits one chunk needs no partials
    assert f(2, 1, 256, 8, 2, 128, BF16) == plan(2)
    assert f(2, 1, 0, 8, 2, 128, F16) == plan(2)
    # 4 KV heads x 2 sequences = 8 row blocks of n_rep * max_q = 4 rows want 1024 chunks
    # each: 512 keys split into two of 256; a partial slot per (entry, KV head)
    slots = 2 * 2 * 4
    assert f(2, 1, 512, 16, 4, 128, BF16) == plan(2 * 2, True) + _r(slots * 4 * 128 * 4) + _r(slots * 4 * 4)
    # 12 new tokens x 4 heads per KV head = 48 rows: two row blocks of 32 rows per sequence
    slots = 2 * 2 * 2 * 4
    assert f(2, 12, 512, 16, 4, 64, F16) == plan(2 * 2 * 2, True) + _r(slots * 32 * 64 * 4) + _r(slots * 32 * 4)
    # a large batch keeps whole caches in one chunk when that already gives 8192 waves
    assert f(8192, 1, 4000, 8, 1, 128, BF16) == plan(8192)


def test_short_query_forward_workspace(lib):
    """Calls without a bias and with at most 32 (new token, head) rows per KV head take the
    decode kernels; the packed forward's workspace then also covers their work list,
    bounded by total_q (max_seqlen_q is only a hint there)."""
    f = lib.va_varlen_fwd_workspace_size
    # 256 sequences x 1 token, 32/8 heads (rows of 4), caches of up to 1024 keys: 2048 row
    # blocks want 4 chunks each -> chunks of 256 keys, 4 per row block; the work list holds
    # (256 * 4 / 4 + 256) * 4 entries, each with a partial slot per KV head
    cap = (256 * 4 // 4 + 256) * 4
    want = 256 + _r(cap * 32) + _r(cap // 2 * 4) + _r(cap * 8 * 4 * 128 * 4) + _r(cap * 8 * 4 * 4)
    assert f(256, 256, 256 * 1024, 1, 1024, 32, 8, 128, BF16) == want
    assert f(256, 256, 256 * 1024, 1, 1024, 32, 8, 128, F16) == want
    assert f(256, 256, 256 * 1024, 1, 1024, 32, 8, 128, F32) == want  # the float32 decode kernel
    # more than 32 tokens, or 17..32 tokens with more than 128 rows per KV head keep the
    # 128-row tiles' (much smaller) workspace
    assert f(256, 256 * 48, 256 * 1024, 48, 1024, 16, 16, 64, BF16) < want // 100
    assert f(256, 256 * 20, 256 * 1024, 20, 1024, 32, 4, 128, BF16) < want // 100
    # 16 tokens with 8 heads per KV head (128 rows) and 24 tokens with 4 (96 rows) do not
    assert f(256, 256 * 16, 256 * 1024, 16, 1024, 32, 4, 128, BF16) > want // 100
    assert f(256, 256 * 24, 256 * 1024, 24, 1024, 16, 4, 128, BF16) > want // 100


def _fwd_noalloc(lib, **kw):
    a = dict(q=P, k=P, v=P, cq=P, ck=P, mq=8, mk=8, scale=0.125, causal=1, bias=None,
             bstr=None, rs=None, out=P, lse=P, batch=2, tq=16, tk=16, hq=4, hkv=2, d=64, dt=BF16)
    a.update(kw)
    bstr = _lib.strides_arg(a["bstr"]) if a["bstr"] is not None else None
    rs = _lib.strides_arg(a["rs"]) if a["rs"] is not None else None
    return lib.va_varlen_fwd_noalloc(a["q"], a["k"], a["v"], a["cq"], a["ck"], a["mq"], a["mk"], a["scale"],
                                     a["causal"], a["bias"], bstr, a["out"], a["lse"], rs, a["batch"], a["tq"],
                                     a["tk"], a["hq"], a["hkv"], a["d"], a["dt"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), INVALID),
    (dict(tq=0), INVALID),
    (dict(hq=6, hkv=4), INVALID),
    (dict(mq=0), INVALID),
    (dict(d=80), UNSUPPORTED),
    (dict(dt=7), UNSUPPORTED),
    # a work plan larger than the library's scratch array (2^20 sequences)
    (dict(batch=1 << 20, tq=1 << 22, tk=1 << 22, mq=1 << 22, mk=1 << 22, hq=64, hkv=8), WORKSPACE),
])
def test_fwd_noalloc_validation(lib, kw, code):
    """The allocation-free forward checks sizes on the host before it looks up its scratch array."""
    assert _fwd_noalloc(lib, **kw) == code
    msg = lib.va_last_error()
    assert msg
    if code == WORKSPACE:
        assert b"allocation-free" in msg
