"""GPU parity of the packing steps (include/va_pack.h) with the oracle: bit-exact.

Packing metadata of seeded padding masks (right-, left- and interior-padded,
empty and full rows, sizes that are not multiples of a workgroup), the unpad
gather and the pad scatter of bf16 and float32 Q/K/V (rows of different sizes
in one call, every copy width the library picks), and unpad -> varlen
attention -> pad against the oracle's attention on the padded batch.
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_amd as va
from workloads import make_case, padding_mask

from . import _gpu

pytestmark = pytest.mark.gpu

DEV = _gpu.DEV

MASKS = [
    ("right-16x2048", 11, 16, 2048, "right"),
    ("left-7x300", 12, 7, 300, "left"),
    ("interior-5x1000", 13, 5, 1000, "random"),
    ("one-row-1x1", 14, 1, 1, "right"),
    ("tall-4099x3", 15, 4099, 3, "random"),
]


def _mask(seed, b, s, kind):
    return padding_mask(seed, b, s, kind)


def _meta(m):
    cu, mx, idx, pos, inv = va.pack_metadata(torch.from_numpy(m).to(DEV))
    torch.cuda.synchronize()
    return [t.cpu().numpy() for t in (cu, mx, idx, pos, inv)]


@pytest.mark.parametrize("name,seed,b,s,kind", MASKS, ids=[m[0] for m in MASKS])
def test_metadata_bit_exact(name, seed, b, s, kind):
    print(f"[case] metadata {name}", flush=True)
    m = _mask(seed, b, s, kind)
    cu, mx, idx, pos, inv = _meta(m)
    rcu, rmx, ridx, rpos, rinv = oracle.pack_metadata(m)
    total = int(rcu[-1])
    assert np.array_equal(cu, rcu)
    assert int(mx[0]) == rmx
    assert np.array_equal(idx[:total], ridx)
    assert np.array_equal(pos[:total], rpos)
    assert np.array_equal(inv, rinv)


@pytest.mark.parametrize("special", ["all-padding", "no-padding", "nonzero-values"])
def test_metadata_special_masks(special):
    print(f"[case] metadata {special}", flush=True)
    if special == "all-padding":
        m = np.zeros((9, 70), dtype=np.uint8)
    elif special == "no-padding":
        m = np.ones((3, 513), dtype=np.uint8)
    else:
        m = _mask(21, 6, 129, "random") * np.uint8(7)
    cu, mx, idx, pos, inv = _meta(m)
    rcu, rmx, ridx, rpos, rinv = oracle.pack_metadata(m)
    total = int(rcu[-1])
    assert np.array_equal(cu, rcu) and int(mx[0]) == rmx
    assert np.array_equal(idx[:total], ridx) and np.array_equal(pos[:total], rpos)
    assert np.array_equal(inv, rinv)


def _qkv(seed, b, s, shapes, dtype):
    rng = np.random.default_rng(seed)
    return [torch.from_numpy(rng.standard_normal((b, s) + sh).astype(np.float32)).to(DEV).to(dtype)
            for sh in shapes]


# (row shapes of up to four tensors, dtype): 16-byte rows, 8-byte, 4-byte, 2-byte, 1-byte widths
ROWS = [
    ("qkv-bf16-14x64-2x64", [(14, 64), (2, 64), (2, 64)], torch.bfloat16),
    ("qkv-f32-8x64", [(8, 64), (8, 64), (8, 64), (8, 64)], torch.float32),
    ("bf16-rows-of-4", [(4,)], torch.bfloat16),
    ("f32-rows-of-3", [(3,), (1,)], torch.float32),
    ("bf16-rows-of-3", [(3,)], torch.bfloat16),
    ("u8-rows-of-5", [(5,)], torch.uint8),
]


@pytest.mark.parametrize("mi", [0, 1, 2, 4])
@pytest.mark.parametrize("rname,shapes,dtype", ROWS, ids=[r[0] for r in ROWS])
def test_unpad_pad_bit_exact(mi, rname, shapes, dtype):
    name, seed, b, s, kind = MASKS[mi]
    print(f"[case] unpad/pad {name} {rname}", flush=True)
    m = _mask(seed, b, s, kind)
    dm = torch.from_numpy(m).to(DEV)
    cu, _, idx, _, inv = va.pack_metadata(dm)
    if dtype == torch.uint8:
        rng = np.random.default_rng(seed)
        xs = [torch.from_numpy(rng.integers(0, 256, (b, s) + sh, dtype=np.uint8)).to(DEV) for sh in shapes]
    else:
        xs = _qkv(seed, b, s, shapes, dtype)
    total = int(m.astype(bool).sum())
    packed = va.unpad(xs, idx, cu, packed_rows=total)
    back = va.pad(packed, inv, b, s)
    torch.cuda.synchronize()
    _, _, ridx, _, rinv = oracle.pack_metadata(m)
    for x, y, z in zip(xs, packed, back):
        xh = x.cpu().view(torch.uint8 if x.element_size() == 1 else (torch.int16 if x.element_size() == 2 else torch.int32)).numpy()
        yh = y.cpu().view(torch.uint8 if y.element_size() == 1 else (torch.int16 if y.element_size() == 2 else torch.int32)).numpy()
        zh = z.cpu().view(torch.uint8 if z.element_size() == 1 else (torch.int16 if z.element_size() == 2 else torch.int32)).numpy()
        assert np.array_equal(yh, oracle.unpad(xh, ridx))            # bitwise
        assert np.array_equal(zh, oracle.pad(yh, rinv, b, s))
        # the padding positions are exactly zero
        assert not zh.reshape(b * s, -1)[m.reshape(-1) == 0].any()


def test_unpad_leaves_rows_past_the_total_alone():
    print("[case] unpad capacity", flush=True)
    m = _mask(31, 8, 40, "right")
    dm = torch.from_numpy(m).to(DEV)
    cu, _, idx, _, _ = va.pack_metadata(dm)
    x = _qkv(31, 8, 40, [(2, 8)], torch.float32)[0]
    packed = va.unpad([x], idx, cu)[0]          # capacity batch * seqlen
    packed2 = torch.full_like(packed, 7.0)
    lib = va.api._lib.load()
    arr = va.api._pack_tensors([x], [packed2], 8, 40)
    assert lib.va_unpad(arr, 1, idx.data_ptr(), cu.data_ptr(), 8, 40, packed2.shape[0],
                        va.api._stream(DEV)) == 0
    torch.cuda.synchronize()
    total = int(m.sum())
    assert torch.equal(packed2[:total], packed[:total])
    assert bool((packed2[total:] == 7.0).all())


@pytest.mark.parametrize("kind,dtype,causal", [("right", "bf16", True), ("left", "f32", False),
                                               ("random", "bf16", False)])
def test_unpad_attention_pad_matches_oracle(kind, dtype, causal):
    """Padded Q/K/V -> unpad -> va_varlen_fwd -> pad equals the oracle's attention per real row."""
    print(f"[case] unpad-attention-pad {kind} {dtype} causal={causal}", flush=True)
    b, s, hq, hkv, d = 6, 300, 14, 2, 64
    m = padding_mask(41, b, s, kind, lengths=[300, 1, 0, 129, 64, 257] if kind != "random" else None)
    lens = [int(x) for x in m.sum(axis=1)]
    # the packed oracle case with these row lengths, laid into padded buffers at the mask's positions
    w = make_case(42, lens, hq=hq, hkv=hkv, d=d, causal=causal, dtype=dtype)
    dt = _gpu.tdtype(w)
    _, _, ridx, _, rinv = oracle.pack_metadata(m)
    pq, pk, pv = (oracle.pad(getattr(w, n), rinv, b, s) for n in "qkv")
    dm = torch.from_numpy(m).to(DEV)
    cu, mx, idx, _, inv = va.pack_metadata(dm)
    total = int(sum(lens))
    q, k, v = va.unpad([_gpu.to_dev(pq, dt), _gpu.to_dev(pk, dt), _gpu.to_dev(pv, dt)], idx, cu, packed_rows=total)
    out, lse = va.va_varlen_fwd(q, k, v, cu, cu, s, s, w.scale, causal)
    o_pad = va.pad([out], inv, b, s)[0]
    torch.cuda.synchronize()
    ref_out, _ = oracle.forward(w.q, w.k, w.v, w.cu_q, w.cu_k, w.scale, causal)
    ref_pad = oracle.pad(ref_out, rinv, b, s)
    err = np.max(np.abs(_gpu.host(o_pad) - ref_pad))
    tol = _gpu.TOL[dtype]["abs"]
    assert err <= tol, err
    assert not _gpu.host(o_pad).reshape(b * s, -1)[m.reshape(-1) == 0].any()
