"""GPU parity of decode steps against a paged KV cache (include/va_kvcache.h) with the oracle.

Single-token steps and multi-token steps (beams, drafts), causal and not,
GQA, MQA and MHA, head_dim 32, 64, 96 and 128, bf16, float16 and float32, pages of 1 to 256
keys handed out in random order, empty caches, sequences with no new token,
caches shorter than the new tokens (rows that see no key), caches long enough
to split into tens of chunks, and the full decode workload the bench times
(sampled sequences against the oracle).  Unused cache slots hold NaN and
unused block-table entries -1, so a read of either shows.  Tolerances as for
the packed forward (``tests/_gpu.py``).
"""

import numpy as np
import pytest
import torch

import oracle
import variable_length_packed_amd as va
from workloads.kvcache import DECODE_SHAPE, decode_device_inputs, kvcache_case

from . import _gpu

pytestmark = pytest.mark.gpu

DEV = _gpu.DEV
_DT = {"bf16": torch.bfloat16, "f16": torch.float16, "f32": torch.float32}

CASES = [
    ("decode-gqa4-d128-p16", dict(seed=1, lens_q=[1] * 6, lens_k=[1, 17, 300, 1000, 4000, 0], hq=32, hkv=8,
                                  d=128, dtype="bf16", page_size=16)),
    ("decode-mqa-d64-f16-p1", dict(seed=2, lens_q=[1, 1, 1], lens_k=[5, 33, 700], hq=8, hkv=1, d=64,
                                   dtype="f16", page_size=1)),
    ("draft4-gqa8-d128-p64", dict(seed=3, lens_q=[4, 4, 4, 4], lens_k=[4, 100, 2000, 3], hq=16, hkv=2, d=128,
                                  dtype="bf16", page_size=64)),
    ("beam12-noncausal-d64-p32", dict(seed=4, lens_q=[12, 12, 7], lens_k=[300, 64, 1025], hq=8, hkv=2, d=64,
                                      dtype="bf16", page_size=32, causal=False)),
    ("mixed-q-mha-d64-p256", dict(seed=5, lens_q=[1, 5, 0, 3], lens_k=[600, 9, 50, 3], hq=4, hkv=4, d=64,
                                  dtype="f16", page_size=256)),
    ("long-split-d128", dict(seed=6, lens_q=[1, 2], lens_k=[8000, 12000], hq=8, hkv=2, d=128, dtype="bf16",
                             page_size=16)),
    ("long-split-d64-causal-draft", dict(seed=7, lens_q=[6, 1, 3], lens_k=[5000, 2, 9001], hq=12, hkv=3, d=64,
                                         dtype="f16", page_size=128)),
    # head_dim 32: 64-key steps, so pages of 64 take one lookup per step and pages of 8 one per load
    ("decode-gqa4-d32-p64", dict(seed=13, lens_q=[1] * 5, lens_k=[1, 63, 64, 3000, 0], hq=16, hkv=4, d=32,
                                 dtype="bf16", page_size=64)),
    ("draft3-mqa-d32-f16-p8-split", dict(seed=14, lens_q=[3, 1, 2], lens_k=[9000, 5, 700], hq=8, hkv=1, d=32,
                                         dtype="f16", page_size=8)),
    ("beam6-noncausal-d32-p16", dict(seed=15, lens_q=[6, 6], lens_k=[129, 2000], hq=4, hkv=2, d=32,
                                     dtype="bf16", page_size=16, causal=False)),
    # head_dim 96: 12 pieces per cache row, so some wave loads straddle two rows (and,
    # with pages of 4 keys, two pages); 32-key steps
    ("decode-gqa4-d96-p4", dict(seed=16, lens_q=[1] * 4, lens_k=[31, 32, 33, 2500], hq=16, hkv=4, d=96,
                                dtype="bf16", page_size=4)),
    ("draft2-mqa-d96-f16-p32-split", dict(seed=17, lens_q=[2, 2, 1], lens_k=[7000, 1, 300], hq=8, hkv=1, d=96,
                                          dtype="f16", page_size=32)),
    ("beam5-noncausal-d96-p128", dict(seed=18, lens_q=[5, 3], lens_k=[777, 40], hq=6, hkv=3, d=96,
                                      dtype="bf16", page_size=128, causal=False)),
    # float32 caches (the float32 MFMA kernel, 32-key steps): every head dim, pages smaller
    # and larger than a step, split caches merged, beams without a mask
    ("decode-gqa4-d128-f32-p16-split", dict(seed=21, lens_q=[1] * 5, lens_k=[1, 17, 300, 4000, 0], hq=32, hkv=8,
                                            d=128, dtype="f32", page_size=16)),
    ("draft3-mqa-d64-f32-p8-split", dict(seed=22, lens_q=[3, 1, 2], lens_k=[9000, 5, 700], hq=8, hkv=1, d=64,
                                         dtype="f32", page_size=8)),
    ("beam5-noncausal-d32-f32-p64", dict(seed=23, lens_q=[5, 3], lens_k=[777, 40], hq=6, hkv=3, d=32,
                                         dtype="f32", page_size=64, causal=False)),
    ("decode-gqa4-d96-f32-p4", dict(seed=24, lens_q=[1] * 4, lens_k=[31, 32, 33, 2500], hq=16, hkv=4, d=96,
                                    dtype="f32", page_size=4)),
]


def _dev(c):
    dt = _DT[c.dtype]
    return dict(q=_gpu.to_dev(c.q, dt), kc=_gpu.to_dev(c.k_cache, dt), vc=_gpu.to_dev(c.v_cache, dt),
                cu=torch.from_numpy(c.cu_q).to(DEV), sk=torch.from_numpy(c.seqlens_k).to(DEV),
                bt=torch.from_numpy(c.block_table).to(DEV))


def _run(c, inp, max_k=None, **kw):
    return va.kvcache_fwd(inp["q"], inp["kc"], inp["vc"], inp["cu"], inp["sk"], inp["bt"], max(1, c.max_q),
                          c.max_k if max_k is None else max_k, c.scale, c.causal, **kw)


def _ref(c):
    return oracle.kvcache_forward(c.q, c.k_cache, c.v_cache, c.cu_q, c.seqlens_k, c.block_table, c.page_size,
                                  c.scale, c.causal)


@pytest.mark.parametrize("name,kw", CASES, ids=[x[0] for x in CASES])
def test_kvcache_parity(name, kw):
    print(f"[case] kvcache {name}", flush=True)
    c = kvcache_case(**kw)
    inp = _dev(c)
    out, lse = _run(c, inp)
    torch.cuda.synchronize()
    o_ref, l_ref = _ref(c)
    _gpu.check("out", _gpu.host(out), o_ref, c.dtype)
    _gpu.check_lse(_gpu.host(lse), l_ref, c.dtype)


def test_kvcache_bounds_are_hints():
    """A larger max_seqlen_k (more, shorter chunks for some sequences) and a wider block
    table change nothing beyond rounding; every output element is written, nothing past it."""
    print("[case] kvcache hints", flush=True)
    c = kvcache_case(8, [1, 3, 1], [700, 2500, 40], hq=16, hkv=4, d=64, dtype="bf16", page_size=16,
                     max_pages=400)
    inp = _dev(c)
    o_ref, l_ref = _ref(c)
    pad = 4096
    buf = torch.full((c.q.size + 2 * pad,), 777.0, dtype=torch.bfloat16, device=DEV)
    out = buf[pad:pad + c.q.size].view(c.q.shape)
    out.fill_(float("nan"))
    for max_k in (c.max_k, 6400):
        _, lse = _run(c, inp, max_k=max_k, out=out)
        torch.cuda.synchronize()
        assert bool((buf[:pad] == 777.0).all()) and bool((buf[pad + c.q.size:] == 777.0).all())
        assert not torch.isnan(out).any()
        _gpu.check("out", _gpu.host(out), o_ref, "bf16")
        _gpu.check_lse(_gpu.host(lse), l_ref, "bf16")


def test_kvcache_single_token_ignores_causal_flag():
    print("[case] kvcache causal flag", flush=True)
    c = kvcache_case(9, [1, 1, 1], [33, 1000, 4097], hq=8, hkv=2, d=128, dtype="bf16", page_size=64)
    inp = _dev(c)
    o1, l1 = _run(c, inp)
    c.causal = False
    o0, l0 = _run(c, inp)
    torch.cuda.synchronize()
    assert torch.equal(o1, o0) and torch.equal(l1, l0)


def test_kvcache_deterministic():
    print("[case] kvcache determinism", flush=True)
    c = kvcache_case(10, [1, 2, 1], [9000, 3000, 17], hq=8, hkv=2, d=64, dtype="bf16", page_size=16)
    inp = _dev(c)
    a = [t.clone() for t in _run(c, inp)]
    b = _run(c, inp)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


def test_kvcache_matches_the_packed_forward():
    """The same step through va_varlen_fwd on the gathered keys agrees to rounding."""
    print("[case] kvcache vs packed forward", flush=True)
    c = kvcache_case(12, [1, 4, 2], [400, 1300, 64], hq=16, hkv=4, d=128, dtype="bf16", page_size=32)
    inp = _dev(c)
    out, lse = _run(c, inp)
    k, cu_k = oracle.gather_pages(c.k_cache, c.block_table, c.seqlens_k, c.page_size)
    v, _ = oracle.gather_pages(c.v_cache, c.block_table, c.seqlens_k, c.page_size)
    o2, l2 = va.va_varlen_fwd(inp["q"], _gpu.to_dev(k, torch.bfloat16), _gpu.to_dev(v, torch.bfloat16),
                              inp["cu"], torch.from_numpy(cu_k).to(DEV), c.max_q, c.max_k, c.scale, True)
    torch.cuda.synchronize()
    assert float((out.float() - o2.float()).abs().max()) <= 2e-2
    assert float((lse - l2).abs().max()) <= 1e-3


def test_decode_workload_sampled_rows():
    """The bench's decode workload at full size, in the bench's launch configuration;
    sampled sequences (shortest, longest, and random ones) checked against the oracle."""
    print("[case] decode workload, sampled", flush=True)
    d = decode_device_inputs(DEV)
    sh = DECODE_SHAPE
    B = len(d["lens_k"])
    scale = 1.0 / np.sqrt(sh["d"])
    out, lse = va.kvcache_fwd(d["q"], d["kc"], d["vc"], d["cu"], d["sk"], d["btd"], 1, int(d["lens_k"].max()),
                              scale, True)
    torch.cuda.synchronize()
    rng = np.random.default_rng(5)
    picks = sorted(set([int(np.argmin(d["lens_k"])), int(np.argmax(d["lens_k"]))] +
                       list(rng.choice(B, 6, replace=False))))
    for b in picks:
        n = int(d["lens_k"][b])
        pages = d["bt"][b, : (n + sh["page_size"] - 1) // sh["page_size"]]
        idx = torch.from_numpy(pages.astype(np.int64)).to(DEV)
        kc = _gpu.host(d["kc"][idx])
        vc = _gpu.host(d["vc"][idx])
        bt_local = np.arange(len(pages), dtype=np.int32)[None, :]
        o_ref, l_ref = oracle.kvcache_forward(_gpu.host(d["q"][b:b + 1]), kc, vc, [0, 1], [n], bt_local,
                                              sh["page_size"], scale, True)
        _gpu.check(f"out[{b}] (Lk {n})", _gpu.host(out[b:b + 1]), o_ref, "bf16")
        _gpu.check_lse(_gpu.host(lse[:, b:b + 1]), l_ref, "bf16")
