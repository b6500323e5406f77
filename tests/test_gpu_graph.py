"""HIP graph capture of the library's calls.

Every call only enqueues kernels (no allocation, memset or synchronisation
inside the library), so a forward + backward step and a decode step can be
captured once and replayed.  Each replay runs after unrelated eager work on
the same buffers' device and must reproduce the eager results bitwise (the
kernels are deterministic); the inputs are rewritten between replays to show
that a replay reads the current contents.
"""

import numpy as np
import pytest
import torch

import variable_length_packed_amd as va
from workloads import make_case
from workloads.kvcache import kvcache_case

from . import _gpu

pytestmark = pytest.mark.gpu

DEV = _gpu.DEV


def _alloc_step(w, inp):
    tq, tk = w.total_q, w.total_k
    buf = dict(
        out=torch.empty_like(inp["q"]), lse=torch.empty((w.hq, tq), dtype=torch.float32, device=DEV),
        dq=torch.empty((tq, w.hq, w.d), dtype=torch.float32, device=DEV),
        dk=torch.empty((tk, w.hkv, w.d), dtype=torch.float32, device=DEV),
        dv=torch.empty((tk, w.hkv, w.d), dtype=torch.float32, device=DEV),
        wf=torch.empty(va.va_varlen_fwd_workspace_size(w.batch, tq, tk, w.max_q, w.max_k, w.hq, w.hkv, w.d,
                                                        inp["q"].dtype), dtype=torch.uint8, device=DEV),
        wb=torch.empty(va.va_varlen_bwd_workspace_size(w.batch, tq, tk, w.max_q, w.max_k, w.hq, w.hkv, w.d,
                                                        inp["q"].dtype, torch.float32),
                       dtype=torch.uint8, device=DEV))
    return buf


def _step(w, inp, b):
    va.va_varlen_fwd(inp["q"], inp["k"], inp["v"], inp["cu_q"], inp["cu_k"], w.max_q, w.max_k, w.scale,
                     w.causal, out=b["out"], lse=b["lse"], workspace=b["wf"])
    va.va_varlen_bwd(inp["dout"], inp["q"], inp["k"], inp["v"], b["out"], b["lse"], inp["cu_q"], inp["cu_k"],
                     w.max_q, w.max_k, w.scale, w.causal, dq=b["dq"], dk=b["dk"], dv=b["dv"], workspace=b["wb"])


def _snapshot(b, names):
    return [b[n].clone() for n in names]


@pytest.mark.parametrize("short", [False, True])
def test_fwd_bwd_step_replays(short):
    print(f"[case] graph fwd+bwd short={short}", flush=True)
    if short:  # the short-query path (decode kernels) in the forward
        w = make_case(131, [1, 4, 2, 3], lens_k=[900, 40, 3000, 5], hq=16, hkv=4, d=64, causal=True,
                      dtype="bf16", with_dout=True)
    else:  # split tiles in every pass
        w = make_case(132, [37, 300, 2600, 129], hq=14, hkv=2, d=64, causal=True, dtype="bf16", with_dout=True)
    names = ("out", "lse", "dq", "dk", "dv")
    inp = _gpu.device_inputs(w)
    b = _alloc_step(w, inp)
    _step(w, inp, b)  # warm up (loads the library's code objects outside the capture)
    torch.cuda.synchronize()
    eager = _snapshot(b, names)
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            _step(w, inp, b)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    scratch = torch.randn(1 << 20, device=DEV)
    for rep in range(3):
        for n in names:  # garbage in the outputs: the replay must overwrite all of it
            b[n].fill_(float("nan"))
        scratch.mul_(1.0001).add_(float(rep))  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for n, e in zip(names, eager):
            assert torch.equal(b[n], e), (rep, n)
    # new input values: the replay reads the buffers' current contents
    x2 = make_case(133, w.lens_q, lens_k=w.lens_k, hq=w.hq, hkv=w.hkv, d=w.d, causal=w.causal, dtype="bf16",
                   with_dout=True)
    inp2 = _gpu.device_inputs(x2)
    for n in ("q", "k", "v", "dout"):
        inp[n].copy_(inp2[n])
    g.replay()
    torch.cuda.synchronize()
    replayed = _snapshot(b, names)
    _step(w, inp, b)
    torch.cuda.synchronize()
    for n, r in zip(names, replayed):
        assert torch.equal(b[n], r), n
    assert not torch.equal(replayed[0], eager[0])


def test_decode_step_replays():
    print("[case] graph decode step", flush=True)
    c = kvcache_case(134, [1] * 8, [5, 700, 3000, 1, 0, 64, 1025, 9000], hq=32, hkv=8, d=128, dtype="bf16",
                     page_size=64)
    q = _gpu.to_dev(c.q, torch.bfloat16)
    kc, vc = _gpu.to_dev(c.k_cache, torch.bfloat16), _gpu.to_dev(c.v_cache, torch.bfloat16)
    cu = torch.from_numpy(c.cu_q).to(DEV)
    sk = torch.from_numpy(c.seqlens_k).to(DEV)
    bt = torch.from_numpy(c.block_table).to(DEV)
    out = torch.empty_like(q)
    lse = torch.empty((c.hq, c.total_q), dtype=torch.float32, device=DEV)
    ws = torch.empty(va.kvcache_fwd_workspace_size(c.batch, 1, c.max_k, c.hq, c.hkv, c.d, torch.bfloat16),
                     dtype=torch.uint8, device=DEV)

    def step():
        va.kvcache_fwd(q, kc, vc, cu, sk, bt, 1, c.max_k, c.scale, True, out=out, lse=lse, workspace=ws)

    step()
    torch.cuda.synchronize()
    eager = (out.clone(), lse.clone())
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        with torch.cuda.graph(g, stream=side):
            step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    for rep in range(3):
        out.fill_(float("nan"))
        lse.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, eager[0]) and torch.equal(lse, eager[1]), rep
    # sequence 0 becomes a copy of sequence 7 (its query, length and pages, all
    # changed on the device): the replay follows, and the two rows agree bitwise
    q[0].copy_(q[7])
    sk[0] = int(c.seqlens_k[7])
    bt2 = bt.clone()
    bt2[0] = bt[7]
    bt.copy_(bt2)
    g.replay()
    torch.cuda.synchronize()
    r = (out.clone(), lse.clone())
    step()
    torch.cuda.synchronize()
    assert torch.equal(out, r[0]) and torch.equal(lse, r[1])
    assert torch.equal(out[0], out[7])
    assert np.isfinite(_gpu.host(lse)[:, [0, 1, 2, 3, 5, 6, 7]]).all()
