"""Seeded generators and exact pair/FLOP counters (CPU)."""

import json
import math
import os

import numpy as np
import pytest
import torch

from workloads import bf16_bits, bf16_round, config, make_case, visible_pairs, workload_pairs
from workloads import count as cnt

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_bf16_round_matches_torch_cast():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([1.0, -0.0, 0.0, 3.0e38, -3.0e38, 1e-40, 1.00390625, 1.01171875],
                                 dtype=np.float32)])
    # ties: 1 + 2^-8 is halfway between 1 and 1 + 2^-7 -> even (1.0); 1 + 3*2^-8 -> 1 + 2^-6
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(bf16_bits(x), ref)
    r = bf16_round(x)
    assert np.array_equal(r, torch.from_numpy(x).to(torch.bfloat16).float().numpy())
    assert r[-2] == 1.0 and r[-1] == np.float32(1.015625)


def test_pair_counts_golden():
    with open(os.path.join(GOLDEN, "pair_counts.json")) as f:
        g = json.load(f)
    ex = g["worked_example"]
    assert cnt.dense_mask_pairs(ex["lengths"]) == ex["dense_mask_pairs"]
    assert cnt.padded_pairs(ex["lengths"]) == ex["padded_pairs"]
    assert workload_pairs(ex["lengths"], ex["lengths"], False) == ex["varlen_pairs_noncausal"]
    for c in g["closed_forms"]:
        assert workload_pairs(c["lens_q"], c["lens_k"], c["causal"]) == c["pairs"], c["what"]


@pytest.mark.parametrize("lq,lk", [(1, 1), (5, 2), (2, 5), (7, 7), (0, 3), (3, 0), (17, 40), (40, 17)])
def test_visible_pairs_brute(lq, lk):
    for causal in (False, True):
        n = sum(1 for i in range(lq) for j in range(lk) if (not causal) or j <= i + lk - lq)
        assert visible_pairs(lq, lk, causal) == n


def test_configs_are_deterministic_and_shaped():
    a, b = config(1), config(1)
    assert np.array_equal(a.q, b.q) and np.array_equal(a.v, b.v)
    assert list(a.lens_q) == [3, 17, 64, 128] and a.total_q == 212 and a.dtype == "f32"
    assert a.q.shape == (212, 2, 64) and a.scale == 1.0 / 8.0 and a.causal
    c5 = config(5)
    assert c5.q.shape == (112, 32, 128) and c5.k.shape == (262, 8, 128)
    assert c5.dout is not None and c5.dtype == "bf16"
    assert np.array_equal(c5.q, bf16_round(c5.q))


def test_length_laws():
    c2 = config(2)
    assert c2.batch == 20 and c2.lens_q.min() >= 64 and c2.lens_q.max() <= 1024
    assert c2.hq == 14 and c2.hkv == 2 and c2.d == 64
    c3 = config(3, with_dout=False)
    assert c3.batch == 16 and c3.lens_q.max() == 2048 and c3.lens_q.min() >= 128
    c4 = config(4)
    assert c4.batch == 512 and c4.lens_q.min() >= 1 and c4.lens_q.max() <= 256
    assert not c4.causal and c4.hq == 8 == c4.hkv


def test_config4_bias_views():
    w = config(4, dtype="bf16", bias="per_key")
    assert w.bias.shape == (512 * 8 * 256,) and w.bias_strides == (2048, 256, 0, 1)
    assert np.array_equal(w.bias, bf16_round(w.bias))


def test_make_case_bias_layouts():
    for layout in ("contiguous", "permuted", "head_shared"):
        w = make_case(3, [3, 5], lens_k=[4, 2], hq=2, hkv=1, d=4, bias="per_pair",
                      bias_layout=layout)
        s0, s1, s2, s3 = w.bias_strides
        # every valid (b, h, r, c) addresses inside the array
        mx = max(b * s0 + h * s1 + r * s2 + c * s3
                 for b in range(2) for h in range(2) for r in range(5) for c in range(4))
        assert mx < w.bias.size
        if layout == "head_shared":
            assert s1 == 0
        if layout == "permuted":
            assert s3 != 1
    wk = make_case(3, [3, 5], hq=2, hkv=1, d=4, bias="per_key")
    assert wk.bias_strides[2] == 0


def test_flop_counts():
    w = config(1)
    assert cnt.fwd_flops(w) == 4 * 64 * 2 * 10495
    assert cnt.bwd_flops(w) == 10 * 64 * 2 * 10495
    c5 = config(5)
    assert cnt.fwd_flops(c5) == 4 * 128 * 32 * 23128
    assert math.isclose(cnt.fwd_flops(c5) / 1e9, 0.379, rel_tol=2e-3)
