"""Pins for the paged-KV-cache oracle (``oracle.kvcache``), each against something
other than itself:

* a gather worked out by hand on a four-page pool (page/slot codes written out);
* renumbering the pages of the pool (moving every page and rewriting the block
  table to match) leaves the result bitwise unchanged;
* a decode step of Lq new tokens equals the last Lq rows of causal attention
  over the whole sequence (bottom-right alignment: the new tokens are the last
  rows of the prefill);
* for Lq = 1 the causal flag changes nothing (the flash-sparse-attention pull
  request 118 page, section "Key Implementation Points", drops the flag for
  single-token decode steps);
* empty caches give O = 0, LSE = -inf.

Planted mistakes in the oracle's source must fail them.
"""

import types

import numpy as np
import pytest

import oracle
from oracle import kvcache as okv
from workloads.kvcache import kvcache_case


def test_gather_by_hand():
    # pool of 4 pages of 2 slots; element [p, s, 0, 0] holds code 10 p + s
    cache = np.zeros((4, 2, 1, 1))
    for p in range(4):
        for s in range(2):
            cache[p, s, 0, 0] = 10 * p + s
    bt = np.array([[2, 0], [3, -1], [-1, -1]], dtype=np.int32)
    rows, cu = okv.gather_pages(cache, bt, [3, 1, 0], 2)
    # sequence 0: keys 0, 1 on page 2, key 2 on page 0; sequence 1: key 0 on page 3
    assert rows[:, 0, 0].tolist() == [20.0, 21.0, 0.0, 30.0]
    assert cu.tolist() == [0, 3, 4, 4]


def _run(c, mod=okv, causal=None):
    return mod.kvcache_forward(c.q, c.k_cache, c.v_cache, c.cu_q, c.seqlens_k, c.block_table,
                               c.page_size, c.scale, c.causal if causal is None else causal)


CASES = [
    dict(seed=1, lens_q=[1, 1, 1], lens_k=[5, 17, 1], hq=4, hkv=2, d=8, page_size=4),
    dict(seed=2, lens_q=[3, 1, 2], lens_k=[7, 9, 2], hq=6, hkv=2, d=4, page_size=2),
    dict(seed=3, lens_q=[2, 4], lens_k=[40, 33], hq=2, hkv=1, d=4, page_size=16),
]


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_page_renumbering_is_invisible(ci):
    c = kvcache_case(**CASES[ci])
    o, lse = _run(c)
    perm = np.random.default_rng(ci).permutation(c.num_pages)
    k2 = np.empty_like(c.k_cache)
    v2 = np.empty_like(c.v_cache)
    k2[perm] = c.k_cache
    v2[perm] = c.v_cache
    bt2 = np.where(c.block_table >= 0, perm[np.maximum(c.block_table, 0)], -1).astype(np.int32)
    o2, lse2 = okv.kvcache_forward(c.q, k2, v2, c.cu_q, c.seqlens_k, bt2, c.page_size, c.scale, c.causal)
    assert np.array_equal(o, o2) and np.array_equal(lse, lse2)


@pytest.mark.parametrize("ci", range(len(CASES)))
def test_decode_rows_are_the_last_rows_of_a_causal_prefill(ci, mod=okv):
    c = kvcache_case(**CASES[ci])
    o, lse = _run(c, mod)
    k, cu_k = okv.gather_pages(c.k_cache, c.block_table, c.seqlens_k, c.page_size)
    v, _ = okv.gather_pages(c.v_cache, c.block_table, c.seqlens_k, c.page_size)
    rng = np.random.default_rng(100 + ci)
    cu_q = c.cu_q
    for b in range(c.batch):
        lq, lk = int(c.lens_q[b]), int(c.lens_k[b])
        if lq > lk:
            continue
        # queries of the whole sequence: lk - lq earlier tokens, then the decode step's
        full_q = np.concatenate([rng.standard_normal((lk - lq, c.hq, c.d)), c.q[cu_q[b]:cu_q[b + 1]]])
        ks, vs = k[cu_k[b]:cu_k[b + 1]], v[cu_k[b]:cu_k[b + 1]]
        of, lf = oracle.forward(full_q, ks, vs, [0, lk], [0, lk], c.scale, True)
        assert np.max(np.abs(of[lk - lq:] - o[cu_q[b]:cu_q[b + 1]])) <= 1e-12
        assert np.max(np.abs(lf[:, lk - lq:] - lse[:, cu_q[b]:cu_q[b + 1]])) <= 1e-12


def test_single_token_steps_ignore_the_causal_flag():
    c = kvcache_case(**CASES[0])
    o1, l1 = _run(c, causal=True)
    o0, l0 = _run(c, causal=False)
    assert np.array_equal(o1, o0) and np.array_equal(l1, l0)


def test_empty_cache_rows():
    c = kvcache_case(seed=4, lens_q=[2, 1], lens_k=[0, 3], hq=2, hkv=2, d=4, page_size=2)
    o, lse = _run(c)
    assert not o[:2].any() and np.all(np.isneginf(lse[:, :2]))
    assert np.all(np.isfinite(lse[:, 2:]))


MUTATIONS = [
    ("slot off by one", "cache[page, j % page_size]", "cache[page, (j + 1) % page_size]"),
    ("another sequence's table", "int(bt[b, j // page_size])", "int(bt[0, j // page_size])"),
    ("causal flag dropped", "return forward(q, k, v, cu_q, cu_k, scale, causal)",
     "return forward(q, k, v, cu_q, cu_k, scale, False)"),
]


def _mutant(old, new):
    with open(okv.__file__) as f:
        src = f.read()
    assert src.count(old) == 1, old
    mod = types.ModuleType("oracle.kvcache_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), okv.__file__, "exec"), mod.__dict__)
    return mod


@pytest.mark.parametrize("name,old,new", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_planted_mistakes_are_caught(name, old, new):
    mod = _mutant(old, new)
    caught = False
    try:
        rows, _ = mod.gather_pages(np.arange(8.0).reshape(4, 2, 1, 1), np.array([[2, 0], [3, -1]]), [3, 1], 2)
        caught = rows[:, 0, 0].tolist() != [4.0, 5.0, 0.0, 6.0]
    except (IndexError, ValueError):
        caught = True
    for ci in range(len(CASES)):
        if caught:
            break
        try:
            test_decode_rows_are_the_last_rows_of_a_causal_prefill(ci, mod)
        except AssertionError:
            caught = True
    assert caught, name
