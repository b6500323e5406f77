"""CPU oracle for attention against a paged KV cache (decode steps).

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import it.  It shares no code
with the HIP library or its Python binding, and neither side imports the
other.

What it computes.  A decode step attends the few new query tokens of each
sequence (one per step; a handful for beams or speculative drafts) to every
key the sequence has cached.  The noether pull request 236 page (section
"module") names ``flash_attn_with_kvcache``, the cached-decode call of the
FlashAttention library, among the functions its code base needs; the
TorchEasyRec pull request 663 page (section "Test plan") tests ragged beam
decoding; the flash-sparse-attention pull request 118 page (sections "Key
Implementation Points" and "Recommended Automated Tests") notes that for a
single-token decode step the causal mask changes nothing.  The pages do not
spell the cache layout out; the plainest reading, that library's paged
layout, is used:

* ``k_cache`` and ``v_cache`` are ``[num_pages, page_size, Hkv, d]``;
* key ``j`` of sequence ``b`` (``0 <= j < seqlens_k[b]``) is slot
  ``j % page_size`` of page ``block_table[b, j // page_size]``;
* the queries are packed ``[total_q, Hq, d]`` with ``cu_seqlens_q``, the
  outputs ``O [total_q, Hq, d]`` and ``LSE [Hq, total_q]`` as for the packed
  forward, and a causal mask is bottom-right aligned (query ``i`` of ``Lq``
  sees key ``j`` iff ``j <= i + Lk - Lq``).

So the step is the packed forward over each sequence's gathered keys.  The
gather below is written out key by key; the attention itself is
``attention.forward``, pinned on its own.

Pins: ``tests/test_oracle_kvcache.py`` (a hand-gathered example, page
permutations, the last rows of a causal prefill, q_len = 1 with and without
the causal flag, planted mistakes).
"""

from __future__ import annotations

import numpy as np

from .attention import forward


def gather_pages(cache, block_table, seqlens_k, page_size):
    """Keys (or values) of every sequence, packed: ([total_k, Hkv, d] float64, cu_seqlens_k int32).

    Row ``cu[b] + j`` is slot ``j % page_size`` of page ``block_table[b][j // page_size]``.
    """
    cache = np.asarray(cache, dtype=np.float64)
    bt = np.asarray(block_table)
    lens = [int(x) for x in np.asarray(seqlens_k).reshape(-1)]
    cu = np.zeros(len(lens) + 1, dtype=np.int32)
    rows = []
    for b, n in enumerate(lens):
        cu[b + 1] = cu[b] + n
        for j in range(n):
            page = int(bt[b, j // page_size])
            rows.append(cache[page, j % page_size])
    if rows:
        out = np.stack(rows)
    else:
        out = np.zeros((0,) + cache.shape[2:], dtype=np.float64)
    return out, cu


def kvcache_forward(q, k_cache, v_cache, cu_q, seqlens_k, block_table, page_size, scale, causal):
    """Attention of the packed queries to their sequences' cached keys.

    Returns ``(O [total_q, Hq, d], LSE [Hq, total_q])`` in float64.
    """
    k, cu_k = gather_pages(k_cache, block_table, seqlens_k, page_size)
    v, _ = gather_pages(v_cache, block_table, seqlens_k, page_size)
    return forward(q, k, v, cu_q, cu_k, scale, causal)
