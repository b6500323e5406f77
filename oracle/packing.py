"""CPU oracle for the steps on either side of the packed path: packing metadata
from a padding mask, and unpad (gather) / pad (scatter) between the padded
[batch, seqlen, ...] layout and the packed [total, ...] stream.

TEST INFRASTRUCTURE.  Only ``tests/``, the smoke check in ``__graft_entry__``
and the CPU-baseline leg of ``bench.py`` may import it.  It shares no code
with the HIP library or its Python binding.

What it computes (the TorchEasyRec pull request 663 page, intro: one packed
stream with explicit cu_seq_lens boundaries and per-row position_ids; the
FDMA pull request 118 page, section "Key Implementation Points" under
"Variable Length Flow": unpad before the kernel and pad back after, one
indexing pass shared by Q, K and V):

For a padding mask M [batch, seqlen] (nonzero = a real token), row b keeps
the positions s with M[b, s] != 0 in increasing order:

    L_b           = number of kept positions of row b
    cu_seqlens    = [0, L_0, L_0 + L_1, ...]            (int32, batch + 1)
    max_seqlen    = max_b L_b                            (0 for an empty batch)
    indices[t]    = b * seqlen + s of the t-th kept token, rows in order
    position_ids[t] = the rank of that token inside its row (0 .. L_b - 1)
    inverse[b * seqlen + s] = t for a kept token, -1 for padding

    unpad: packed[t] = padded_flat[indices[t]]
    pad:   padded_flat[p] = packed[inverse[p]] if inverse[p] >= 0, else 0

The mask need not be left- or right-aligned: kept tokens keep their order.
"""

from __future__ import annotations

import numpy as np


def pack_metadata(mask):
    """(cu_seqlens, max_seqlen, indices, position_ids, inverse) of a [batch, seqlen] mask."""
    m = np.asarray(mask) != 0
    batch, seqlen = m.shape
    lens = [int(m[b].sum()) for b in range(batch)]
    cu = np.zeros(batch + 1, dtype=np.int32)
    for b in range(batch):
        cu[b + 1] = cu[b] + lens[b]
    indices, position_ids = [], []
    inverse = np.full(batch * seqlen, -1, dtype=np.int32)
    for b in range(batch):
        rank = 0
        for s in range(seqlen):
            if m[b, s]:
                inverse[b * seqlen + s] = len(indices)
                indices.append(b * seqlen + s)
                position_ids.append(rank)
                rank += 1
    return (cu, max(lens) if lens else 0, np.asarray(indices, dtype=np.int32),
            np.asarray(position_ids, dtype=np.int32), inverse)


def unpad(padded, indices):
    """Rows of the flattened padded tensor [batch * seqlen, ...] picked by indices."""
    x = np.asarray(padded)
    flat = x.reshape((x.shape[0] * x.shape[1],) + x.shape[2:])
    return flat[np.asarray(indices, dtype=np.int64)]


def pad(packed, inverse, batch, seqlen):
    """[batch, seqlen, ...] tensor holding packed[inverse[p]] at p, zeros where inverse is -1."""
    y = np.asarray(packed)
    inv = np.asarray(inverse)
    out = np.zeros((batch * seqlen,) + y.shape[1:], dtype=y.dtype)
    for p in range(batch * seqlen):
        if inv[p] >= 0:
            out[p] = y[inv[p]]
    return out.reshape((batch, seqlen) + y.shape[1:])
