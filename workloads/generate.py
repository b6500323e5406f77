"""Seeded synthetic packed-attention workloads.

Every tensor is drawn as float32 from a counter-free PCG64 stream keyed by
``SeedSequence([config_id, stream_id])`` and laid out token-major,
``[tokens, heads, head_dim]``, the packed layout of the FlashAttention-2
varlen path that the TorchEasyRec pull request 663 page describes (intro:
one concatenated stream with explicit cumulative sequence boundaries).  A
bf16 workload stores the round-to-nearest-even bf16 value of each float32
draw; the float32 array that carries it is exact, so the oracle and the GPU
read identical numbers.

The five named configurations are the synthetic stand-ins for the pages'
private workloads (GenRec batches of real length on the TorchEasyRec page,
section "Measured"; the graph encoder of the GiGL pull request 858 page,
section "Performance"; the short GQA shape of the ASpec pull request 25 page,
section "Verification").  Their length laws and value distributions are
stated in each builder below.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Optional, Sequence

import numpy as np

# Stream ids inside one SeedSequence([config_id, stream_id]).
STREAM_LENGTHS = 0
STREAM_Q = 1
STREAM_K = 2
STREAM_V = 3
STREAM_DOUT = 4
STREAM_BIAS = 5

CONFIG_IDS = (1, 2, 3, 4, 5)

# Grid edge of the graph-encoder bias: the encoder's max_seq_len (GiGL page,
# section "Performance": max_seq_len 256).
GRAPH_GRID = 256


def _rng(*key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(list(key))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bf16 (nearest, ties to even); return the uint16 bit patterns.

    Inputs must be finite.  The upper 16 bits of the float32 pattern are kept
    after adding 0x7FFF plus the lowest kept bit, which is round-half-to-even
    on the discarded 16 bits.
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("bf16_bits expects finite values")
    # finite patterns are at most 0xFF7FFFFF, so the sum stays below 2^32
    u = x.view(np.uint32)
    r = (u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are the bf16 rounding of ``x`` (exactly representable)."""
    bits = bf16_bits(x).astype(np.uint32) << 16
    return bits.view(np.float32).reshape(np.shape(x))


def f16_round(x: np.ndarray) -> np.ndarray:
    """float32 array whose values are the IEEE binary16 rounding of ``x`` (nearest, ties to even).

    Inputs must be finite and below the binary16 overflow threshold (65520).
    """
    x = np.asarray(x, dtype=np.float32)
    if not np.all(np.abs(x) < 65520.0):
        raise ValueError("f16_round expects finite values below 65520")
    return x.astype(np.float16).astype(np.float32)


def _cu(lengths: Sequence[int]) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, dtype=np.int64))
    return cu


@dataclass
class Workload:
    """One packed attention problem: host arrays plus metadata.

    ``q``/``k``/``v``/``dout`` are float32 arrays ``[T, H, d]`` holding values
    exactly representable in ``dtype``.  ``bias`` (if any) is a flat float32
    array, likewise representable, read at element offset
    ``b*s0 + h*s1 + r*s2 + c*s3`` with ``(s0, s1, s2, s3) = bias_strides`` and
    ``r``, ``c`` the query and key index local to sequence ``b``.
    """

    name: str
    dtype: str  # "f32", "bf16" or "f16"
    causal: bool
    lens_q: np.ndarray
    lens_k: np.ndarray
    hq: int
    hkv: int
    d: int
    scale: float
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dout: Optional[np.ndarray] = None
    bias: Optional[np.ndarray] = None
    bias_strides: Optional[tuple] = None
    bias_kind: str = "none"
    notes: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return int(len(self.lens_q))

    @property
    def cu_q(self) -> np.ndarray:
        return _cu(self.lens_q)

    @property
    def cu_k(self) -> np.ndarray:
        return _cu(self.lens_k)

    @property
    def total_q(self) -> int:
        return int(np.sum(self.lens_q))

    @property
    def total_k(self) -> int:
        return int(np.sum(self.lens_k))

    @property
    def max_q(self) -> int:
        return int(np.max(self.lens_q)) if len(self.lens_q) else 0

    @property
    def max_k(self) -> int:
        return int(np.max(self.lens_k)) if len(self.lens_k) else 0

    def describe(self) -> dict:
        return {
            "name": self.name,
            "dtype": self.dtype,
            "causal": self.causal,
            "batch": self.batch,
            "total_q": self.total_q,
            "total_k": self.total_k,
            "max_q": self.max_q,
            "max_k": self.max_k,
            "hq": self.hq,
            "hkv": self.hkv,
            "d": self.d,
            "bias": self.bias_kind,
        }


def _draw(rng: np.random.Generator, shape, dtype: str, std: float = 1.0) -> np.ndarray:
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    if dtype == "bf16":
        return bf16_round(x)
    if dtype == "f16":
        return f16_round(x)
    return x


def _lengths(cfg_id: int) -> tuple:
    r = _rng(cfg_id, STREAM_LENGTHS)
    if cfg_id == 1:
        lq = np.array([3, 17, 64, 128], dtype=np.int64)
        return lq, lq.copy()
    if cfg_id == 2:
        # 20 sequences, lengths uniform on the integers 64..1024 inclusive.
        lq = r.integers(64, 1025, size=20).astype(np.int64)
        return lq, lq.copy()
    if cfg_id == 3:
        # 16 sequences, log-uniform on [128, 2048], rounded to integers and
        # clamped; the longest draw is set to exactly 2048.
        u = r.uniform(math.log(128.0), math.log(2048.0), size=16)
        lq = np.clip(np.rint(np.exp(u)), 128, 2048).astype(np.int64)
        lq[int(np.argmax(lq))] = 2048
        return lq, lq.copy()
    if cfg_id == 4:
        # 512 graph sequences, lengths uniform on 1..256 inclusive.
        lq = r.integers(1, 257, size=512).astype(np.int64)
        return lq, lq.copy()
    if cfg_id == 5:
        return np.array([112], dtype=np.int64), np.array([262], dtype=np.int64)
    raise ValueError(f"unknown config {cfg_id}")


_SHAPES = {
    # cfg: (hq, hkv, d, causal, default dtype, has backward)
    1: (2, 2, 64, True, "f32", False),
    2: (14, 2, 64, True, "bf16", False),
    3: (14, 2, 64, True, "bf16", True),
    4: (8, 8, 64, False, "f32", False),
    5: (32, 8, 128, True, "bf16", True),
}

_NAMES = {
    1: "tiny fp32 causal varlen fwd, 4 seqs {3,17,64,128}, 2/2 heads, d64",
    2: "Qwen2.5-0.5B-shaped causal GQA fwd, 20 seqs U[64,1024], 14/2 heads, d64",
    3: "long-row causal GQA fwd+bwd, 16 seqs logU[128,2048] incl. 2048, 14/2 heads, d64",
    4: "graph-encoder non-causal fwd, 512 seqs U[1,256], 8/8 heads, d64",
    5: "short GQA cross-length causal fwd+bwd, Lq 112 / Lk 262, 32/8 heads, d128",
}


def config(cfg_id: int, dtype: Optional[str] = None, bias: str = "none",
           with_dout: Optional[bool] = None) -> Workload:
    """Build one of the five named workloads.

    ``bias`` applies to config 4 only: ``"none"``, ``"per_key"`` (a
    ``[512, 8, 256]`` vector per sequence and head, N(0, 1), strides
    ``(2048, 256, 0, 1)``) or ``"per_pair"`` (a contiguous ``[512, 8, 256, 256]``
    grid, normal with standard deviation 0.5, read through strides
    ``(524288, 65536, 256, 1)``).
    """
    hq, hkv, d, causal, dt0, has_bwd = _SHAPES[cfg_id]
    dtype = dtype or dt0
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(dtype)
    lq, lk = _lengths(cfg_id)
    tq, tk = int(lq.sum()), int(lk.sum())
    q = _draw(_rng(cfg_id, STREAM_Q), (tq, hq, d), dtype)
    k = _draw(_rng(cfg_id, STREAM_K), (tk, hkv, d), dtype)
    v = _draw(_rng(cfg_id, STREAM_V), (tk, hkv, d), dtype)
    if with_dout is None:
        with_dout = has_bwd
    dout = _draw(_rng(cfg_id, STREAM_DOUT), (tq, hq, d), dtype) if with_dout else None
    b_arr, b_str = None, None
    if bias != "none":
        if cfg_id != 4:
            raise ValueError("only config 4 carries a bias")
        B, G = len(lq), GRAPH_GRID
        if bias == "per_key":
            b_arr = _draw(_rng(cfg_id, STREAM_BIAS), (B * hq * G,), dtype)
            b_str = (hq * G, G, 0, 1)
        elif bias == "per_pair":
            b_arr = _draw(_rng(cfg_id, STREAM_BIAS), (B * hq * G * G,), dtype, std=0.5)
            b_str = (hq * G * G, G * G, G, 1)
        else:
            raise ValueError(bias)
    name = _NAMES[cfg_id]
    if cfg_id == 4:
        name += f", {dtype}, bias={bias}"
    return Workload(name=name, dtype=dtype, causal=causal, lens_q=lq, lens_k=lk,
                    hq=hq, hkv=hkv, d=d, scale=1.0 / math.sqrt(d), q=q, k=k, v=v,
                    dout=dout, bias=b_arr, bias_strides=b_str, bias_kind=bias,
                    notes={"config": cfg_id})


def make_case(seed: int, lens_q: Sequence[int], lens_k: Optional[Sequence[int]] = None,
              hq: int = 2, hkv: int = 2, d: int = 64, causal: bool = False,
              dtype: str = "f32", bias: str = "none", bias_layout: str = "contiguous",
              bias_std: float = 1.0, with_dout: bool = False,
              scale: Optional[float] = None, grid: Optional[tuple] = None) -> Workload:
    """A small seeded case for unit tests.

    ``bias``: ``"none"``, ``"per_key"`` or ``"per_pair"``.  ``bias_layout``:
    ``"contiguous"`` (``[B, H, R, C]`` row-major, R = 1 for per-key),
    ``"permuted"`` (storage ``[B, C, H, R]`` viewed as ``[B, H, R, C]``, so no
    stride is 1 on the key axis), or ``"head_shared"`` (head stride 0).
    ``grid`` = (R, C) fixes the bias grid edge (default: the max lengths).
    """
    if dtype not in ("f32", "bf16", "f16"):
        raise ValueError(dtype)
    lens_q = np.asarray(list(lens_q), dtype=np.int64)
    lens_k = lens_q.copy() if lens_k is None else np.asarray(list(lens_k), dtype=np.int64)
    if len(lens_q) != len(lens_k):
        raise ValueError("lens_q and lens_k differ in batch")
    tq, tk = int(lens_q.sum()), int(lens_k.sum())
    base = (100, int(seed))
    q = _draw(_rng(*base, STREAM_Q), (tq, hq, d), dtype)
    k = _draw(_rng(*base, STREAM_K), (tk, hkv, d), dtype)
    v = _draw(_rng(*base, STREAM_V), (tk, hkv, d), dtype)
    dout = _draw(_rng(*base, STREAM_DOUT), (tq, hq, d), dtype) if with_dout else None
    b_arr, b_str = None, None
    if bias != "none":
        B = len(lens_q)
        R0 = max(1, int(lens_q.max()) if B else 1)
        C0 = max(1, int(lens_k.max()) if B else 1)
        if grid is not None:
            R0, C0 = grid
        R = 1 if bias == "per_key" else R0
        C = C0
        H = 1 if bias_layout == "head_shared" else hq
        b_arr = _draw(_rng(*base, STREAM_BIAS), (B * H * R * C,), dtype, std=bias_std)
        if bias_layout in ("contiguous", "head_shared"):
            s = (H * R * C, R * C, C, 1)
            if H == 1:
                s = (R * C, 0, C, 1)
        elif bias_layout == "permuted":
            # storage [B, C, H, R]
            s = (C * H * R, R, 1, H * R)
        else:
            raise ValueError(bias_layout)
        if bias == "per_key":
            s = (s[0], s[1], 0, s[3])
        b_str = tuple(int(x) for x in s)
    sc = (1.0 / math.sqrt(d)) if scale is None else float(scale)
    return Workload(name=f"case seed={seed}", dtype=dtype, causal=causal,
                    lens_q=lens_q, lens_k=lens_k, hq=hq, hkv=hkv, d=d, scale=sc,
                    q=q, k=k, v=v, dout=dout, bias=b_arr, bias_strides=b_str,
                    bias_kind=bias, notes={"seed": seed, "bias_layout": bias_layout})


def padding_mask(seed: int, batch: int, seqlen: int, kind: str = "random",
                 lengths: Optional[Sequence[int]] = None) -> np.ndarray:
    """uint8 [batch, seqlen] padding mask (1 = real token) of a padded batch.

    kind "right" / "left": each row holds ``lengths[b]`` real tokens (drawn
    uniform in [0, seqlen] when not given) at its start / end; "random": every
    position is real with probability 0.6 (interior padding).
    """
    rng = _rng(seed, batch, seqlen, 7)
    m = np.zeros((batch, seqlen), dtype=np.uint8)
    if kind == "random":
        m[:] = rng.random((batch, seqlen)) < 0.6
        return m
    lens = list(lengths) if lengths is not None else list(rng.integers(0, seqlen + 1, size=batch))
    for b, L in enumerate(lens):
        if kind == "right":
            m[b, :L] = 1
        elif kind == "left":
            m[b, seqlen - L:] = 1
        else:
            raise ValueError(kind)
    return m
