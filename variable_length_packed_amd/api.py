"""Torch-facing marshalling over the C ABI (include/va_varlen.h, include/va_pack.h).

Tensors are checked for device, dtype, rank and contiguity, outputs are
allocated with torch, pointers and the current HIP stream are handed to the
library.  Nothing here computes attention.
"""

from __future__ import annotations

import math
from typing import Optional, Sequence

import torch

from . import _lib


class VaError(RuntimeError):
    """The HIP runtime reported an error inside the library."""


_DTYPES = {torch.float32: _lib.VA_F32, torch.bfloat16: _lib.VA_BF16, torch.float16: _lib.VA_F16}


def _dt(t: torch.Tensor) -> int:
    try:
        return _DTYPES[t.dtype]
    except KeyError:
        raise ValueError(f"dtype {t.dtype} not supported (float32, bfloat16 or float16)") from None


def _raise(status: int, lib) -> None:
    if status == _lib.VA_OK:
        return
    msg = (lib.va_last_error() or b"").decode(errors="replace")
    name = (lib.va_status_string(status) or b"").decode()
    if status == _lib.VA_ERR_HIP:
        raise VaError(f"{name}: {msg}")
    raise ValueError(f"{name}: {msg}")


def _need_dev(name: str, t: torch.Tensor, device, rows: bool = False) -> None:
    """A device tensor on `device`, contiguous -- or, with ``rows``, a [tokens, heads, d]
    view whose heads and elements are dense (its token stride goes to the library)."""
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be on the GPU (got {t.device})")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if rows and t.dim() == 3:
        if t.stride(2) != 1 or (t.shape[1] > 1 and t.stride(1) != t.shape[2]):
            raise ValueError(f"{name} must have dense heads and head_dim (any token stride)")
    elif not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _row_strides(q, k, v):
    """HOST int64[3] token strides of q, k, v, or None when all three are contiguous."""
    if q.is_contiguous() and k.is_contiguous() and v.is_contiguous():
        return None
    return _lib.strides_arg([q.stride(0) if q.shape[0] > 1 else q.shape[1] * q.shape[2],
                             k.stride(0) if k.shape[0] > 1 else k.shape[1] * k.shape[2],
                             v.stride(0) if v.shape[0] > 1 else v.shape[1] * v.shape[2]])


def _bias_args(bias, bias_stride, q, batch, hq, max_q, max_k):
    if bias is None:
        if bias_stride is not None:
            raise ValueError("bias_stride given without bias")
        return None, None
    if bias.device != q.device:
        raise ValueError("bias must be on the same device as q")
    if bias.dtype != q.dtype:
        raise ValueError(f"bias dtype {bias.dtype} must equal the input dtype {q.dtype}")
    if bias_stride is None:
        if bias.dim() != 4:
            raise ValueError("a bias without bias_stride must be 4-D [batch, heads, rows, cols]")
        s = list(bias.stride())
        if bias.shape[1] == 1:
            s[1] = 0
        if bias.shape[2] == 1:
            s[2] = 0
        bias_stride = s
    bias_stride = [int(x) for x in bias_stride]
    if len(bias_stride) != 4 or min(bias_stride) < 0:
        raise ValueError("bias_stride must be 4 non-negative element strides")
    # every element a valid (b, h, r < max_q, c < max_k) may address lies in the storage
    s0, s1, s2, s3 = bias_stride
    hi = (batch - 1) * s0 + (hq - 1) * s1 + (max_q - 1) * s2 + (max_k - 1) * s3
    avail = bias.untyped_storage().nbytes() // bias.element_size() - bias.storage_offset()
    if hi >= avail:
        raise ValueError(f"bias view reaches element {hi} but only {avail} exist")
    return bias.data_ptr(), _lib.strides_arg(bias_stride)


def _stream(device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def va_varlen_fwd(q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                  max_seqlen_q: int, max_seqlen_k: int,
                  softmax_scale: Optional[float] = None, causal: bool = False,
                  bias: Optional[torch.Tensor] = None,
                  bias_stride: Optional[Sequence[int]] = None,
                  out: Optional[torch.Tensor] = None, lse: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  bwd_workspace: Optional[torch.Tensor] = None):
    """Forward.  Returns (out [Tq, Hq, d] in q's dtype, lse [Hq, Tq] float32).

    With ``bwd_workspace`` (a uint8 device buffer of va_varlen_bwd_workspace_size bytes),
    the forward's planner launch also builds the backward's work plans in it
    (va_varlen_fwd_bwdplan); pass the same buffer to va_varlen_bwd with planned=True."""
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_dev(n, t, q.device, rows=True)
    for n, t in (("cu_seqlens_q", cu_seqlens_q), ("cu_seqlens_k", cu_seqlens_k)):
        _need_dev(n, t, q.device)
    if q.dim() != 3 or k.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [tokens, heads, head_dim]")
    if k.shape != v.shape or k.shape[2] != q.shape[2]:
        raise ValueError("k and v must be [total_k, Hkv, d] with q's head_dim")
    if k.dtype != q.dtype or v.dtype != q.dtype:
        raise ValueError("q, k, v must share one dtype")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32:
        raise ValueError("cu_seqlens must be int32")
    if cu_seqlens_q.dim() != 1 or cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens_q and cu_seqlens_k must be 1-D of equal length")
    dt = _dt(q)
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    batch = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    bptr, bstr = _bias_args(bias, bias_stride, q, batch, hq, int(max_seqlen_q), int(max_seqlen_k))
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need_dev("out", out, q.device)
    _need_dev("lse", lse, q.device)
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (hq, tq) or \
            lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or dtype")
    need = lib.va_varlen_fwd_workspace_size(batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k),
                                            hq, hkv, d, dt)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    _need_dev("workspace", workspace, q.device)
    if bwd_workspace is None:
        st = lib.va_varlen_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                               cu_seqlens_k.data_ptr(), int(max_seqlen_q), int(max_seqlen_k), scale,
                               int(bool(causal)), bptr, bstr, out.data_ptr(), lse.data_ptr(),
                               _row_strides(q, k, v), workspace.data_ptr(),
                               workspace.numel() * workspace.element_size(),
                               batch, tq, tk, hq, hkv, d, dt, _stream(q.device))
    else:
        _need_dev("bwd_workspace", bwd_workspace, q.device)
        st = lib.va_varlen_fwd_bwdplan(q.data_ptr(), k.data_ptr(), v.data_ptr(), cu_seqlens_q.data_ptr(),
                                       cu_seqlens_k.data_ptr(), int(max_seqlen_q), int(max_seqlen_k), scale,
                                       int(bool(causal)), bptr, bstr, out.data_ptr(), lse.data_ptr(),
                                       _row_strides(q, k, v), workspace.data_ptr(),
                                       workspace.numel() * workspace.element_size(),
                                       bwd_workspace.data_ptr(),
                                       bwd_workspace.numel() * bwd_workspace.element_size(),
                                       batch, tq, tk, hq, hkv, d, dt, _stream(q.device))
    _raise(st, lib)
    return out, lse


def kvcache_fwd_workspace_size(batch: int, max_seqlen_q: int, max_seqlen_k: int, num_heads_q: int,
                               num_heads_kv: int, head_dim: int, dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.va_kvcache_fwd_workspace_size(batch, max_seqlen_q, max_seqlen_k, num_heads_q,
                                                 num_heads_kv, head_dim, _DTYPES.get(dtype, -1)))


def kvcache_fwd(q: torch.Tensor, k_cache: torch.Tensor, v_cache: torch.Tensor,
                cu_seqlens_q: torch.Tensor, seqlens_k: torch.Tensor, block_table: torch.Tensor,
                max_seqlen_q: int, max_seqlen_k: int, softmax_scale: Optional[float] = None,
                causal: bool = True, out: Optional[torch.Tensor] = None,
                lse: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None):
    """Decode step against a paged KV cache (include/va_kvcache.h).

    q [total_q, Hq, d] (the new tokens, packed by cu_seqlens_q), k_cache / v_cache
    [num_pages, page_size, Hkv, d], seqlens_k int32 [batch], block_table int32
    [batch, pages_per_seq].  Returns (out [total_q, Hq, d], lse [Hq, total_q] float32).
    """
    lib = _lib.load()
    for n, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("cu_seqlens_q", cu_seqlens_q),
                 ("seqlens_k", seqlens_k), ("block_table", block_table)):
        _need_dev(n, t, q.device)
    if q.dim() != 3 or k_cache.dim() != 4 or k_cache.shape != v_cache.shape:
        raise ValueError("q must be [tokens, heads, d] and the caches [pages, page_size, heads, d]")
    if k_cache.shape[3] != q.shape[2] or k_cache.dtype != q.dtype or v_cache.dtype != q.dtype:
        raise ValueError("the caches must share q's head_dim and dtype")
    if cu_seqlens_q.dtype != torch.int32 or seqlens_k.dtype != torch.int32 or block_table.dtype != torch.int32:
        raise ValueError("cu_seqlens_q, seqlens_k and block_table must be int32")
    batch = cu_seqlens_q.numel() - 1
    if cu_seqlens_q.dim() != 1 or seqlens_k.shape != (batch,) or block_table.dim() != 2 or \
            block_table.shape[0] != batch:
        raise ValueError("seqlens_k must be [batch] and block_table [batch, pages_per_seq]")
    dt = _dt(q)
    tq, hq, d = q.shape
    n_pages, page_size, hkv, _ = k_cache.shape
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    if out is None:
        out = torch.empty_like(q)
    if lse is None:
        lse = torch.empty((hq, tq), dtype=torch.float32, device=q.device)
    _need_dev("out", out, q.device)
    _need_dev("lse", lse, q.device)
    if out.shape != q.shape or out.dtype != q.dtype or lse.shape != (hq, tq) or lse.dtype != torch.float32:
        raise ValueError("out/lse have the wrong shape or dtype")
    need = lib.va_kvcache_fwd_workspace_size(batch, int(max_seqlen_q), int(max_seqlen_k), hq, hkv, d, dt)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    _need_dev("workspace", workspace, q.device)
    st = lib.va_kvcache_fwd(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), cu_seqlens_q.data_ptr(),
                            seqlens_k.data_ptr(), block_table.data_ptr(), block_table.shape[1], page_size,
                            n_pages, int(max_seqlen_q), int(max_seqlen_k), scale, int(bool(causal)),
                            out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                            workspace.numel() * workspace.element_size(), batch, tq, hq, hkv, d, dt,
                            _stream(q.device))
    _raise(st, lib)
    return out, lse


def va_varlen_fwd_workspace_size(batch: int, total_q: int, total_k: int, max_seqlen_q: int,
                                 max_seqlen_k: int, num_heads_q: int, num_heads_kv: int,
                                 head_dim: int, dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.va_varlen_fwd_workspace_size(batch, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                                num_heads_q, num_heads_kv, head_dim,
                                                _DTYPES.get(dtype, -1)))


def va_varlen_bwd_workspace_size(batch: int, total_q: int, total_k: int, max_seqlen_q: int,
                                 max_seqlen_k: int, num_heads_q: int, num_heads_kv: int,
                                 head_dim: int, dtype: torch.dtype,
                                 grad_dtype: torch.dtype) -> int:
    lib = _lib.load()
    return int(lib.va_varlen_bwd_workspace_size(batch, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                                num_heads_q, num_heads_kv, head_dim,
                                                _DTYPES.get(dtype, -1),
                                                _DTYPES.get(grad_dtype, -1)))


def va_varlen_bwd(dout: torch.Tensor, q: torch.Tensor, k: torch.Tensor, v: torch.Tensor,
                  out: torch.Tensor, lse: torch.Tensor,
                  cu_seqlens_q: torch.Tensor, cu_seqlens_k: torch.Tensor,
                  max_seqlen_q: int, max_seqlen_k: int,
                  softmax_scale: Optional[float] = None, causal: bool = False,
                  bias: Optional[torch.Tensor] = None,
                  bias_stride: Optional[Sequence[int]] = None,
                  grad_dtype: torch.dtype = torch.float32,
                  dq: Optional[torch.Tensor] = None, dk: Optional[torch.Tensor] = None,
                  dv: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None,
                  dbias: Optional[torch.Tensor] = None,
                  dbias_stride: Optional[Sequence[int]] = None,
                  planned: bool = False):
    """Backward.  Returns (dq, dk, dv) in ``grad_dtype``.

    ``planned``: ``workspace`` holds the work plans a va_varlen_fwd(..., bwd_workspace=workspace)
    of the same batch built (va_varlen_bwd_planned); each such forward feeds one backward.

    With ``dbias`` (a float32 device tensor) and ``dbias_stride`` (4 element
    strides relative to ``dbias``'s first element; 0 sums over that axis), the
    bias gradient is written into ``dbias`` as include/va_varlen.h describes
    (every element of a valid (row, key) pair, 0 where a causal mask hides it;
    elements no valid pair addresses are left as they are).
    """
    lib = _lib.load()
    for n, t in (("q", q), ("k", k), ("v", v)):
        _need_dev(n, t, q.device, rows=True)
    for n, t in (("dout", dout), ("out", out), ("lse", lse), ("cu_seqlens_q", cu_seqlens_q),
                 ("cu_seqlens_k", cu_seqlens_k)):
        _need_dev(n, t, q.device)
    if q.dim() != 3 or k.shape != v.shape or dout.shape != q.shape or out.shape != q.shape:
        raise ValueError("shape mismatch among dout, q, k, v, out")
    if any(t.dtype != q.dtype for t in (k, v, dout, out)):
        raise ValueError("dout, q, k, v, out must share one dtype")
    if lse.dtype != torch.float32 or lse.shape != (q.shape[1], q.shape[0]):
        raise ValueError("lse must be float32 [Hq, total_q]")
    if cu_seqlens_q.dtype != torch.int32 or cu_seqlens_k.dtype != torch.int32 or \
            cu_seqlens_q.shape != cu_seqlens_k.shape:
        raise ValueError("cu_seqlens must be int32 of equal length")
    dt = _dt(q)
    gdt = _DTYPES.get(grad_dtype)
    if gdt is None:
        raise ValueError(f"grad_dtype {grad_dtype} not supported")
    tq, hq, d = q.shape
    tk, hkv, _ = k.shape
    batch = cu_seqlens_q.numel() - 1
    scale = 1.0 / math.sqrt(d) if softmax_scale is None else float(softmax_scale)
    bptr, bstr = _bias_args(bias, bias_stride, q, batch, hq, int(max_seqlen_q), int(max_seqlen_k))
    if dq is None:
        dq = torch.empty(q.shape, dtype=grad_dtype, device=q.device)
    if dk is None:
        dk = torch.empty(k.shape, dtype=grad_dtype, device=q.device)
    if dv is None:
        dv = torch.empty(v.shape, dtype=grad_dtype, device=q.device)
    for n, t, shp in (("dq", dq, q.shape), ("dk", dk, k.shape), ("dv", dv, v.shape)):
        _need_dev(n, t, q.device)
        if t.shape != shp or t.dtype != grad_dtype:
            raise ValueError(f"{n} has the wrong shape or dtype")
    dbptr, dbstr = None, None
    if (dbias is None) != (dbias_stride is None):
        raise ValueError("dbias and dbias_stride go together")
    if dbias is not None:
        if bias is None:
            raise ValueError("dbias needs a bias")
        if dbias.device != q.device or dbias.dtype != torch.float32:
            raise ValueError("dbias must be a float32 tensor on q's device")
        t = [int(x) for x in dbias_stride]
        if len(t) != 4 or min(t) < 0:
            raise ValueError("dbias_stride must be 4 non-negative element strides")
        hi = (batch - 1) * t[0] + (hq - 1) * t[1] + (int(max_seqlen_q) - 1) * t[2] + (int(max_seqlen_k) - 1) * t[3]
        avail = dbias.untyped_storage().nbytes() // 4 - dbias.storage_offset()
        if hi >= avail:
            raise ValueError(f"dbias view reaches element {hi} but only {avail} exist")
        dbptr, dbstr = dbias.data_ptr(), _lib.strides_arg(t)
    need = lib.va_varlen_bwd_workspace_size(batch, tq, tk, int(max_seqlen_q), int(max_seqlen_k),
                                            hq, hkv, d, dt, gdt)
    if workspace is None:
        workspace = torch.empty(max(int(need), 1), dtype=torch.uint8, device=q.device)
    _need_dev("workspace", workspace, q.device)
    if planned and workspace is None:
        raise ValueError("planned=True needs the workspace the forward built the plans in")
    fn = lib.va_varlen_bwd_planned if planned else lib.va_varlen_bwd
    st = fn(dout.data_ptr(), q.data_ptr(), k.data_ptr(), v.data_ptr(),
            out.data_ptr(), lse.data_ptr(), cu_seqlens_q.data_ptr(),
            cu_seqlens_k.data_ptr(), int(max_seqlen_q), int(max_seqlen_k), scale,
            int(bool(causal)), bptr, bstr, dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), dbptr,
            dbstr, _row_strides(q, k, v), workspace.data_ptr(),
            workspace.numel() * workspace.element_size(), batch, tq, tk, hq, hkv,
            d, dt, gdt, _stream(q.device))
    _raise(st, lib)
    return dq, dk, dv


class _VarlenAttn(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, cu_q, cu_k, max_q, max_k, scale, causal, bias, bias_stride,
                grad_dtype):
        out, lse = va_varlen_fwd(q, k, v, cu_q, cu_k, max_q, max_k, scale, causal, bias,
                                 bias_stride)
        ctx.save_for_backward(q, k, v, out, lse, cu_q, cu_k)
        ctx.mark_non_differentiable(lse)
        ctx.bias = bias
        ctx.args = (max_q, max_k, scale, causal, bias_stride, grad_dtype)
        return out, lse

    @staticmethod
    def backward(ctx, dout, dlse):
        q, k, v, out, lse, cu_q, cu_k = ctx.saved_tensors
        max_q, max_k, scale, causal, bias_stride, grad_dtype = ctx.args
        bias = ctx.bias
        db, dbs = None, None
        if bias is not None and ctx.needs_input_grad[9]:
            # a dense float32 gradient shaped like the bias; its size-1 head or row axis
            # (a head-shared or per-key bias) is summed over by a zero stride.  Zeroed:
            # grid elements past a sequence's length belong to no valid pair, so the
            # library leaves them alone, and their gradient is 0
            db = torch.zeros(bias.shape, dtype=torch.float32, device=bias.device)
            dbs = list(db.stride())
            for ax in (1, 2):
                if bias.shape[ax] == 1:
                    dbs[ax] = 0
        dq, dk, dv = va_varlen_bwd(dout.contiguous(), q, k, v, out, lse, cu_q, cu_k, max_q, max_k,
                                   scale, causal, bias, bias_stride, grad_dtype, dbias=db,
                                   dbias_stride=dbs)
        return (dq.to(q.dtype), dk.to(k.dtype), dv.to(v.dtype), None, None, None, None, None,
                None, db.to(bias.dtype) if db is not None else None, None, None)


def varlen_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                softmax_scale=None, causal=False, bias=None, bias_stride=None,
                grad_dtype=torch.float32):
    """Differentiable packed attention: returns (out, lse); gradients flow to q, k, v and
    to a 4-D bias [batch, heads or 1, rows or 1, cols] given without ``bias_stride``.

    A bias read through an explicit ``bias_stride`` view cannot require grad
    (call va_varlen_bwd with dbias for that).  The LSE output carries no gradient.
    """
    if bias is not None and bias.requires_grad and bias_stride is not None:
        raise ValueError("a bias read through bias_stride cannot require grad here: use "
                         "va_varlen_bwd(..., dbias=, dbias_stride=)")
    return _VarlenAttn.apply(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                             softmax_scale, causal, bias, bias_stride, grad_dtype)


def va_timing_start(max_launches: int = 4096) -> None:
    """Record a HIP event pair around each kernel this thread's later calls launch."""
    lib = _lib.load()
    _raise(lib.va_timing_start(int(max_launches)), lib)


def va_timing_stop() -> dict:
    """Stop timing; returns {kernel name: (launches, total milliseconds)}."""
    lib = _lib.load()
    buf = (_lib.KernelTime * 64)()
    n = lib.va_timing_stop(buf, 64)
    if n < 0:
        raise VaError("event timing failed")
    return {buf[i].name.decode(): (int(buf[i].launches), float(buf[i].total_ms))
            for i in range(min(n, 64))}


def va_status_string(status: int) -> str:
    return _lib.load().va_status_string(status).decode()


def va_last_error() -> str:
    return _lib.load().va_last_error().decode(errors="replace")


def va_version() -> int:
    return int(_lib.load().va_version())


# ---------------------------------------------------------------- packing (include/va_pack.h)
def pack_metadata(mask: torch.Tensor):
    """Packing metadata of a padding mask [batch, seqlen] (nonzero = real token), on its device.

    Returns (cu_seqlens int32 [batch+1], max_seqlen int32 [1], indices int32 [batch*seqlen],
    position_ids int32 [batch*seqlen], inverse int32 [batch*seqlen]); only the first
    cu_seqlens[-1] entries of indices and position_ids are meaningful.  No host sync.
    """
    lib = _lib.load()
    _need_dev("mask", mask, None)
    if mask.dim() != 2:
        raise ValueError("mask must be 2-D [batch, seqlen]")
    m = mask if mask.dtype == torch.uint8 else (mask != 0).to(torch.uint8)
    batch, seqlen = m.shape
    dev = m.device
    i32 = dict(dtype=torch.int32, device=dev)
    cu = torch.empty(batch + 1, **i32)
    mx = torch.empty(1, **i32)
    idx = torch.empty(batch * seqlen, **i32)
    pos = torch.empty(batch * seqlen, **i32)
    inv = torch.empty(batch * seqlen, **i32)
    _raise(lib.va_pack_metadata(m.data_ptr(), batch, seqlen, cu.data_ptr(), mx.data_ptr(), idx.data_ptr(),
                                pos.data_ptr(), inv.data_ptr(), _stream(dev)), lib)
    return cu, mx, idx, pos, inv


def _pack_tensors(padded, packed, batch, seqlen):
    if not 1 <= len(padded) <= _lib.VA_PACK_MAX_TENSORS:
        raise ValueError(f"1..{_lib.VA_PACK_MAX_TENSORS} tensors per call")
    arr = (_lib.PackTensor * len(padded))()
    for i, (x, y) in enumerate(zip(padded, packed)):
        _need_dev(f"padded[{i}]", x, padded[0].device)
        _need_dev(f"packed[{i}]", y, padded[0].device)
        if x.shape[0] != batch or x.shape[1] != seqlen:
            raise ValueError(f"padded[{i}] must be [batch, seqlen, ...]")
        if y.shape[1:] != x.shape[2:] or y.dtype != x.dtype:
            raise ValueError(f"packed[{i}] must be [rows, ...] with the padded tensor's row shape and dtype")
        arr[i].padded = x.data_ptr()
        arr[i].packed = y.data_ptr()
        arr[i].row_bytes = x[0, 0].numel() * x.element_size()
    return arr


def unpad(padded: Sequence[torch.Tensor], indices: torch.Tensor, cu_seqlens: torch.Tensor,
          packed_rows: Optional[int] = None):
    """Gather the real tokens of padded [batch, seqlen, ...] tensors into packed [rows, ...] ones.

    Rows past cu_seqlens[-1] of the outputs are left unwritten; ``packed_rows`` defaults
    to batch * seqlen (pass the known total to get exact-size outputs).
    """
    lib = _lib.load()
    padded = list(padded)
    batch, seqlen = padded[0].shape[:2]
    rows = batch * seqlen if packed_rows is None else int(packed_rows)
    packed = [torch.empty((rows,) + tuple(x.shape[2:]), dtype=x.dtype, device=x.device) for x in padded]
    arr = _pack_tensors(padded, packed, batch, seqlen)
    _need_dev("indices", indices, padded[0].device)
    _need_dev("cu_seqlens", cu_seqlens, padded[0].device)
    _raise(lib.va_unpad(arr, len(padded), indices.data_ptr(), cu_seqlens.data_ptr(), batch, seqlen, rows,
                        _stream(padded[0].device)), lib)
    return packed


def pad(packed: Sequence[torch.Tensor], inverse: torch.Tensor, batch: int, seqlen: int):
    """Scatter packed [rows, ...] tensors back to padded [batch, seqlen, ...] ones (zeros elsewhere)."""
    lib = _lib.load()
    packed = list(packed)
    padded = [torch.empty((batch, seqlen) + tuple(y.shape[1:]), dtype=y.dtype, device=y.device)
              for y in packed]
    arr = _pack_tensors(padded, packed, batch, seqlen)
    _need_dev("inverse", inverse, packed[0].device)
    _raise(lib.va_pad(arr, len(packed), inverse.data_ptr(), batch, seqlen, packed[0].shape[0],
                      _stream(packed[0].device)), lib)
    return padded
