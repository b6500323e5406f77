"""Packed variable-length attention on MI355X: Python binding over libva_varlen.so.

Argument marshalling only.  Every step of the computation runs in the HIP
kernels behind the C ABI (include/va_varlen.h); PyTorch supplies device
memory and the current stream.  There is no CPU or PyTorch fallback: if the
library is missing, calls raise.

    out, lse = va_varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                             softmax_scale, causal, bias=None, bias_stride=None)
    dq, dk, dv = va_varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, ...)
    out = varlen_attn(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, ...)
    out, lse = kvcache_fwd(q, k_cache, v_cache, cu_seqlens_q, seqlens_k, block_table, ...)

Layouts: q/out [total_q, Hq, d], k/v [total_k, Hkv, d], lse [Hq, total_q]
float32, cu_seqlens int32 [batch + 1] on the device, bias a device tensor of
the input dtype read at element offset b*s0 + h*s1 + r*s2 + c*s3 with
``bias_stride = (s0, s1, s2, s3)`` (default: the tensor's own strides when
it is 4-D ``[batch, Hq, rows, cols]``; a per-key bias is rows stride 0).
"""

from .api import (  # noqa: F401
    VaError,
    kvcache_fwd,
    kvcache_fwd_workspace_size,
    pack_metadata,
    pad,
    unpad,
    va_varlen_bwd,
    va_varlen_bwd_workspace_size,
    va_varlen_fwd,
    va_varlen_fwd_workspace_size,
    va_last_error,
    va_status_string,
    va_timing_start,
    va_timing_stop,
    va_version,
    varlen_attn,
)
