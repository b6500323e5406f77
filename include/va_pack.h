/*
 * va_pack.h -- the steps on either side of the packed attention path: packing
 * metadata from a padding mask, and the gather (unpad) / scatter (pad) between
 * the padded [batch, seqlen, ...] layout and the packed [total, ...] stream
 * that va_varlen_fwd / va_varlen_bwd read (include/va_varlen.h).
 *
 * What is computed.  The TorchEasyRec pull request 663 page (intro) packs
 * every row into one stream with explicit cumulative boundaries and per-row
 * position ids; the FDMA pull request 118 page (section "Key Implementation
 * Points", "Variable Length Flow") unpads Q, K and V before the kernel with
 * one shared indexing pass and pads the output back.  For a padding mask
 * M [batch, seqlen] (nonzero byte = a real token), row b keeps the positions
 * s with M[b][s] != 0 in increasing order:
 *
 *     cu_seqlens[0] = 0,  cu_seqlens[b + 1] = cu_seqlens[b] + L_b
 *     max_seqlen    = max_b L_b
 *     indices[t]    = b * seqlen + s of the t-th kept token (rows in order)
 *     position_ids[t] = rank of that token inside its row (0 .. L_b - 1)
 *     inverse[b * seqlen + s] = its packed index t, or -1 for padding
 *     unpad:  packed[t] = padded[indices[t]]            for t < cu_seqlens[batch]
 *     pad:    padded[p] = packed[inverse[p]], or zeros  for every p
 *
 * All integer and byte work: results are exact and deterministic.  The mask
 * need not be left- or right-aligned.  The library never reads device memory
 * on the host, so the packed total is only known on the device
 * (cu_seqlens[batch]); a caller sizes packed buffers by batch * seqlen, or
 * reads the total itself.
 *
 * Ownership, streams and errors as in va_varlen.h: the caller owns every
 * buffer (device memory), each call only enqueues kernels on `stream`, and a
 * non-VA_OK return means nothing was enqueued (message in va_last_error()).
 */
#ifndef VA_PACK_H
#define VA_PACK_H

#include "va_varlen.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Packing metadata of a padding mask.
 *   mask           device uint8 [batch][seqlen], row-major
 *   cu_seqlens     device int32 [batch + 1]            (written)
 *   max_seqlen     device int32 [1]                    (written)
 *   indices        device int32 [batch * seqlen]; entries t < total written
 *   position_ids   device int32 [batch * seqlen]; entries t < total written
 *   inverse        device int32 [batch * seqlen]       (every entry written)
 * Three kernels: row lengths, their running sum, then each row's ranks.
 * Returns VA_ERR_INVALID for a NULL pointer, batch or seqlen <= 0, or
 * batch * seqlen >= 2^31; VA_ERR_HIP if a launch fails.
 */
va_status va_pack_metadata(const uint8_t* mask, int32_t batch, int32_t seqlen,
                           int32_t* cu_seqlens, int32_t* max_seqlen,
                           int32_t* indices, int32_t* position_ids, int32_t* inverse,
                           va_stream stream);

/* One tensor of an unpad / pad call: row r is row_bytes bytes at base + r * row_bytes. */
typedef struct {
  void* padded;       /* [batch * seqlen] rows, device */
  void* packed;       /* [packed_rows] rows, device */
  int64_t row_bytes;  /* bytes of one token row, e.g. heads * head_dim * element size */
} va_pack_tensor;

#define VA_PACK_MAX_TENSORS 4

/*
 * Unpad (gather): for t < min(cu_seqlens[batch], packed_rows), packed row t of
 * every tensor = padded row indices[t] (indices clamped into the padded rows).
 * Rows of the packed buffers at or past the total are not written.  Up to
 * VA_PACK_MAX_TENSORS tensors share one launch and one read of each index
 * (Q, K and V together, as the FDMA page's fused unpad does).
 * Returns VA_ERR_INVALID for a NULL pointer, n_tensors outside
 * 1..VA_PACK_MAX_TENSORS, row_bytes <= 0, batch/seqlen <= 0,
 * batch * seqlen >= 2^31 or packed_rows < 0; VA_ERR_HIP if the launch fails.
 */
va_status va_unpad(const va_pack_tensor* tensors, int32_t n_tensors,
                   const int32_t* indices, const int32_t* cu_seqlens,
                   int32_t batch, int32_t seqlen, int64_t packed_rows, va_stream stream);

/*
 * Pad (scatter): every padded row p of every tensor = packed row inverse[p]
 * when 0 <= inverse[p] < packed_rows, else zeros.  Errors as for va_unpad.
 */
va_status va_pad(const va_pack_tensor* tensors, int32_t n_tensors, const int32_t* inverse,
                 int32_t batch, int32_t seqlen, int64_t packed_rows, va_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* VA_PACK_H */
