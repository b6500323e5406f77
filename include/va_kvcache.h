/*
 * va_kvcache.h -- decode steps: attention of the few new query tokens of each
 * sequence against the sequence's paged KV cache.
 *
 * What is computed.  The noether pull request 236 page (section "module")
 * lists flash_attn_with_kvcache, FlashAttention's cached-decode call, among
 * the attention functions its code base needs; the TorchEasyRec pull request
 * 663 page (section "Test plan") covers ragged beam decoding; the
 * flash-sparse-attention pull request 118 page (section "Key Implementation
 * Points") notes that a single-token decode step needs no causal mask.  The
 * cache layout is that call's paged layout:
 *
 *   k_cache, v_cache   [num_pages][page_size][Hkv][d], row-major, dtype
 *   block_table        int32 [batch][block_table_stride]: key j of sequence b
 *                      is slot j % page_size of page block_table[b][j / page_size]
 *   seqlens_k          int32 [batch]: cached keys of each sequence (the new
 *                      tokens' own keys included, if the caller appended them)
 *   q                  [total_q][Hq][d] packed new tokens, cu_seqlens_q [batch+1]
 *
 * and the result is the packed forward of include/va_varlen.h over each
 * sequence's cached keys: O [total_q][Hq][d] in dtype, LSE [Hq][total_q]
 * float32 (natural log); with causal = 1 the mask is bottom-right aligned
 * (new token i of Lq sees keys j <= i + Lk - Lq, so a single new token sees
 * every key); a row that sees no key (an empty cache) gets O = 0 and
 * LSE = -inf.  Query head h reads KV head h / (Hq / Hkv).
 *
 * How.  One wave per (sequence, KV head, block of up to 32 rows of (new
 * token, query head), chunk of keys): every K/V byte of a KV head is read
 * once per row block for all the query heads of its group; long caches are
 * split over chunks whose partial results a last kernel merges in chunk order
 * (deterministic).  A first one-workgroup kernel lists the (sequence, row
 * block, chunk) triples that have work, from the true lengths.  The step is
 * bound by HBM bandwidth (K and V read once).
 *
 * Memory safety against bad metadata: a sequence's length is clamped to
 * [0, min(max_seqlen_k, block_table_stride * page_size)], page indices to
 * [0, num_pages), and keys past a chunk's end are never loaded.  Such input
 * gives undefined values but no access outside the buffers.  Entries of the
 * block table past a sequence's last page are never read.
 *
 * Ownership, streams and errors as in va_varlen.h: the caller owns every
 * buffer (device memory, 16-byte aligned for q, caches and out), the call
 * only enqueues kernels on `stream`, reads no device memory on the host, and
 * a non-VA_OK return means nothing was enqueued (message in va_last_error()).
 */
#ifndef VA_KVCACHE_H
#define VA_KVCACHE_H

#include "va_varlen.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Bytes of device workspace va_kvcache_fwd needs: the work list (a planner
 * kernel lists the (sequence, row block, key chunk) triples that have work,
 * so the waves share them evenly) and, when caches can be longer than one
 * chunk, float32 partial results.  The split of long caches into chunks, and so this size,
 * depends only on these arguments.  Returns 0 for arguments the call would
 * reject.
 */
size_t va_kvcache_fwd_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                     va_dtype dtype);

/*
 * Decode-step attention against a paged cache (layout above).
 *   max_seqlen_q      >= every Lq (a bound; sizes the row blocks and the work
 *                     list: rows of a longer sequence past the list are not
 *                     computed), > 0
 *   max_seqlen_k      >= every seqlens_k[b] (a bound; sizes the chunks), >= 0
 *   block_table_stride int32 entries per block-table row; must cover
 *                     max_seqlen_k: stride * page_size >= max_seqlen_k
 *   page_size         a power of two, 1 .. 2^20;  num_pages > 0
 *   dtype             VA_BF16, VA_F16 or VA_F32 (q, the caches and out all of it; float32
 *                     runs on the float32 MFMA); head_dim 32, 64, 96 or 128
 *   workspace         device memory, 256-byte aligned, of at least the size above
 * Returns VA_ERR_INVALID for a NULL required pointer, a misaligned buffer,
 * a non-positive size, Hq % Hkv != 0, a bad page_size / num_pages / stride,
 * a non-finite or non-positive scale, causal not 0/1; VA_ERR_UNSUPPORTED for
 * the dtype or head_dim, or max_seqlen_q * Hq * head_dim * element size >= 2^31;
 * VA_ERR_WORKSPACE if workspace_bytes is below the size above; VA_ERR_HIP if
 * a launch fails.
 */
va_status va_kvcache_fwd(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                         const int32_t* block_table, int32_t block_table_stride,
                         int32_t page_size, int32_t num_pages,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                         int causal, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, int32_t batch, int32_t total_q,
                         int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                         va_dtype dtype, va_stream stream);

#ifdef __cplusplus
}
#endif

#endif /* VA_KVCACHE_H */
