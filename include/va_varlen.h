/*
 * va_varlen.h -- exact scaled-dot-product attention over packed variable-length
 * sequences on AMD Instinct MI355X (gfx950).  Plain C ABI: no C++ or PyTorch
 * types cross it, so a caller needs neither libtorch nor a matching compiler.
 *
 * What is computed.  Sequences are concatenated into one token stream; the
 * boundaries of sequence b are rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of
 * Q (and of O) and rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1 of K and V
 * (the FlashAttention-2 varlen layout on the TorchEasyRec pull request 663
 * page: one packed stream with explicit cumulative boundaries).  For every
 * sequence b, query head h and KV head g = h / (num_heads_q / num_heads_kv)
 * (contiguous GQA/MQA groups):
 *
 *     S   = softmax_scale * Q_bh K_bg^T + Bias_bh
 *     S[i][j] = -inf   if causal and j > i + (Lk_b - Lq_b)    (bottom-right)
 *     O_bh = softmax(S) V_bg,    LSE_bh[i] = ln sum_j exp(S[i][j])
 *
 * A query row that sees no key (causal with Lq_b > Lk_b, or Lk_b = 0) gets
 * O = 0 and LSE = -inf.  With Lq_b = 1 causal equals non-causal, as the FDMA
 * pull request 118 page notes for single-token decode (section "Key
 * Implementation Points").  No dropout (that page assumes dropout 0).
 *
 * Layouts (row-major; heads and head_dim elements dense):
 *   q                   [total_q, num_heads_q, head_dim], token stride qkv_row_stride[0]
 *   k, v                [total_k, num_heads_kv, head_dim], token strides qkv_row_stride[1], [2]
 *   out, dout, dq       [total_q, num_heads_q, head_dim], contiguous
 *   dk, dv              [total_k, num_heads_kv, head_dim], contiguous
 *   qkv_row_stride      optional HOST int64[3]: elements from one token's row
 *                       of q (k, v) to the next; NULL = contiguous (num_heads
 *                       * head_dim).  Each must be >= num_heads * head_dim and
 *                       keep rows 16-byte aligned (q, k, v bases too), so the
 *                       Q, K and V slices of one fused projection output
 *                       [total, (Hq + 2 Hkv) * head_dim] -- the QKV-packed
 *                       input of the flash_attn_qkvpacked_func call the noether
 *                       pull request 236 page lists (section "module") -- are
 *                       read in place, without a copy.
 *   lse                 [num_heads_q, total_q]  float32, natural log
 *   cu_seqlens_q/_k     [batch + 1] int32, device memory, cu[0] = 0,
 *                       non-decreasing, cu[batch] = total_q / total_k
 *   bias                optional; element (b, h, r, c) -- r, c local to the
 *                       sequence -- at bias[b*s0 + h*s1 + r*s2 + c*s3], with
 *                       bias_stride = {s0, s1, s2, s3} a HOST int64[4] of
 *                       element strides >= 0.  A per-key bias is s2 = 0; a
 *                       head-shared bias is s1 = 0; any permuted view is just
 *                       other strides.  This is the strided per-sequence view of
 *                       the GiGL pull request 858 page (section "Approach": the
 *                       bias of sequence i sits at i * stride(0)).  The bias has
 *                       the input dtype, is added after scaling, and only
 *                       elements with r < Lq_b and c < Lk_b are ever read.
 *
 * Ownership and synchronisation.  The caller allocates every buffer, inputs,
 * outputs and workspace, in device memory (except bias_stride, on the host).
 * The library allocates nothing per call, frees nothing, never reads device
 * memory on the host and never synchronises: each call only enqueues kernels
 * on `stream` and returns (the per-step host sync the TorchEasyRec page's
 * review flags is avoided by construction).  Outputs are fully overwritten
 * (zeros for empty rows); they are valid for later work on `stream`.
 *
 * Workspace.  Each call first runs a planner kernel that reads cu_seqlens on
 * the device and writes, into the workspace, the list of work units of each
 * pass sorted by cost, so that the persistent workgroups take the heaviest
 * units first.  A query tile that sees more than 1024 keys (a key tile seen
 * by more than 768 query-row x head pairs in the backward) is split into
 * units whose float32 partial results are merged in a fixed order.  The rule
 * depends only on the tile's own sequence, so results are deterministic and a
 * sequence's results do not depend on the other sequences of the batch --
 * unless the batch would need more partial slots than the workspace's fixed
 * budget, in which case the planner doubles the split length (up to 32x, then
 * no splitting) until they fit.  Contents need no initialisation; a workspace
 * must not be shared by calls that may overlap.
 *
 * Errors.  A non-VA_OK return means nothing was enqueued; va_last_error()
 * then holds a message for the calling thread.  Invalid device metadata
 * (cu_seqlens not monotone, cu[batch] != total, a length above max_seqlen)
 * is not detected: results are then unspecified, but every index is clamped
 * so no access leaves the buffers the other arguments describe.
 */
#ifndef VA_VARLEN_H
#define VA_VARLEN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  VA_OK = 0,
  VA_ERR_INVALID = 1,     /* null pointer, zero/negative size, Hq % Hkv != 0, bad stride */
  VA_ERR_UNSUPPORTED = 2, /* head_dim not supported, unknown dtype, bf16 grads of fp32 inputs */
  VA_ERR_WORKSPACE = 3,   /* workspace smaller than va_varlen_{fwd,bwd}_workspace_size() */
  VA_ERR_HIP = 4          /* the HIP runtime reported an error; text in va_last_error() */
} va_status;

typedef enum {
  VA_F32 = 0,  /* IEEE float32; products and sums in float32 (no reduced-precision shortcut) */
  VA_BF16 = 1, /* bfloat16 storage; matrix products on bf16 MFMA with float32 accumulation */
  VA_F16 = 2   /* float16 storage; matrix products on f16 MFMA with float32 accumulation */
} va_dtype;

/* A hipStream_t passed as an opaque pointer; NULL is the default stream. */
typedef void* va_stream;

/*
 * Forward.  Writes out [total_q, num_heads_q, head_dim] in `dtype` and lse
 * [num_heads_q, total_q] in float32.
 *   q, k, v            device, `dtype`, layouts above
 *   cu_seqlens_q/_k    device int32 [batch + 1]
 *   max_seqlen_q/_k    host upper bounds on Lq_b / Lk_b (>= 1); they size the
 *                      workspace, never the results (a bound that is too small
 *                      only disables splitting)
 *   softmax_scale      multiplies Q K^T (callers usually pass 1/sqrt(head_dim));
 *                      must be finite and > 0
 *   causal             0 or 1; 1 = bottom-right aligned causal mask
 *   bias, bias_stride  both NULL (no bias) or both non-NULL
 *   out, lse           device outputs, layouts above
 *   qkv_row_stride     NULL or HOST int64[3] token strides of q, k, v (above)
 *   workspace          device scratch of at least va_varlen_fwd_workspace_size()
 *                      bytes, 256-byte aligned
 *   head_dim           32, 64, 96, 128 or 256 (multiples of the 32-wide MFMA output tile)
 * Returns VA_ERR_INVALID for a NULL required pointer, exactly one of
 * bias/bias_stride NULL, batch/total/heads/head_dim <= 0, Hq % Hkv != 0,
 * max_seqlen <= 0, a negative stride, a scale that is not finite and > 0, a
 * misaligned workspace, a row stride below num_heads * head_dim or rows or
 * bases of q/k/v not 16-byte aligned; VA_ERR_UNSUPPORTED for head_dim not in
 * {32, 64, 96, 128, 256}, an unknown dtype, a bias view spanning 2 GiB or more inside one
 * (sequence, head), or max_seqlen * row stride reaching 2 GiB (the kernels
 * address one sequence's rows with 32-bit byte offsets); VA_ERR_WORKSPACE for
 * too small a workspace; VA_ERR_HIP if a launch fails.  A bias with
 * contiguous keys (bias_stride[3] = 1), strides that are multiples of 4 and a
 * base aligned to 4 elements is read 4 keys per load; a 16-bit one whose
 * strides are multiples of 8 and whose base is 16-byte aligned is staged
 * through LDS a block of keys at a time (results identical either way).
 * Short queries: with max_seqlen_q <= 16 (or <= 32 with
 * max_seqlen_q * num_heads_q / num_heads_kv <= 128) -- decode steps, beams and
 * drafts over contiguous K/V -- the call runs the decode kernels of
 * include/va_kvcache.h (K/V read through cu_seqlens_k; any dtype; a bias read
 * per element, or four keys at a time under the vector-load conditions above,
 * when its view over one sequence and KV group of heads spans less than 2 GiB)
 * instead of 128-row query tiles; results agree up to rounding order, and the
 * hints still only size the work.
 */
va_status va_varlen_fwd(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                        float softmax_scale, int causal,
                        const void* bias, const int64_t* bias_stride,
                        void* out, float* lse,
                        const int64_t* qkv_row_stride,
                        void* workspace, size_t workspace_bytes,
                        int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        va_dtype dtype, va_stream stream);

/*
 * Bytes of device workspace va_varlen_fwd / va_varlen_bwd need for these
 * sizes (256-byte aligned pointer required).  Return 0 for arguments the call
 * would reject.  Pure host arithmetic.
 */
size_t va_varlen_fwd_workspace_size(int32_t batch, int32_t total_q, int32_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t head_dim, va_dtype dtype);
size_t va_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv,
                                    int32_t head_dim, va_dtype dtype, va_dtype grad_dtype);

/*
 * Backward: dq, dk, dv of sum(dout * out) for the forward above, recomputing
 * the softmax from `lse` (the forward's own output) instead of storing it,
 * and optionally the bias gradient.
 *   dout, out          device, `dtype`, [total_q, num_heads_q, head_dim], contiguous
 *   q, k, v            as for the forward, with the same qkv_row_stride (passed
 *                      after the gradient outputs)
 *   lse                device float32 [num_heads_q, total_q] from va_varlen_fwd
 *   dq                 [total_q, num_heads_q, head_dim] in grad_dtype
 *   dk, dv             [total_k, num_heads_kv, head_dim] in grad_dtype; the
 *                      query heads of a GQA group are summed
 *   dbias, dbias_stride  both NULL (no bias gradient) or both non-NULL, and then
 *                      a bias is required.  The bias enters the logits additively,
 *                      so its gradient is dS = P * (dP - D) (the GiGL pull request
 *                      858 page, section "Approach", notes the varlen kernel it
 *                      calls has no such backward).  dbias is float32, written at
 *                      element b*t0 + h*t1 + r*t2 + c*t3 with dbias_stride = {t0,
 *                      t1, t2, t3} (HOST int64[4]); a stride of 0 sums over that
 *                      axis.  Supported: t0 > 0 (or batch 1) and t3 > 0;
 *                      per pair (t2 > 0): t1 > 0 (or one query head), every
 *                      element of a valid pair (r < Lq_b, c < Lk_b) written,
 *                      0 where the causal mask hides the pair; per key
 *                      (t2 = 0): summed over rows, every (b, h, c < Lk) written,
 *                      with t1 > 0 and at most 32 query heads per KV head (8 at
 *                      head_dim 256), or
 *                      t1 = 0 (summed over heads too) with one KV head.  Other
 *                      layouts return VA_ERR_UNSUPPORTED.  Typically dbias_stride
 *                      equals bias_stride of a float32 buffer shaped like the bias.
 *                      Elements no valid pair addresses (rows or keys past a
 *                      sequence's length in a padded grid) are left untouched.
 *   workspace          device scratch of at least va_varlen_bwd_workspace_size()
 *                      bytes, 256-byte aligned
 *   grad_dtype         VA_F32, or the input dtype when that is VA_BF16 or VA_F16
 * Deterministic: a call's results do not depend on scheduling (no atomics on
 * values; split tiles are summed in a fixed order).  Errors as for the forward, plus VA_ERR_WORKSPACE, and
 * VA_ERR_UNSUPPORTED for a 16-bit grad_dtype other than the input dtype.
 */
va_status va_varlen_bwd(const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k,
                        float softmax_scale, int causal,
                        const void* bias, const int64_t* bias_stride,
                        void* dq, void* dk, void* dv,
                        float* dbias, const int64_t* dbias_stride,
                        const int64_t* qkv_row_stride,
                        void* workspace, size_t workspace_bytes,
                        int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        va_dtype dtype, va_dtype grad_dtype, va_stream stream);

/*
 * One plan for a forward and its backward.  The work plans of both passes
 * depend only on cu_seqlens and the sizes (TorchEasyRec intro: one set of
 * cumulative boundaries per packed batch), so the forward's planner launch can
 * build the backward's plans as well:
 *
 * va_varlen_fwd_bwdplan: va_varlen_fwd, and in the same planner launch the
 *   dK/dV and dQ work plans of va_varlen_bwd for the same cu_seqlens and sizes,
 *   written into bwd_workspace (device memory, 256-byte aligned, at least
 *   va_varlen_bwd_workspace_size bytes for these sizes; the caller keeps it
 *   for the backward).  Results of the forward are those of va_varlen_fwd.
 *   Errors: those of va_varlen_fwd; VA_ERR_INVALID for a NULL or misaligned
 *   bwd_workspace; VA_ERR_WORKSPACE if bwd_workspace_bytes is too small.
 * va_varlen_bwd_planned: va_varlen_bwd that takes its work plans from
 *   `workspace` as the forward left them (it builds none: the preprocessing
 *   launch only computes D = rowsum(dO * O)).  The caller guarantees that the
 *   last call that wrote `workspace` was a va_varlen_fwd_bwdplan with the same
 *   cu_seqlens, max_seqlen, sizes and causal flag on the same stream (or one
 *   ordered before it); the backward consumes the plans, so each forward
 *   feeds one backward.  Results are bitwise those of va_varlen_bwd.  Errors:
 *   those of va_varlen_bwd.
 */
va_status va_varlen_fwd_bwdplan(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                float softmax_scale, int causal,
                                const void* bias, const int64_t* bias_stride,
                                void* out, float* lse,
                                const int64_t* qkv_row_stride,
                                void* workspace, size_t workspace_bytes,
                                void* bwd_workspace, size_t bwd_workspace_bytes,
                                int32_t batch, int32_t total_q, int32_t total_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                va_dtype dtype, va_stream stream);
va_status va_varlen_bwd_planned(const void* dout, const void* q, const void* k, const void* v,
                                const void* out, const float* lse,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                float softmax_scale, int causal,
                                const void* bias, const int64_t* bias_stride,
                                void* dq, void* dk, void* dv,
                                float* dbias, const int64_t* dbias_stride,
                                const int64_t* qkv_row_stride,
                                void* workspace, size_t workspace_bytes,
                                int32_t batch, int32_t total_q, int32_t total_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                va_dtype dtype, va_dtype grad_dtype, va_stream stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  The same computation and arguments as va_varlen_fwd (results
 * bitwise identical whenever both plan the same split tiles), without the
 * workspace arguments: the work plan and the partial results of split tiles
 * go to a fixed array of VA_NOALLOC_SCRATCH_BYTES in the library's own device
 * memory, one per GPU, held until the process ends.  The call allocates and
 * frees nothing.  Sizes whose work plan does not fit the array return
 * VA_ERR_WORKSPACE (use va_varlen_fwd with a workspace); when the plan fits
 * but the hints allow more split tiles than the rest of the array holds,
 * tiles are split into longer chunks (or not at all), as for a workspace
 * whose partial budget is exhausted.  Every call on one GPU shares that GPU's
 * array: calls that may overlap on one GPU (several streams or threads) race
 * and must be serialised by the caller.  Nothing in the array needs clearing
 * between calls.
 */
#define VA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)

va_status va_varlen_fwd_noalloc(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k,
                                float softmax_scale, int causal,
                                const void* bias, const int64_t* bias_stride,
                                void* out, float* lse,
                                const int64_t* qkv_row_stride,
                                int32_t batch, int32_t total_q, int32_t total_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                va_dtype dtype, va_stream stream);

/*
 * Measurement.  The metric of this library is non-padded attention TFLOP/s
 * per kernel against the MI355X roofline, so a caller can time each kernel a
 * call launches.  After va_timing_start(n), the calling thread's library
 * calls record a HIP event pair around each kernel they launch, on that
 * call's stream, for up to n launches (events are created here, not per
 * call).  va_timing_stop() waits for the recorded events, writes up to
 * max_entries per-kernel aggregates (name, launches, total milliseconds) and
 * returns how many kernels were seen (or -1 on a HIP error), then releases
 * the events.  Timing adds an event record between launches; it is off by
 * default.
 */
typedef struct {
  const char* name; /* static string naming the kernel */
  int launches;
  double total_ms;
} va_kernel_time;

va_status va_timing_start(int max_launches);
int va_timing_stop(va_kernel_time* out, int max_entries);

/* Static text for a status code (never NULL). */
const char* va_status_string(va_status s);

/* Message for the last non-VA_OK return on the calling thread ("" if none). */
const char* va_last_error(void);

/* Library version as MAJOR*10000 + MINOR*100 + PATCH. */
int va_version(void);

#ifdef __cplusplus
}
#endif

#endif /* VA_VARLEN_H */
