// C ABI of the packed varlen attention library: argument validation (host
// only, no device reads), schedule sizing and kernel launch.  Declarations
// and the contract of every entry point are in include/va_varlen.h,
// include/va_kvcache.h and include/va_pack.h.
#include "va_varlen.h"
#include "va_kvcache.h"
#include "va_pack.h"

#include <hip/hip_runtime.h>

#include <atomic>
#include <string>
#include <vector>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "va_kernels.h"

namespace {

thread_local char g_err[512] = "";

va_status fail(va_status s, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return s;
}

// Head dims of the packed forward and backward (multiples of the 32-wide
// MFMA output tile); the decode kernels take 32, 64, 96 and 128.
bool varlen_head_dim(int d) { return d == 32 || d == 64 || d == 96 || d == 128 || d == 256; }
bool decode_head_dim(int d) { return d == 32 || d == 64 || d == 96 || d == 128; }

struct Common {
  int batch, total_q, total_k, hq, hkv, d, max_q, max_k;
  int causal;
  va_dtype dtype;
};

va_status check_common(const Common& c, float scale, const void* bias, const int64_t* bstride) {
  if (c.batch <= 0) return fail(VA_ERR_INVALID, "batch must be > 0 (got %d)", c.batch);
  if (c.total_q <= 0 || c.total_k <= 0)
    return fail(VA_ERR_INVALID, "total_q and total_k must be > 0 (got %d, %d)", c.total_q, c.total_k);
  if (c.hq <= 0 || c.hkv <= 0)
    return fail(VA_ERR_INVALID, "head counts must be > 0 (got %d, %d)", c.hq, c.hkv);
  if (c.d <= 0) return fail(VA_ERR_INVALID, "head_dim must be > 0 (got %d)", c.d);
  if (c.hq % c.hkv != 0)
    return fail(VA_ERR_INVALID, "num_heads_q (%d) must be a multiple of num_heads_kv (%d)", c.hq, c.hkv);
  if (c.max_q <= 0 || c.max_k <= 0)
    return fail(VA_ERR_INVALID, "max_seqlen_q/k must be > 0 (got %d, %d)", c.max_q, c.max_k);
  if (c.causal != 0 && c.causal != 1) return fail(VA_ERR_INVALID, "causal must be 0 or 1");
  if (!(std::isfinite(scale) && scale > 0.f))
    return fail(VA_ERR_INVALID, "softmax_scale must be finite and > 0");
  if ((bias == nullptr) != (bstride == nullptr))
    return fail(VA_ERR_INVALID, "bias and bias_stride must both be NULL or both non-NULL");
  if (bstride)
    for (int i = 0; i < 4; ++i)
      if (bstride[i] < 0) return fail(VA_ERR_INVALID, "bias_stride[%d] is negative", i);
  if (c.dtype != VA_F32 && c.dtype != VA_BF16 && c.dtype != VA_F16)
    return fail(VA_ERR_UNSUPPORTED, "unknown dtype %d", (int)c.dtype);
  if (!varlen_head_dim(c.d))
    return fail(VA_ERR_UNSUPPORTED, "head_dim %d not supported (32, 64, 96, 128 or 256)", c.d);
  if ((int64_t)c.total_q * c.hq * c.d >= ((int64_t)1 << 40) ||
      (int64_t)c.total_k * c.hkv * c.d >= ((int64_t)1 << 40))
    return fail(VA_ERR_UNSUPPORTED, "tensor too large");
  return VA_OK;
}

// Token strides of q, k, v (elements): the caller's, or the contiguous ones.
// Rows are read with 16-byte loads at 32-bit byte offsets inside a sequence.
va_status row_strides(const Common& c, const void* q, const void* k, const void* v, const int64_t* rs,
                      int64_t out[3]) {
  const int64_t dense[3] = {(int64_t)c.hq * c.d, (int64_t)c.hkv * c.d, (int64_t)c.hkv * c.d};
  const int elt = c.dtype == VA_F32 ? 4 : 2;
  for (int i = 0; i < 3; ++i) {
    out[i] = rs ? rs[i] : dense[i];
    if (out[i] < dense[i])
      return fail(VA_ERR_INVALID, "qkv_row_stride[%d] = %lld is below heads * head_dim = %lld", i,
                  (long long)out[i], (long long)dense[i]);
    if ((out[i] * elt) % 16 != 0)
      return fail(VA_ERR_INVALID, "qkv_row_stride[%d] must keep rows 16-byte aligned", i);
    const int64_t rows = i == 0 ? c.max_q : c.max_k;
    if (rows * out[i] * elt >= ((int64_t)1 << 31))
      return fail(VA_ERR_UNSUPPORTED, "max_seqlen * qkv_row_stride[%d] spans 2 GiB or more", i);
  }
  if ((((uintptr_t)q) | ((uintptr_t)k) | ((uintptr_t)v)) % 16 != 0)
    return fail(VA_ERR_INVALID, "q, k and v must be 16-byte aligned");
  return VA_OK;
}

// ---------------------------------------------------------------------------
// Workspace.  Every pass gets a work plan (a header, the unit list and the
// split-tile list) and, when some tile can be split, float32 partial-result
// slots.  Sizes are bounds from host arguments only: at most total/tile +
// batch tiles (each sequence adds at most one ragged tile), and a tile of
// s steps splits into ceil(s / chunk) units.  Partial slots are capped by a
// byte budget; a batch that would need more is planned without splitting.
// ---------------------------------------------------------------------------
constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

constexpr int kChunkKeys = 2048;      // forward / dQ: most keys per unit
constexpr int kDkdvUnitRows = 1536;   // dK/dV: most (query row, head) pairs per unit
constexpr size_t kFwdPartBudget = (size_t)64 << 20;
constexpr size_t kDkdvPartBudget = (size_t)128 << 20;
constexpr size_t kDqPartBudget = (size_t)64 << 20;

struct PlanLayout {
  int unit_cap = 0, slot_cap = 0, split_cap = 0, chunk = 1;
  int heads = 0;           // work items per unit, each with its own count of chunks left
  size_t plan_bytes = 0;   // header + lists
  size_t slot_bytes = 0;   // bytes of one partial slot
};

PlanLayout plan_layout(int total_t, int batch, int tile, int max_other, int step, int chunk,
                       size_t slot_bytes, size_t budget, int heads) {
  PlanLayout L;
  L.heads = heads;
  const int64_t tiles = (int64_t)total_t / tile + batch;
  const int64_t max_steps = ((int64_t)max_other + step - 1) / step;
  int64_t slots = 0;
  if (max_steps > chunk) {
    slots = tiles * ((max_steps + chunk - 1) / chunk);
    const int64_t cap = (int64_t)(budget / slot_bytes);
    if (slots > cap) slots = cap;
    if (slots < 2) slots = 0;
  }
  L.slot_cap = (int)slots;
  L.split_cap = (int)(slots / 2);
  L.unit_cap = (int)(tiles + slots);
  L.chunk = chunk;
  L.slot_bytes = slot_bytes;
  L.plan_bytes = round_up(256) + 2 * round_up((size_t)L.unit_cap * 16) + 2 * round_up((size_t)L.unit_cap * 4) +
                 round_up((size_t)(L.split_cap > 0 ? L.split_cap : 1) * 16) +
                 round_up((size_t)(L.split_cap > 0 ? L.split_cap : 1) * heads * 4);
  return L;
}

// Carves a plan out of the workspace at `p`; returns the bytes used.
size_t carve_plan(char* p, const PlanLayout& L, va::Plan& plan) {
  plan.hdr = (int*)p;
  size_t o = round_up(256);
  plan.units = (int4*)(p + o);
  o += round_up((size_t)L.unit_cap * 16);
  plan.bounds = (int4*)(p + o);
  o += round_up((size_t)L.unit_cap * 16);
  plan.slots = (int*)(p + o);
  o += round_up((size_t)L.unit_cap * 4);
  plan.sidx = (int*)(p + o);
  o += round_up((size_t)L.unit_cap * 4);
  plan.splits = (int4*)(p + o);
  o += round_up((size_t)(L.split_cap > 0 ? L.split_cap : 1) * 16);
  plan.left = (int*)(p + o);
  o += round_up((size_t)(L.split_cap > 0 ? L.split_cap : 1) * L.heads * 4);
  return o;
}

va::PlanArgs plan_args(const va::Plan& plan, const PlanLayout& L, const int32_t* cu_t,
                       const int32_t* cu_o, int total_t, int total_o, int batch, int tile,
                       int step, int kside, int causal) {
  va::PlanArgs a{};
  a.plan = plan;
  a.cu_t = cu_t; a.cu_o = cu_o;
  a.total_t = total_t; a.total_o = total_o; a.batch = batch;
  a.tile = tile; a.step = step; a.kside = kside; a.causal = causal;
  a.chunk = L.chunk;
  a.unit_cap = L.unit_cap; a.slot_cap = L.slot_cap; a.split_cap = L.split_cap;
  a.heads = L.heads;
  return a;
}

// budget: bytes the partial results of split tiles may take
PlanLayout fwd_plan(int batch, int total_q, int max_k, int hq, int d, bool bf16, size_t budget) {
  const int bm = va::fwd_block_m(), bn = va::fwd_block_n(bf16, d);
  return plan_layout(total_q, batch, bm, max_k, bn, kChunkKeys / bn,
                     (size_t)hq * bm * (d + 1) * sizeof(float), budget, hq);
}

size_t fwd_workspace(int batch, int total_q, int max_k, int hq, int d, bool bf16, size_t budget) {
  const PlanLayout L = fwd_plan(batch, total_q, max_k, hq, d, bf16, budget);
  return L.plan_bytes + round_up(L.slot_bytes * L.slot_cap);
}

PlanLayout dkdv_plan(int batch, int total_k, int max_q, int hkv, int n_rep, int d) {
  const int bnk = va::bwd_block_k(), bmq = va::bwd_dkdv_block_q();
  int chunk = kDkdvUnitRows / (bmq * n_rep);
  if (chunk < 1) chunk = 1;
  // (its split tiles are merged by the dQ pass after the dK/dV pass: no counts)
  return plan_layout(total_k, batch, bnk, max_q, bmq, chunk,
                     (size_t)hkv * 2 * bnk * d * sizeof(float), kDkdvPartBudget, 0);
}

PlanLayout dq_plan(int batch, int total_q, int max_k, int hq, int d, bool bf16) {
  const int bm = va::bwd_block_q(), bn = va::bwd_dq_block_n(bf16, d);
  return plan_layout(total_q, batch, bm, max_k, bn, kChunkKeys / bn,
                     (size_t)hq * bm * d * sizeof(float), kDqPartBudget, hq);
}

// per-key bias-gradient sums of one dK/dV partial slot: [Hkv][n_rep][128 keys] floats
size_t dbias_slot_bytes(int hq) { return (size_t)hq * va::bwd_block_k() * sizeof(float); }

size_t bwd_workspace(int batch, int total_q, int total_k, int max_q, int max_k, int hq, int hkv,
                     int d, bool bf16) {
  const PlanLayout K = dkdv_plan(batch, total_k, max_q, hkv, hq / hkv, d);
  const PlanLayout Q = dq_plan(batch, total_q, max_k, hq, d, bf16);
  return round_up((size_t)hq * total_q * sizeof(float)) + K.plan_bytes + Q.plan_bytes +
         round_up(K.slot_bytes * K.slot_cap) + round_up(Q.slot_bytes * Q.slot_cap) +
         round_up(dbias_slot_bytes(hq) * K.slot_cap);
}

// The backward's two work plans inside its workspace, at the places va_varlen_bwd
// uses (after the D buffer): the dK/dV plan over key tiles, then the dQ plan.
struct BwdPlans {
  PlanLayout K, Q;
  va::Plan pk, pq;
  size_t end = 0;  // bytes from the workspace start to the end of the plans
};
BwdPlans bwd_plans(char* w, int batch, int total_q, int total_k, int max_q, int max_k, int hq, int hkv, int d,
                   bool bf16) {
  BwdPlans r;
  r.K = dkdv_plan(batch, total_k, max_q, hkv, hq / hkv, d);
  r.Q = dq_plan(batch, total_q, max_k, hq, d, bf16);
  size_t o = round_up((size_t)hq * total_q * sizeof(float));
  o += carve_plan(w + o, r.K, r.pk);
  o += carve_plan(w + o, r.Q, r.pq);
  r.end = o;
  return r;
}

// Decode steps: row blocks of `rows` = min(32, n_rep * max_seqlen_q) (new
// token, query head) pairs, and key chunks sized so the grid holds about
// kKvWaves waves (at least 256 keys per chunk, so the partial results of a
// chunk stay a few percent of the K/V bytes it reads).  The planner lists the
// (sequence, row block, chunk) triples with work; `cap` bounds that list:
// from max_seqlen_q when it is a bound the caller promises (paged caches),
// from total_q when it is only a hint (the packed forward's short-query path).
constexpr int64_t kKvWaves = 8192;
struct KvLayout {
  int rows = 1, chunk = 1, nchunk = 1, cap = 1, cap_merge = 0;
  size_t plan_bytes = 0, part_o_bytes = 0, part_lse_bytes = 0;
  size_t total() const { return plan_bytes + part_o_bytes + part_lse_bytes; }
};
KvLayout kv_layout(int batch, int max_q, int max_k, int hq, int hkv, int d, int64_t total_q = -1) {
  KvLayout L;
  const int n_rep = hq / hkv;
  const int64_t R = (int64_t)max_q * n_rep;
  L.rows = (int)(R < 32 ? R : 32);
  const int64_t rb_hint = (R + L.rows - 1) / L.rows;  // row blocks of a sequence at the hint
  const int kb = va::kv_block_n(d);
  const int64_t blocks = (int64_t)batch * hkv * rb_hint;
  const int64_t want = (kKvWaves + blocks - 1) / blocks;  // chunks wanted per row block
  const int64_t steps = ((int64_t)max_k + kb - 1) / kb;
  int64_t cs = (steps + want - 1) / want;
  if (cs < 256 / kb) cs = 256 / kb;
  L.chunk = (int)(cs * kb);
  L.nchunk = (int)(((int64_t)max_k + L.chunk - 1) / L.chunk);
  if (L.nchunk < 1) L.nchunk = 1;
  const int64_t row_blocks = total_q < 0 ? (int64_t)batch * rb_hint
                                         : (total_q * n_rep + L.rows - 1) / L.rows + batch;
  L.cap = (int)(row_blocks * L.nchunk);
  L.cap_merge = L.nchunk > 1 ? L.cap / 2 : 0;  // a merged row block has >= 2 entries
  L.plan_bytes = round_up(256) + round_up((size_t)L.cap * sizeof(va::KvChunk)) +
                 round_up((size_t)(L.cap_merge > 0 ? L.cap_merge : 1) * sizeof(int32_t));
  if (L.nchunk > 1) {
    const size_t slots = (size_t)L.cap * hkv;
    L.part_o_bytes = round_up(slots * L.rows * d * sizeof(float));
    L.part_lse_bytes = round_up(slots * L.rows * sizeof(float));
  }
  return L;
}

// The packed forward's short-query path: without a bias and with
// few new tokens per sequence (by the max_seqlen_q hint) -- decode steps,
// beams, drafts, short chunks over contiguous K/V -- the decode kernels run
// instead of 128-row query tiles, which such rows would mostly leave empty.
// Measured on MI355X (one call, 64 sequences of 2,048-4,096 keys): 16 tokens
// x 8 query heads per KV head 64 against 112 us, 8 x 16 199 against 738 us,
// 32 x 4 106 against 118 us; the tiles win from 48 tokens (41 against 48 us)
// and at 64 x 2 (129 against 194 us).  Hence: at most 16 tokens, or at most
// 32 with at most 128 (token, head) rows per KV head.  The decode kernels read
// K/V through cu_seqlens_k and the token strides; every result is the same up
// to rounding order, and sequences longer than the hints still get every row
// and key (more row blocks, longer chunks).
constexpr int kShortQueryTokens = 16, kShortQueryTokensMax = 32;
constexpr int64_t kShortQueryRows = 128;
bool short_query(va_dtype dtype, int d, int max_q, int n_rep) {
  (void)dtype;  // 16-bit and float32 alike (float32 runs the float32 decode kernel)
  return decode_head_dim(d) &&
         (max_q <= kShortQueryTokens ||
          (max_q <= kShortQueryTokensMax && (int64_t)max_q * n_rep <= kShortQueryRows));
}

bool kv_args_ok(int32_t batch, int32_t max_q, int32_t max_k, int32_t hq, int32_t hkv, int32_t d,
                va_dtype dtype) {
  return batch > 0 && max_q > 0 && max_k >= 0 && hq > 0 && hkv > 0 && hq % hkv == 0 &&
         decode_head_dim(d) && (dtype == VA_BF16 || dtype == VA_F16 || dtype == VA_F32) &&
         (int64_t)max_q * hq * d * (dtype == VA_F32 ? 4 : 2) < ((int64_t)1 << 31);
}

// kernel element code: 0 float32, 1 bfloat16, 2 float16
int elem_code(va_dtype t) { return t == VA_BF16 ? 1 : (t == VA_F16 ? 2 : 0); }

va_status hip_fail(hipError_t e, const char* what) {
  return fail(VA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

extern "C" {

int va_version(void) { return 1 * 10000 + 0 * 100 + 0; }

const char* va_status_string(va_status s) {
  switch (s) {
    case VA_OK: return "ok";
    case VA_ERR_INVALID: return "invalid argument";
    case VA_ERR_UNSUPPORTED: return "unsupported argument";
    case VA_ERR_WORKSPACE: return "workspace too small";
    case VA_ERR_HIP: return "HIP runtime error";
  }
  return "unknown status";
}

const char* va_last_error(void) { return g_err; }

size_t va_varlen_fwd_workspace_size(int32_t batch, int32_t total_q, int32_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    va_dtype dtype) {
  return va::varlen_fwd_need(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                             head_dim, dtype, kFwdPartBudget);
}

va_status va_varlen_fwd(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                        int causal, const void* bias, const int64_t* bias_stride, void* out,
                        float* lse, const int64_t* qkv_row_stride, void* workspace,
                        size_t workspace_bytes, int32_t batch,
                        int32_t total_q, int32_t total_k, int32_t num_heads_q,
                        int32_t num_heads_kv, int32_t head_dim, va_dtype dtype,
                        va_stream stream) {
  return va::varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                        bias, bias_stride, out, lse, qkv_row_stride, workspace, workspace_bytes, kFwdPartBudget,
                        batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, dtype, stream);
}

va_status va_varlen_fwd_bwdplan(const void* q, const void* k, const void* v,
                                const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                int causal, const void* bias, const int64_t* bias_stride, void* out,
                                float* lse, const int64_t* qkv_row_stride, void* workspace,
                                size_t workspace_bytes, void* bwd_workspace, size_t bwd_workspace_bytes,
                                int32_t batch, int32_t total_q, int32_t total_k, int32_t num_heads_q,
                                int32_t num_heads_kv, int32_t head_dim, va_dtype dtype, va_stream stream) {
  if (!bwd_workspace) {
    g_err[0] = 0;
    return fail(VA_ERR_INVALID, "bwd_workspace is NULL");
  }
  return va::varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                        bias, bias_stride, out, lse, qkv_row_stride, workspace, workspace_bytes, kFwdPartBudget,
                        batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, dtype, stream,
                        bwd_workspace, bwd_workspace_bytes);
}

}  // extern "C"

namespace va {

void set_error(const char* msg) { snprintf(g_err, sizeof(g_err), "%s", msg); }

size_t varlen_fwd_need(int32_t batch, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                       va_dtype dtype, size_t part_budget) {
  if (batch <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 ||
      num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0 ||
      !varlen_head_dim(head_dim) || (dtype != VA_F32 && dtype != VA_BF16 && dtype != VA_F16))
    return 0;
  size_t n = fwd_workspace(batch, total_q, max_seqlen_k, num_heads_q, head_dim, dtype != VA_F32, part_budget);
  if (short_query(dtype, head_dim, max_seqlen_q, num_heads_q / num_heads_kv)) {
    const size_t m = kv_layout(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                               total_q).total();
    if (m > n) n = m;
  }
  return n;
}

va_status varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                     float softmax_scale, int causal, const void* bias, const int64_t* bias_stride, void* out,
                     float* lse, const int64_t* qkv_row_stride, void* workspace, size_t workspace_bytes,
                     size_t part_budget, int32_t batch, int32_t total_q, int32_t total_k, int32_t num_heads_q,
                     int32_t num_heads_kv, int32_t head_dim, va_dtype dtype, va_stream stream,
                     void* bwd_ws, size_t bwd_ws_bytes) {
  g_err[0] = 0;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out || !lse)
    return fail(VA_ERR_INVALID, "a required pointer is NULL");
  Common c{batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, max_seqlen_q,
           max_seqlen_k, causal, dtype};
  va_status s = check_common(c, softmax_scale, bias, bias_stride);
  if (s != VA_OK) return s;
  int64_t rs[3];
  s = row_strides(c, q, k, v, qkv_row_stride, rs);
  if (s != VA_OK) return s;
  if (!workspace) return fail(VA_ERR_INVALID, "workspace is NULL");
  if (((uintptr_t)workspace) % kAlign != 0)
    return fail(VA_ERR_INVALID, "workspace must be 256-byte aligned");
  const bool bf16 = dtype != VA_F32;  // a 16-bit kind (bf16 or f16)
  const size_t need = fwd_workspace(batch, total_q, max_seqlen_k, num_heads_q, head_dim, bf16, part_budget);
  if (workspace_bytes < need)
    return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  // the backward's plans, built by this call's planner launch (va_varlen_fwd_bwdplan)
  va::PlanArgs bwd_pk{}, bwd_pq{};
  if (bwd_ws) {
    if (((uintptr_t)bwd_ws) % kAlign != 0)
      return fail(VA_ERR_INVALID, "bwd_workspace must be 256-byte aligned");
    const size_t bneed = bwd_workspace(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                                       num_heads_kv, head_dim, bf16);
    if (bwd_ws_bytes < bneed)
      return fail(VA_ERR_WORKSPACE, "bwd_workspace of %zu bytes < %zu required", bwd_ws_bytes, bneed);
    const BwdPlans B = bwd_plans((char*)bwd_ws, batch, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                 num_heads_q, num_heads_kv, head_dim, bf16);
    bwd_pk = plan_args(B.pk, B.K, cu_seqlens_k, cu_seqlens_q, total_k, total_q, batch, va::bwd_block_k(),
                       va::bwd_dkdv_block_q(), 1, causal);
    bwd_pq = plan_args(B.pq, B.Q, cu_seqlens_q, cu_seqlens_k, total_q, total_k, batch, va::bwd_block_q(),
                       va::bwd_dq_block_n(bf16, head_dim), 0, causal);
  }

  hipStream_t st = (hipStream_t)stream;
  // a bias reaches the decode kernels through one resource per (sequence, KV group):
  // every offset inside it must be a 32-bit byte offset
  bool short_bias_ok = true;
  if (bias) {
    const int64_t elt = bf16 ? 2 : 4;
    const int64_t span = ((int64_t)(num_heads_q / num_heads_kv - 1) * bias_stride[1] +
                          (int64_t)max_seqlen_q * bias_stride[2] + ((int64_t)max_seqlen_k + 64) * bias_stride[3] + 8) *
                         elt;
    short_bias_ok = bias_stride[0] >= 0 && bias_stride[1] >= 0 && bias_stride[2] >= 0 && bias_stride[3] >= 0 &&
                    span < ((int64_t)1 << 31);
  }
  if (short_bias_ok && short_query(dtype, head_dim, max_seqlen_q, num_heads_q / num_heads_kv)) {
    const KvLayout L = kv_layout(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim,
                                 total_q);
    if (workspace_bytes < L.total())
      return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, L.total());
    va::KvArgs a{};
    a.q = q; a.k_cache = k; a.v_cache = v;
    a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
    a.q_rs = rs[0]; a.k_rs = rs[1]; a.v_rs = rs[2];
    a.total_k = total_k;
    a.out = out; a.lse = lse;
    char* w = (char*)workspace;
    a.plan = (int32_t*)w;
    a.chunks = (va::KvChunk*)(w + round_up(256));
    a.merges = (int32_t*)(w + round_up(256) + round_up((size_t)L.cap * sizeof(va::KvChunk)));
    a.part_o = L.part_o_bytes > 0 ? (float*)(w + L.plan_bytes) : nullptr;
    a.part_lse = L.part_lse_bytes > 0 ? (float*)(w + L.plan_bytes + L.part_o_bytes) : nullptr;
    a.batch = batch; a.total_q = total_q;
    a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = num_heads_q / num_heads_kv; a.d = head_dim;
    a.num_pages = 1;
    a.max_k = max_seqlen_k;
    a.rows = L.rows; a.chunk = L.chunk; a.nchunk = L.nchunk; a.cap = L.cap; a.cap_merge = L.cap_merge;
    a.scale_log2 = softmax_scale * 1.4426950408889634f;
    a.causal = causal;
    a.h16 = elem_code(dtype);
    if (bias) {
      const int elt = bf16 ? 2 : 4;
      a.bias = bias;
      a.bs0 = bias_stride[0]; a.bs1 = bias_stride[1]; a.bs2 = bias_stride[2]; a.bs3 = bias_stride[3];
      // four keys per load: contiguous keys, every 4-key group aligned to its own size
      a.bias_vec = a.bs3 == 1 && a.bs0 % 4 == 0 && a.bs1 % 4 == 0 && a.bs2 % 4 == 0 &&
                   ((uintptr_t)bias) % (4 * elt) == 0;
    }
    if (bwd_ws) {
      va::PlanSet pb{};
      pb.p[0] = bwd_pk;
      pb.p[1] = bwd_pq;
      const hipError_t eb = va::launch_plan(pb, 2, st);
      if (eb != hipSuccess) return hip_fail(eb, "backward plan launch");
    }
    const hipError_t e = va::launch_kvcache(a, st);
    if (e != hipSuccess) return hip_fail(e, "short-query forward launch");
    return VA_OK;
  }

  va::FwdArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.bias = bias;
  if (bias) {
    a.bs0 = bias_stride[0]; a.bs1 = bias_stride[1]; a.bs2 = bias_stride[2]; a.bs3 = bias_stride[3];
    // every offset inside one (sequence, head) view is a 32-bit byte offset
    const int elt = bf16 ? 2 : 4;
    const int64_t span = ((int64_t)max_seqlen_q * a.bs2 + ((int64_t)max_seqlen_k + 64) * a.bs3 + 8) * elt;
    if (span >= ((int64_t)1 << 31))
      return fail(VA_ERR_UNSUPPORTED, "a bias view spanning 2 GiB or more per sequence and head");
    // vector bias loads: contiguous keys, every 4-key group aligned to its own size
    a.bias_vec = a.bs3 == 1 && a.bs0 % 4 == 0 && a.bs1 % 4 == 0 && a.bs2 % 4 == 0 &&
                 ((uintptr_t)bias) % (4 * elt) == 0;
    // 16-bit, whole 16-byte pieces of a row: the forward stages the bias through LDS
    a.bias_tile = elt == 2 && a.bs3 == 1 && a.bs0 % 8 == 0 && a.bs1 % 8 == 0 && a.bs2 % 8 == 0 &&
                  ((uintptr_t)bias) % 16 == 0;
  }
  a.out = out; a.lse = lse;
  a.q_rs = rs[0]; a.k_rs = rs[1]; a.v_rs = rs[2];
  a.batch = batch; a.total_q = total_q; a.total_k = total_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = num_heads_q / num_heads_kv; a.d = head_dim;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.bf16 = elem_code(dtype);
  const PlanLayout L = fwd_plan(batch, total_q, max_seqlen_k, num_heads_q, head_dim, bf16, part_budget);
  char* w = (char*)workspace;
  const size_t used = carve_plan(w, L, a.plan);
  a.part_o = (float*)(w + used);
  a.part_lse = a.part_o + (size_t)L.slot_cap * num_heads_q * va::fwd_block_m() * head_dim;
  a.split_cap = L.split_cap;
  va::PlanSet ps{};
  ps.p[0] = plan_args(a.plan, L, cu_seqlens_q, cu_seqlens_k, total_q, total_k, batch,
                      va::fwd_block_m(), va::fwd_block_n(bf16, head_dim), 0, causal);
  ps.p[1] = bwd_pk;
  ps.p[2] = bwd_pq;
  hipError_t e = va::launch_plan(ps, bwd_ws ? 3 : 1, st);
  if (e != hipSuccess) return hip_fail(e, "forward plan launch");
  e = va::launch_fwd(a, (int64_t)L.unit_cap * num_heads_q, st);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return VA_OK;
}

}  // namespace va

extern "C" {

size_t va_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t total_k,
                                    int32_t max_seqlen_q, int32_t max_seqlen_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    va_dtype dtype, va_dtype grad_dtype) {
  if (batch <= 0 || total_q <= 0 || total_k <= 0 || max_seqlen_q <= 0 || max_seqlen_k <= 0 ||
      num_heads_q <= 0 || num_heads_kv <= 0 ||
      num_heads_q % num_heads_kv != 0 || !varlen_head_dim(head_dim) ||
      (dtype != VA_F32 && dtype != VA_BF16 && dtype != VA_F16) ||
      (grad_dtype != VA_F32 && grad_dtype != dtype))
    return 0;
  return bwd_workspace(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                       num_heads_kv, head_dim, dtype != VA_F32);
}

}  // extern "C"

// The backward; `planned`: the workspace already holds the work plans, built by the
// forward of the same call shape (va_varlen_fwd_bwdplan).
static va_status varlen_bwd(const void* dout, const void* q, const void* k, const void* v,
                            const void* out, const float* lse, const int32_t* cu_seqlens_q,
                            const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                            float softmax_scale, int causal, const void* bias,
                            const int64_t* bias_stride, void* dq, void* dk, void* dv, float* dbias,
                            const int64_t* dbias_stride, const int64_t* qkv_row_stride, void* workspace,
                            size_t workspace_bytes, int32_t batch, int32_t total_q, int32_t total_k,
                            int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                            va_dtype dtype, va_dtype grad_dtype, va_stream stream, bool planned) {
  g_err[0] = 0;
  if (!dout || !q || !k || !v || !out || !lse || !cu_seqlens_q || !cu_seqlens_k || !dq || !dk ||
      !dv || !workspace)
    return fail(VA_ERR_INVALID, "a required pointer is NULL");
  Common c{batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, max_seqlen_q,
           max_seqlen_k, causal, dtype};
  va_status s = check_common(c, softmax_scale, bias, bias_stride);
  if (s != VA_OK) return s;
  int64_t rs[3];
  s = row_strides(c, q, k, v, qkv_row_stride, rs);
  if (s != VA_OK) return s;
  if (grad_dtype != VA_F32 && grad_dtype != VA_BF16 && grad_dtype != VA_F16)
    return fail(VA_ERR_UNSUPPORTED, "unknown grad_dtype %d", (int)grad_dtype);
  if (grad_dtype != VA_F32 && grad_dtype != dtype)
    return fail(VA_ERR_UNSUPPORTED, "gradients are float32 or the input dtype");
  int dbias_mode = 0;
  if ((dbias == nullptr) != (dbias_stride == nullptr))
    return fail(VA_ERR_INVALID, "dbias and dbias_stride must both be NULL or both non-NULL");
  if (dbias) {
    if (!bias) return fail(VA_ERR_INVALID, "dbias requires a bias");
    const int64_t* t = dbias_stride;
    for (int i = 0; i < 4; ++i)
      if (t[i] < 0) return fail(VA_ERR_INVALID, "dbias_stride[%d] is negative", i);
    const int n_rep_ = num_heads_q / num_heads_kv;
    if ((t[0] == 0 && batch > 1) || t[3] == 0)
      return fail(VA_ERR_UNSUPPORTED, "a bias gradient summed over sequences or keys is not supported");
    if (t[2] != 0) {  // per pair: every (b, h, r, c) its own element
      if (t[1] == 0 && num_heads_q > 1)
        return fail(VA_ERR_UNSUPPORTED, "a per-pair bias gradient summed over heads is not supported");
      dbias_mode = 1;
    } else {  // per key: summed over rows (and over heads when t1 = 0)
      const int max_heads = head_dim <= 128 ? 32 : 8;  // the dK/dV pass's LDS accumulators
      if (t[1] == 0 ? num_heads_kv != 1 : n_rep_ > max_heads)
        return fail(VA_ERR_UNSUPPORTED,
                    "a per-key bias gradient needs a head stride with at most %d query heads per "
                    "KV head (head_dim %d), or one KV head when summed over heads", max_heads, head_dim);
      dbias_mode = 2;
    }
  }
  if (((uintptr_t)workspace) % kAlign != 0)
    return fail(VA_ERR_INVALID, "workspace must be 256-byte aligned");
  const bool bf16 = dtype != VA_F32;  // a 16-bit kind (bf16 or f16)
  const int n_rep = num_heads_q / num_heads_kv;
  const size_t need = bwd_workspace(batch, total_q, total_k, max_seqlen_q, max_seqlen_k,
                                    num_heads_q, num_heads_kv, head_dim, bf16);
  if (workspace_bytes < need)
    return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);

  va::BwdArgs a{};
  a.dout = dout; a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.bias = bias;
  if (bias) {
    a.bs0 = bias_stride[0]; a.bs1 = bias_stride[1]; a.bs2 = bias_stride[2]; a.bs3 = bias_stride[3];
    const int elt = bf16 ? 2 : 4;
    const int64_t span = ((int64_t)max_seqlen_q * a.bs2 + ((int64_t)max_seqlen_k + 64) * a.bs3 + 8) * elt;
    if (span >= ((int64_t)1 << 31))
      return fail(VA_ERR_UNSUPPORTED, "a bias view spanning 2 GiB or more per sequence and head");
    a.bias_vec = a.bs3 == 1 && a.bs0 % 4 == 0 && a.bs1 % 4 == 0 && a.bs2 % 4 == 0 &&
                 ((uintptr_t)bias) % (4 * elt) == 0;
    const int64_t ve = 16 / elt;  // elements per 16 bytes
    a.bias_tile = a.bs3 == 1 && a.bs0 % ve == 0 && a.bs1 % ve == 0 && a.bs2 % ve == 0 &&
                  ((uintptr_t)bias) % 16 == 0;
  }
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.q_rs = rs[0]; a.k_rs = rs[1]; a.v_rs = rs[2];
  a.batch = batch; a.total_q = total_q; a.total_k = total_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = n_rep; a.d = head_dim;
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.bf16 = elem_code(dtype);
  a.grad_bf16 = grad_dtype == VA_F32 ? 0 : elem_code(grad_dtype);

  char* w = (char*)workspace;
  const BwdPlans B = bwd_plans(w, batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q,
                               num_heads_kv, head_dim, bf16);
  const PlanLayout& K = B.K;
  const PlanLayout& Q = B.Q;
  a.dsum = (float*)w;
  a.plan_k = B.pk;
  a.plan_q = B.pq;
  size_t o = B.end;
  a.part_kv = (float*)(w + o);
  o += round_up(K.slot_bytes * K.slot_cap);
  a.part_q = (float*)(w + o);
  o += round_up(Q.slot_bytes * Q.slot_cap);
  a.part_db = (float*)(w + o);
  a.dbias = dbias;
  a.dbias_mode = dbias_mode;
  if (dbias) { a.ds0 = dbias_stride[0]; a.ds1 = dbias_stride[1]; a.ds2 = dbias_stride[2]; a.ds3 = dbias_stride[3]; }
  a.split_cap_k = K.split_cap;
  a.split_cap_q = Q.split_cap;

  va::PlanSet ps{};
  ps.p[0] = plan_args(a.plan_k, K, cu_seqlens_k, cu_seqlens_q, total_k, total_q, batch,
                      va::bwd_block_k(), va::bwd_dkdv_block_q(), 1, causal);
  ps.p[1] = plan_args(a.plan_q, Q, cu_seqlens_q, cu_seqlens_k, total_q, total_k, batch,
                      va::bwd_block_q(), va::bwd_dq_block_n(bf16, head_dim), 0, causal);
  ps.nplans = planned ? 0 : 2;
  hipError_t e = va::launch_bwd(a, ps, (int64_t)Q.unit_cap * num_heads_q,
                                (int64_t)K.unit_cap * num_heads_kv, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
  return VA_OK;
}

extern "C" {

va_status va_varlen_bwd(const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        float softmax_scale, int causal, const void* bias,
                        const int64_t* bias_stride, void* dq, void* dk, void* dv, float* dbias,
                        const int64_t* dbias_stride, const int64_t* qkv_row_stride, void* workspace,
                        size_t workspace_bytes, int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        va_dtype dtype, va_dtype grad_dtype, va_stream stream) {
  return varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    softmax_scale, causal, bias, bias_stride, dq, dk, dv, dbias, dbias_stride, qkv_row_stride,
                    workspace, workspace_bytes, batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim,
                    dtype, grad_dtype, stream, false);
}

va_status va_varlen_bwd_planned(const void* dout, const void* q, const void* k, const void* v,
                                const void* out, const float* lse, const int32_t* cu_seqlens_q,
                                const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                float softmax_scale, int causal, const void* bias,
                                const int64_t* bias_stride, void* dq, void* dk, void* dv, float* dbias,
                                const int64_t* dbias_stride, const int64_t* qkv_row_stride, void* workspace,
                                size_t workspace_bytes, int32_t batch, int32_t total_q, int32_t total_k,
                                int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                va_dtype dtype, va_dtype grad_dtype, va_stream stream) {
  return varlen_bwd(dout, q, k, v, out, lse, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k,
                    softmax_scale, causal, bias, bias_stride, dq, dk, dv, dbias, dbias_stride, qkv_row_stride,
                    workspace, workspace_bytes, batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim,
                    dtype, grad_dtype, stream, true);
}

// ---------------------------------------------------------------------------
// Packing (include/va_pack.h)
// ---------------------------------------------------------------------------
size_t va_kvcache_fwd_workspace_size(int32_t batch, int32_t max_seqlen_q, int32_t max_seqlen_k,
                                     int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                     va_dtype dtype) {
  if (!kv_args_ok(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, dtype)) return 0;
  const KvLayout L = kv_layout(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  return L.total();
}

va_status va_kvcache_fwd(const void* q, const void* k_cache, const void* v_cache,
                         const int32_t* cu_seqlens_q, const int32_t* seqlens_k,
                         const int32_t* block_table, int32_t block_table_stride,
                         int32_t page_size, int32_t num_pages,
                         int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                         int causal, void* out, float* lse, void* workspace,
                         size_t workspace_bytes, int32_t batch, int32_t total_q,
                         int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                         va_dtype dtype, va_stream stream) {
  g_err[0] = 0;
  if (!q || !k_cache || !v_cache || !cu_seqlens_q || !seqlens_k || !block_table || !out || !lse)
    return fail(VA_ERR_INVALID, "a required pointer is NULL");
  if (batch <= 0 || total_q <= 0) return fail(VA_ERR_INVALID, "batch and total_q must be > 0");
  if (num_heads_q <= 0 || num_heads_kv <= 0 || num_heads_q % num_heads_kv != 0)
    return fail(VA_ERR_INVALID, "head counts must be > 0, num_heads_q a multiple of num_heads_kv");
  if (head_dim <= 0) return fail(VA_ERR_INVALID, "head_dim must be > 0");
  if (max_seqlen_q <= 0 || max_seqlen_k < 0)
    return fail(VA_ERR_INVALID, "max_seqlen_q must be > 0 and max_seqlen_k >= 0");
  if (page_size <= 0 || page_size > (1 << 20) || (page_size & (page_size - 1)) != 0)
    return fail(VA_ERR_INVALID, "page_size must be a power of two in [1, 2^20] (got %d)", page_size);
  if (num_pages <= 0) return fail(VA_ERR_INVALID, "num_pages must be > 0");
  if (block_table_stride <= 0 || (int64_t)block_table_stride * page_size < max_seqlen_k)
    return fail(VA_ERR_INVALID, "block_table_stride * page_size must cover max_seqlen_k");
  if (causal != 0 && causal != 1) return fail(VA_ERR_INVALID, "causal must be 0 or 1");
  if (!(std::isfinite(softmax_scale) && softmax_scale > 0.f))
    return fail(VA_ERR_INVALID, "softmax_scale must be finite and > 0");
  if ((((uintptr_t)q) | ((uintptr_t)k_cache) | ((uintptr_t)v_cache) | ((uintptr_t)out)) % 16 != 0)
    return fail(VA_ERR_INVALID, "q, k_cache, v_cache and out must be 16-byte aligned");
  if (dtype != VA_BF16 && dtype != VA_F16 && dtype != VA_F32)
    return fail(VA_ERR_UNSUPPORTED, "decode steps take bf16, float16 or float32 (got dtype %d)", (int)dtype);
  if (!decode_head_dim(head_dim))
    return fail(VA_ERR_UNSUPPORTED, "head_dim %d not supported in decode steps (32, 64, 96 or 128)", head_dim);
  if (!kv_args_ok(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim, dtype))
    return fail(VA_ERR_UNSUPPORTED, "max_seqlen_q * num_heads_q * head_dim * element size must be < 2^31");
  const KvLayout L = kv_layout(batch, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv, head_dim);
  const size_t need = L.total();
  if (!workspace) return fail(VA_ERR_INVALID, "workspace is NULL");
  if (((uintptr_t)workspace) % kAlign != 0) return fail(VA_ERR_INVALID, "workspace must be 256-byte aligned");
  if (workspace_bytes < need)
    return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);
  va::KvArgs a{};
  a.q = q; a.k_cache = k_cache; a.v_cache = v_cache;
  a.cu_q = cu_seqlens_q; a.seqlens_k = seqlens_k; a.block_table = block_table;
  a.out = out; a.lse = lse;
  char* w = (char*)workspace;
  a.plan = (int32_t*)w;
  a.chunks = (va::KvChunk*)(w + round_up(256));
  a.merges = (int32_t*)(w + round_up(256) + round_up((size_t)L.cap * sizeof(va::KvChunk)));
  a.part_o = L.part_o_bytes > 0 ? (float*)(w + L.plan_bytes) : nullptr;
  a.part_lse = L.part_lse_bytes > 0 ? (float*)(w + L.plan_bytes + L.part_o_bytes) : nullptr;
  a.batch = batch; a.total_q = total_q;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = num_heads_q / num_heads_kv; a.d = head_dim;
  a.bt_stride = block_table_stride;
  int shift = 0;
  while ((1 << shift) < page_size) ++shift;
  a.page_shift = shift;
  a.num_pages = num_pages;
  const int64_t reach = (int64_t)block_table_stride * page_size;
  a.max_k = (int)(reach < max_seqlen_k ? reach : max_seqlen_k);
  a.rows = L.rows; a.chunk = L.chunk; a.nchunk = L.nchunk; a.cap = L.cap; a.cap_merge = L.cap_merge;
  a.q_rs = (int64_t)num_heads_q * head_dim;
  a.k_rs = a.v_rs = (int64_t)num_heads_kv * head_dim;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.h16 = elem_code(dtype);
  const hipError_t e = va::launch_kvcache(a, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return VA_OK;
}

va_status va_pack_metadata(const uint8_t* mask, int32_t batch, int32_t seqlen,
                           int32_t* cu_seqlens, int32_t* max_seqlen,
                           int32_t* indices, int32_t* position_ids, int32_t* inverse,
                           va_stream stream) {
  if (!mask || !cu_seqlens || !max_seqlen || !indices || !position_ids || !inverse)
    return fail(VA_ERR_INVALID, "NULL pointer argument");
  if (batch <= 0 || seqlen <= 0)
    return fail(VA_ERR_INVALID, "batch and seqlen must be > 0 (got %d, %d)", batch, seqlen);
  if ((int64_t)batch * seqlen >= ((int64_t)1 << 31))
    return fail(VA_ERR_INVALID, "batch * seqlen must be < 2^31");
  const hipError_t e = va::launch_pack_metadata(mask, batch, seqlen, cu_seqlens, max_seqlen, indices,
                                                position_ids, inverse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "packing metadata launch");
  return VA_OK;
}

static va_status pack_args(const va_pack_tensor* tensors, int32_t n, int32_t batch, int32_t seqlen,
                           int64_t packed_rows, va::PackArgs& a, int& width) {
  if (!tensors) return fail(VA_ERR_INVALID, "NULL tensors");
  if (n < 1 || n > VA_PACK_MAX_TENSORS)
    return fail(VA_ERR_INVALID, "n_tensors must be 1..%d (got %d)", VA_PACK_MAX_TENSORS, n);
  if (batch <= 0 || seqlen <= 0)
    return fail(VA_ERR_INVALID, "batch and seqlen must be > 0 (got %d, %d)", batch, seqlen);
  if ((int64_t)batch * seqlen >= ((int64_t)1 << 31))
    return fail(VA_ERR_INVALID, "batch * seqlen must be < 2^31");
  if (packed_rows < 0) return fail(VA_ERR_INVALID, "packed_rows must be >= 0");
  a = va::PackArgs{};
  a.n = n;
  a.batch = batch;
  a.padded_rows = (int64_t)batch * seqlen;
  a.packed_rows = packed_rows;
  // the widest copy that divides every row size and base address
  uint64_t g = 16;
  for (int i = 0; i < n; ++i) {
    const va_pack_tensor& t = tensors[i];
    if (!t.padded || !t.packed) return fail(VA_ERR_INVALID, "NULL pointer in tensor %d", i);
    if (t.row_bytes <= 0) return fail(VA_ERR_INVALID, "row_bytes of tensor %d must be > 0", i);
    a.padded[i] = t.padded;
    a.packed[i] = t.packed;
    a.row_bytes[i] = t.row_bytes;
    const uint64_t bits = (uint64_t)t.row_bytes | (uint64_t)(uintptr_t)t.padded | (uint64_t)(uintptr_t)t.packed;
    while (g > 1 && (bits & (g - 1)) != 0) g >>= 1;
  }
  width = (int)g;
  return VA_OK;
}

va_status va_unpad(const va_pack_tensor* tensors, int32_t n_tensors,
                   const int32_t* indices, const int32_t* cu_seqlens,
                   int32_t batch, int32_t seqlen, int64_t packed_rows, va_stream stream) {
  if (!indices || !cu_seqlens) return fail(VA_ERR_INVALID, "NULL pointer argument");
  va::PackArgs a;
  int width = 1;
  const va_status st = pack_args(tensors, n_tensors, batch, seqlen, packed_rows, a, width);
  if (st != VA_OK) return st;
  if (packed_rows == 0) return VA_OK;
  const hipError_t e = va::launch_unpad(a, width, indices, cu_seqlens, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "unpad launch");
  return VA_OK;
}

va_status va_pad(const va_pack_tensor* tensors, int32_t n_tensors, const int32_t* inverse,
                 int32_t batch, int32_t seqlen, int64_t packed_rows, va_stream stream) {
  if (!inverse) return fail(VA_ERR_INVALID, "NULL pointer argument");
  va::PackArgs a;
  int width = 1;
  const va_status st = pack_args(tensors, n_tensors, batch, seqlen, packed_rows, a, width);
  if (st != VA_OK) return st;
  const hipError_t e = va::launch_pad(a, width, inverse, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "pad launch");
  return VA_OK;
}

}  // extern "C"

namespace {

struct Timing {
  bool on = false;
  std::vector<hipEvent_t> ev;  // 2 per launch
  std::vector<const char*> names;
  int used = 0;
};
thread_local Timing g_timing;

}  // namespace

extern "C" va_status va_timing_start(int max_launches) {
  Timing& t = g_timing;
  if (max_launches <= 0) return fail(VA_ERR_INVALID, "max_launches must be > 0");
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.assign(2 * (size_t)max_launches, nullptr);
  t.names.assign((size_t)max_launches, nullptr);
  for (auto& e : t.ev) {
    hipError_t r = hipEventCreate(&e);
    if (r != hipSuccess) {
      t.on = false;
      return hip_fail(r, "hipEventCreate");
    }
  }
  t.used = 0;
  t.on = true;
  return VA_OK;
}

extern "C" int va_timing_stop(va_kernel_time* out, int max_entries) {
  Timing& t = g_timing;
  t.on = false;
  std::vector<va_kernel_time> agg;
  int rc = 0;
  for (int i = 0; i < t.used && rc == 0; ++i) {
    if (hipEventSynchronize(t.ev[2 * i + 1]) != hipSuccess) { rc = -1; break; }
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, t.ev[2 * i], t.ev[2 * i + 1]) != hipSuccess) { rc = -1; break; }
    size_t j = 0;
    while (j < agg.size() && std::string(agg[j].name) != t.names[i]) ++j;
    if (j == agg.size()) agg.push_back({t.names[i], 0, 0.0});
    agg[j].launches += 1;
    agg[j].total_ms += ms;
  }
  for (hipEvent_t e : t.ev) (void)hipEventDestroy(e);
  t.ev.clear();
  t.names.clear();
  t.used = 0;
  if (rc != 0) return -1;
  for (int j = 0; j < (int)agg.size() && j < max_entries; ++j) out[j] = agg[j];
  return (int)agg.size();
}

namespace va {

void timing_before(hipStream_t st, const char* name) {
  Timing& t = g_timing;
  if (!t.on || t.used >= (int)t.names.size()) return;
  t.names[t.used] = name;
  (void)hipEventRecord(t.ev[2 * t.used], st);
}

void timing_after(hipStream_t st) {
  Timing& t = g_timing;
  if (!t.on || t.used >= (int)t.names.size() || t.names[t.used] == nullptr) return;
  (void)hipEventRecord(t.ev[2 * t.used + 1], st);
  t.used += 1;
}

// Resident workgroups of `kernel` on the current device, capped by the work.
int resident_grid(const void* kernel, int threads, int64_t max_items) {
  static std::atomic<int> cu_cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return -1;
  int cus = (dev >= 0 && dev < 64) ? cu_cache[dev].load() : 0;
  if (cus <= 0) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return -1;
    if (dev >= 0 && dev < 64) cu_cache[dev].store(cus);
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, 0) != hipSuccess ||
      per_cu < 1)
    per_cu = 1;
  int64_t g = (int64_t)cus * per_cu;
  if (max_items < g) g = max_items;
  if (g < 1) g = 1;
  return (int)g;
}

}  // namespace va
