// C ABI of the packed varlen attention library: argument validation (host
// only, no device reads), schedule sizing and kernel launch.  Declarations
// and the contract of every entry point are in include/va_varlen.h.
#include "va_varlen.h"

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

constexpr int kMaxLevels = 512;  // matches the device schedule's level table

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
  if (c.dtype != VA_F32 && c.dtype != VA_BF16) return fail(VA_ERR_UNSUPPORTED, "unknown dtype %d", (int)c.dtype);
  if (c.d != 64 && c.d != 128) return fail(VA_ERR_UNSUPPORTED, "head_dim %d not supported (64 or 128)", c.d);
  if ((int64_t)c.total_q * c.hq * c.d >= ((int64_t)1 << 40) ||
      (int64_t)c.total_k * c.hkv * c.d >= ((int64_t)1 << 40))
    return fail(VA_ERR_UNSUPPORTED, "tensor too large");
  return VA_OK;
}

// Schedule sizing: tiles of bm rows per sequence, capped by max_seqlen; at
// most kMaxLevels schedule levels.
void sched_dims(int max_len, int bm, int& tcap, int& stride, int& nlev) {
  tcap = (max_len + bm - 1) / bm;
  if (tcap < 1) tcap = 1;
  stride = (tcap + kMaxLevels - 1) / kMaxLevels;
  nlev = (tcap + stride - 1) / stride;
}

int64_t max_tiles(int total, int batch, int bm, int tcap) {
  int64_t a = (int64_t)total / bm + batch;  // each sequence adds at most one ragged tile
  int64_t b = (int64_t)batch * tcap;
  return a < b ? a : b;
}

// Backward workspace: D = rowsum(dO * O) as [hq, total_q] float32, then,
// when the query heads of a GQA group are spread over several workgroups,
// float32 dK/dV partial sums [2 * hsplit][total_k, hkv, d].
constexpr size_t kAlign = 256;
size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

// Split a GQA group's heads over workgroups when the unsplit dK/dV grid
// would be too small to fill the device: at most 2048 work items.
int choose_hsplit(int batch, int total_k, int hkv, int n_rep, int bnk, int tcap_k) {
  if (n_rep <= 1) return 1;
  return max_tiles(total_k, batch, bnk, tcap_k) * hkv < 2048 ? n_rep : 1;
}

size_t bwd_workspace(int batch, int total_q, int total_k, int hq, int hkv, int d, int max_k,
                     int& hsplit) {
  int tcap, stride, nlev;
  sched_dims(max_k, va::bwd_block_k(), tcap, stride, nlev);
  hsplit = choose_hsplit(batch, total_k, hkv, hq / hkv, va::bwd_block_k(), tcap);
  size_t ws = round_up((size_t)hq * total_q * sizeof(float));
  if (hsplit > 1) ws += round_up((size_t)2 * hsplit * total_k * hkv * d * sizeof(float));
  return ws;
}

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

va_status va_varlen_fwd(const void* q, const void* k, const void* v,
                        const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                        int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                        int causal, const void* bias, const int64_t* bias_stride, void* out,
                        float* lse, int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        va_dtype dtype, va_stream stream) {
  g_err[0] = 0;
  if (!q || !k || !v || !cu_seqlens_q || !cu_seqlens_k || !out || !lse)
    return fail(VA_ERR_INVALID, "a required pointer is NULL");
  Common c{batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, max_seqlen_q,
           max_seqlen_k, causal, dtype};
  va_status s = check_common(c, softmax_scale, bias, bias_stride);
  if (s != VA_OK) return s;

  va::FwdArgs a{};
  a.q = q; a.k = k; a.v = v;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.bias = bias;
  if (bias) { a.bs0 = bias_stride[0]; a.bs1 = bias_stride[1]; a.bs2 = bias_stride[2]; a.bs3 = bias_stride[3]; }
  a.out = out; a.lse = lse;
  a.batch = batch; a.total_q = total_q; a.total_k = total_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = num_heads_q / num_heads_kv; a.d = head_dim;
  const int bm = va::fwd_block_m(dtype == VA_BF16, head_dim);
  sched_dims(max_seqlen_q, bm, a.tcap, a.stride, a.nlev);
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.bf16 = dtype == VA_BF16;
  const int64_t items = max_tiles(total_q, batch, bm, a.tcap) * num_heads_q;
  hipError_t e = va::launch_fwd(a, items, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "forward launch");
  return VA_OK;
}

size_t va_varlen_bwd_workspace_size(int32_t batch, int32_t total_q, int32_t total_k,
                                    int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                                    va_dtype dtype, va_dtype grad_dtype) {
  if (batch <= 0 || total_q <= 0 || total_k <= 0 || num_heads_q <= 0 || num_heads_kv <= 0 ||
      num_heads_q % num_heads_kv != 0 || (head_dim != 64 && head_dim != 128) ||
      (dtype != VA_F32 && dtype != VA_BF16) || (grad_dtype != VA_F32 && grad_dtype != VA_BF16) ||
      (dtype == VA_F32 && grad_dtype == VA_BF16))
    return 0;
  int hsplit;
  // the dK/dV tile cap only bounds the grid estimate; use the largest possible
  return bwd_workspace(batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, total_k, hsplit);
}

va_status va_varlen_bwd(const void* dout, const void* q, const void* k, const void* v,
                        const void* out, const float* lse, const int32_t* cu_seqlens_q,
                        const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                        float softmax_scale, int causal, const void* bias,
                        const int64_t* bias_stride, void* dq, void* dk, void* dv, void* workspace,
                        size_t workspace_bytes, int32_t batch, int32_t total_q, int32_t total_k,
                        int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                        va_dtype dtype, va_dtype grad_dtype, va_stream stream) {
  g_err[0] = 0;
  if (!dout || !q || !k || !v || !out || !lse || !cu_seqlens_q || !cu_seqlens_k || !dq || !dk ||
      !dv || !workspace)
    return fail(VA_ERR_INVALID, "a required pointer is NULL");
  Common c{batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim, max_seqlen_q,
           max_seqlen_k, causal, dtype};
  va_status s = check_common(c, softmax_scale, bias, bias_stride);
  if (s != VA_OK) return s;
  if (grad_dtype != VA_F32 && grad_dtype != VA_BF16)
    return fail(VA_ERR_UNSUPPORTED, "unknown grad_dtype %d", (int)grad_dtype);
  if (dtype == VA_F32 && grad_dtype == VA_BF16)
    return fail(VA_ERR_UNSUPPORTED, "bf16 gradients of float32 inputs are not supported");
  if (((uintptr_t)workspace) % kAlign != 0)
    return fail(VA_ERR_INVALID, "workspace must be 256-byte aligned");
  int hsplit = 1;
  const size_t need = bwd_workspace(batch, total_q, total_k, num_heads_q, num_heads_kv, head_dim,
                                    total_k, hsplit);
  if (workspace_bytes < need)
    return fail(VA_ERR_WORKSPACE, "workspace of %zu bytes < %zu required", workspace_bytes, need);

  va::BwdArgs a{};
  a.dout = dout; a.q = q; a.k = k; a.v = v; a.out = out; a.lse = lse;
  a.cu_q = cu_seqlens_q; a.cu_k = cu_seqlens_k;
  a.bias = bias;
  if (bias) { a.bs0 = bias_stride[0]; a.bs1 = bias_stride[1]; a.bs2 = bias_stride[2]; a.bs3 = bias_stride[3]; }
  a.dq = dq; a.dk = dk; a.dv = dv;
  a.dsum = (float*)workspace;
  a.hsplit = hsplit;
  a.part = hsplit > 1 ? (float*)((char*)workspace + round_up((size_t)num_heads_q * total_q * sizeof(float)))
                      : nullptr;
  a.batch = batch; a.total_q = total_q; a.total_k = total_k;
  a.hq = num_heads_q; a.hkv = num_heads_kv; a.n_rep = num_heads_q / num_heads_kv; a.d = head_dim;
  sched_dims(max_seqlen_q, va::bwd_block_q(), a.tcap_q, a.stride_q, a.nlev_q);
  sched_dims(max_seqlen_k, va::bwd_block_k(), a.tcap_k, a.stride_k, a.nlev_k);
  a.scale = softmax_scale;
  a.scale_log2 = softmax_scale * 1.4426950408889634f;
  a.causal = causal;
  a.bf16 = dtype == VA_BF16;
  a.grad_bf16 = grad_dtype == VA_BF16;
  const int64_t q_items = max_tiles(total_q, batch, va::bwd_block_q(), a.tcap_q) * num_heads_q;
  const int64_t k_items = max_tiles(total_k, batch, va::bwd_block_k(), a.tcap_k) * num_heads_kv;
  hipError_t e = va::launch_bwd(a, q_items, k_items, (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(e, "backward launch");
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
