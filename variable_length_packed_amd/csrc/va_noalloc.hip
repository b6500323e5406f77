// The packed forward for callers that cannot allocate device memory (code
// under HIP graph capture, tight serving loops, harnesses that forbid
// allocation): va_varlen_fwd with its workspace taken from a fixed array in
// the library's own device memory instead of a caller buffer.
//
// The array lives in the code object, so each GPU the library runs on holds
// one copy for the life of the process.  In host code `scratch` only names
// the symbol; the address of a device's copy comes from hipGetSymbolAddress,
// asked once per device with that device current and kept here.  Every call
// on a GPU shares that GPU's copy: calls that may overlap on one GPU (other
// streams, other threads) race on it.  Nothing in it needs clearing between
// calls: the planner rewrites the whole work plan, and every partial result
// is written before it is read.
#include <mutex>

#include "va_kernels.h"
#include "va_varlen.h"

static __device__ __align__(256) unsigned char scratch[VA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of each device's copy, once looked up

va_status error(va_status s, const char* msg) {
  va::set_error(msg);
  return s;
}

}  // namespace

extern "C" va_status va_varlen_fwd_noalloc(const void* q, const void* k, const void* v,
                                           const int32_t* cu_seqlens_q, const int32_t* cu_seqlens_k,
                                           int32_t max_seqlen_q, int32_t max_seqlen_k, float softmax_scale,
                                           int causal, const void* bias, const int64_t* bias_stride, void* out,
                                           float* lse, const int64_t* qkv_row_stride, int32_t batch,
                                           int32_t total_q, int32_t total_k, int32_t num_heads_q,
                                           int32_t num_heads_kv, int32_t head_dim, va_dtype dtype,
                                           va_stream stream) {
  constexpr size_t cap = VA_NOALLOC_SCRATCH_BYTES;
  // the partial results of split tiles get what the plan leaves of the array
  // (fewer partial slots only lengthen the split chunks)
  size_t budget = cap;
  size_t need = 0;
  for (int i = 0; i < 64; ++i) {
    need = va::varlen_fwd_need(batch, total_q, total_k, max_seqlen_q, max_seqlen_k, num_heads_q, num_heads_kv,
                               head_dim, dtype, budget);
    if (need <= cap || budget == 0) break;
    budget = budget > need - cap ? budget - (need - cap) : 0;
  }
  // 0: sizes the forward rejects; it names the problem (before it looks at the workspace)
  if (need == 0)
    return va::varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale,
                          causal, bias, bias_stride, out, lse, qkv_row_stride, nullptr, 0, 0, batch, total_q,
                          total_k, num_heads_q, num_heads_kv, head_dim, dtype, stream);
  if (need > cap) {
    char msg[200];
    snprintf(msg, sizeof(msg),
             "these sizes need %zu bytes of scratch, more than the %zu of the allocation-free "
             "forward: call va_varlen_fwd with a workspace",
             need, cap);
    return error(VA_ERR_WORKSPACE, msg);
  }
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return error(VA_ERR_HIP, "hipGetDevice failed");
  if (dev < 0 || dev >= kMaxDevices) return error(VA_ERR_UNSUPPORTED, "device index above 63");
  void* ptr = nullptr;
  {
    std::lock_guard<std::mutex> lock(g_mu);
    if (g_scratch[dev] == nullptr) {
      void* p = nullptr;
      const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
      if (e != hipSuccess || p == nullptr) {
        char msg[200];
        snprintf(msg, sizeof(msg), "hipGetSymbolAddress of the scratch array: %s", hipGetErrorString(e));
        return error(VA_ERR_HIP, msg);
      }
      g_scratch[dev] = p;
    }
    ptr = g_scratch[dev];
  }
  return va::varlen_fwd(q, k, v, cu_seqlens_q, cu_seqlens_k, max_seqlen_q, max_seqlen_k, softmax_scale, causal,
                        bias, bias_stride, out, lse, qkv_row_stride, ptr, cap, budget, batch, total_q, total_k,
                        num_heads_q, num_heads_kv, head_dim, dtype, stream);
}
