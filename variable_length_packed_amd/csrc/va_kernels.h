// Kernel argument blocks and launchers (host <-> device interface inside the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace va {

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const void* bias;  // nullptr = no bias
  int64_t bs0, bs1, bs2, bs3;
  void* out;
  float* lse;
  int32_t batch, total_q, total_k, hq, hkv, n_rep, d;
  int32_t tcap;    // q-tiles per sequence considered (from max_seqlen_q)
  int32_t stride;  // q-tiles per schedule level
  int32_t nlev;    // schedule levels
  float scale_log2;
  int32_t causal;
  int32_t bf16;
};

struct BwdArgs {
  const void* dout;
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const void* bias;
  int64_t bs0, bs1, bs2, bs3;
  void* dq;
  void* dk;
  void* dv;
  float* dsum;  // workspace [hq, total_q]: rowsum(dO * O)
  float* part;  // workspace [2 * hsplit][total_k, hkv, d]: dK/dV partial sums (hsplit > 1)
  int32_t hsplit;  // workgroups sharing one GQA group's query heads (1 or n_rep)
  int32_t batch, total_q, total_k, hq, hkv, n_rep, d;
  int32_t tcap_q, stride_q, nlev_q;  // schedule over q-tiles (dQ kernel)
  int32_t tcap_k, stride_k, nlev_k;  // schedule over k-tiles (dK/dV kernel)
  float scale;
  float scale_log2;
  int32_t causal;
  int32_t bf16;
  int32_t grad_bf16;
};

// Optional per-kernel event timing (see va_timing_start); no-ops when off.
void timing_before(hipStream_t st, const char* name);
void timing_after(hipStream_t st);

// Persistent grids: min(max_items, resident workgroups per device).
int resident_grid(const void* kernel, int threads, int64_t max_items);

int fwd_block_m(bool bf16, int d);
hipError_t launch_fwd(const FwdArgs& a, int64_t max_items, hipStream_t st);

int bwd_block_q();
int bwd_block_k();
hipError_t launch_bwd(const BwdArgs& a, int64_t max_q_items, int64_t max_k_items, hipStream_t st);

}  // namespace va
