// Forward kernel: exact attention over packed variable-length sequences.
//
// softmax(scale * Q K^T + bias + mask) V and its log-sum-exp per query row,
// for every sequence of the packed stream (FlashAttention-2 varlen semantics
// as the TorchEasyRec pull request 663 page uses it; bottom-right causal
// alignment; GQA; the strided per-sequence bias of the GiGL pull request 858
// page, section "Approach").
//
// Layout of the work on gfx950.  A workgroup (4 waves) owns one tile of
// BM = 128 query rows of one (sequence, query head); wave w owns 32 rows.
// Each wave keeps its Q rows in registers and computes the TRANSPOSED score
// tile S^T = K Q^T (keys x queries) on the 32x32 MFMA, so that every lane
// holds the scores of ONE query row against 16 keys of a 32-key block.  That
// layout is exactly the B operand of the 32x32 MFMA for O^T += V^T P^T, so P
// never leaves registers; only V needs a transposed copy, made while staging
// it into LDS.  K and V^T blocks of BN keys are staged in double-buffered
// LDS, shared by the 4 waves, prefetched into registers one block ahead.
// The online softmax runs in base 2 with scale*log2(e) folded into one FMA;
// a row's max needs one cross-half exchange per block, its sum one at the
// end.
#include "va_common.h"
#include "va_kernels.h"

namespace va {

namespace {

constexpr int BM = 128;  // query rows per workgroup
constexpr int NT = 256;  // threads per workgroup

// keys per block: 64 for bf16 (two 32-key score tiles), 32 for f32 (LDS size)
template <bool BF16>
struct BlockN {
  static constexpr int value = BF16 ? 64 : 32;
};

template <bool BF16, int D>
struct FwdSmem {
  static constexpr int BN = BlockN<BF16>::value;
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  // K block: [BN][D] row-major, row pitch padded by 16 bytes.
  static constexpr int KP = D + 16 / (int)sizeof(T);
  // V block: bf16 -> transposed [D][BN] with keys permuted inside each group
  // of 16 (bits 2 and 3 of the key swapped) so a lane's 8 MFMA k-slots are
  // contiguous; f32 -> [BN][D] like K.
  static constexpr int VROWS = BF16 ? D : BN;
  static constexpr int VP = (BF16 ? BN : D) + 16 / (int)sizeof(T);
  T k[2][BN * KP];
  T v[2][VROWS * VP];
};

// Position of key j (0..BN-1) inside a transposed bf16 V row.
__device__ __forceinline__ int vpos(int j) {
  return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1);
}

template <bool BF16, int D>
struct Loader {
  static constexpr int BN = BlockN<BF16>::value;
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  static constexpr int EPV = 16 / sizeof(T);           // elements per 16-byte vector
  static constexpr int KVEC = BN * D / EPV;            // 16-byte vectors per K block
  static constexpr int KPT = (KVEC + NT - 1) / NT;     // per thread
  // V (bf16): tasks of 2 keys x 8 dims; (f32): same as K
  static constexpr int VTASK = BF16 ? (BN / 2) * (D / 8) : KVEC;
  static constexpr int VPT = (VTASK + NT - 1) / NT;
  u32x4_t kr[KPT];
  u32x4_t vr[BF16 ? 2 * VPT : VPT];

  __device__ __forceinline__ void load(const T* __restrict__ kbase, const T* __restrict__ vbase,
                                       size_t row_stride, int kb, int klo, int khi) {
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int u = tid + i * NT;
      int key = u / (D / EPV), c = u % (D / EPV);
      int j = kb + key;
      u32x4_t z = {0, 0, 0, 0};
      if (u < KVEC && j >= klo && j < khi)
        z = *(const u32x4_t*)(kbase + (size_t)j * row_stride + c * EPV);
      kr[i] = z;
    }
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int u = tid + i * NT;
        int dc = u % (D / 8), kp = u / (D / 8);
#pragma unroll
        for (int r = 0; r < 2; ++r) {
          int j = kb + 2 * kp + r;
          u32x4_t z = {0, 0, 0, 0};
          if (u < VTASK && j >= klo && j < khi)
            z = *(const u32x4_t*)(vbase + (size_t)j * row_stride + dc * 8);
          vr[2 * i + r] = z;
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int u = tid + i * NT;
        int key = u / (D / EPV), c = u % (D / EPV);
        int j = kb + key;
        u32x4_t z = {0, 0, 0, 0};
        if (u < KVEC && j >= klo && j < khi)
          z = *(const u32x4_t*)(vbase + (size_t)j * row_stride + c * EPV);
        vr[i] = z;
      }
    }
  }

  __device__ __forceinline__ void store(FwdSmem<BF16, D>& sm, int buf) {
    using S = FwdSmem<BF16, D>;
    const int tid = threadIdx.x;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      int u = tid + i * NT;
      if (u < KVEC) {
        int key = u / (D / EPV), c = u % (D / EPV);
        *(u32x4_t*)(&sm.k[buf][key * S::KP + c * EPV]) = kr[i];
      }
    }
    if constexpr (BF16) {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int u = tid + i * NT;
        if (u < VTASK) {
          int dc = u % (D / 8), kp = u / (D / 8);
          const int pos = vpos(2 * kp);
          u32x4_t a = vr[2 * i], b = vr[2 * i + 1];
          // a holds dims dc*8..+8 of key 2kp, b of key 2kp+1; write pairs (key, key+1) per dim
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            uint32_t lo = (a[e] & 0xFFFFu) | (b[e] << 16);
            uint32_t hi = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
            *(uint32_t*)(&sm.v[buf][(dc * 8 + 2 * e) * S::VP + pos]) = lo;
            *(uint32_t*)(&sm.v[buf][(dc * 8 + 2 * e + 1) * S::VP + pos]) = hi;
          }
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < VPT; ++i) {
        int u = tid + i * NT;
        if (u < KVEC) {
          int key = u / (D / EPV), c = u % (D / EPV);
          *(u32x4_t*)(&sm.v[buf][key * S::VP + c * EPV]) = vr[i];
        }
      }
    }
  }
};

template <bool BF16, int D, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(NT, 2) void fwd_kernel(FwdArgs a) {
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  using S = FwdSmem<BF16, D>;
  constexpr int BN = BlockN<BF16>::value;
  constexpr int NS = BN / 32;                // 32-key score tiles per block
  constexpr int DT = D / 32;                 // 32-wide output tiles along head_dim
  constexpr int QF = BF16 ? D / 16 : D / 2;  // Q fragments (MFMA k-steps) per lane

  __shared__ SchedShared sched;
  __shared__ S sm;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int r32 = lane & 31;

  sched_build(sched, a.cu_q, a.batch, a.total_q, BM, a.tcap, a.stride, a.nlev);
  const int total_items = sched.total_tiles * a.hq;

  const T* __restrict__ qg = (const T*)a.q;
  const T* __restrict__ kg = (const T*)a.k;
  const T* __restrict__ vg = (const T*)a.v;
  T* __restrict__ og = (T*)a.out;
  const size_t qstride = (size_t)a.hq * D;
  const size_t kstride = (size_t)a.hkv * D;

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int tile = item / a.hq;
    const int h = item - tile * a.hq;
    int b, t;
    sched_find(sched, a.cu_q, a.batch, a.total_q, BM, a.tcap, a.stride, a.nlev, tile, b, t);
    int q0, q1, k0, k1;
    seq_bounds(a.cu_q, b, a.total_q, q0, q1);
    seq_bounds(a.cu_k, b, a.total_k, k0, k1);
    q0 = uniform(q0); q1 = uniform(q1); k0 = uniform(k0); k1 = uniform(k1);
    const int Lq = q1 - q0, Lk = k1 - k0;
    const int off = Lk - Lq;
    const int g = h / a.n_rep;
    const int r1 = Lq - t * BM;
    const int w0 = r1 - BM + 32 * wid;  // first row of this wave
    const int rq = w0 + r32;            // this lane's query row
    const bool row_ok = rq >= 0;
    // keys the whole tile may see, and this wave's last visible key + 1
    const int kv_hi = CAUSAL ? min(Lk, r1 + off) : Lk;
    const int wave_hi = CAUSAL ? min(Lk, w0 + 32 + off) : Lk;
    const bool wave_on = (w0 + 31 >= 0) && wave_hi > 0;
    const int nblk = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
    // causal: blocks end exactly at kv_hi (the ragged block holds keys near 0);
    // otherwise blocks start at 0 (the ragged block is the last)
    const int kb0 = CAUSAL ? kv_hi - nblk * BN : 0;

    // ---- Q fragment (B operand of S^T = K Q^T)
    u32x4_t qf4[BF16 ? QF : 1];
    float qff[BF16 ? 1 : QF];
    {
      const T* qrow = qg + (size_t)(q0 + max(rq, 0)) * qstride + (size_t)h * D;
      if constexpr (BF16) {
#pragma unroll
        for (int ks = 0; ks < QF; ++ks) {
          u32x4_t z = {0, 0, 0, 0};
          if (row_ok) z = *(const u32x4_t*)(qrow + 16 * ks + 8 * hh);
          qf4[ks] = z;
        }
      } else {
        // k-slot (group G, step j) of lane half hh reads dim 8G + 4hh + j
#pragma unroll
        for (int G = 0; G < D / 8; ++G) {
          f32x4_t z = {0.f, 0.f, 0.f, 0.f};
          if (row_ok) z = *(const f32x4_t*)(qrow + 8 * G + 4 * hh);
#pragma unroll
          for (int j = 0; j < 4; ++j) qff[4 * G + j] = z[j];
        }
      }
    }

    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = (f32x16_t){};
    float m_run = -INFINITY;  // running max of log2-domain scores
    float l_run = 0.f;        // this half's partial row sum

    const T* kbase = kg + (size_t)k0 * kstride + (size_t)g * D;
    const T* vbase = vg + (size_t)k0 * kstride + (size_t)g * D;
    const T* bias_bh = nullptr;
    if constexpr (HAS_BIAS)
      bias_bh = (const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1 +
                (int64_t)max(rq, 0) * a.bs2;

    Loader<BF16, D> ld;
    if (nblk > 0) {
      ld.load(kbase, vbase, kstride, kb0, 0, kv_hi);
      ld.store(sm, 0);
    }
    __syncthreads();

    for (int n = 0; n < nblk; ++n) {
      const int kb = kb0 + n * BN;
      const int buf = n & 1;
      if (n + 1 < nblk) ld.load(kbase, vbase, kstride, kb + BN, 0, kv_hi);

      if (wave_on && kb < wave_hi) {
        // ---- S^T = K Q^T for two 32-key tiles
        f32x16_t s[NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          s[st] = (f32x16_t){};
          const T* krow = &sm.k[buf][(32 * st + r32) * S::KP];
          if constexpr (BF16) {
#pragma unroll
            for (int ks = 0; ks < QF; ++ks) {
              u32x4_t ka = *(const u32x4_t*)(krow + 16 * ks + 8 * hh);
              s[st] = mfma32_bf16(ka, qf4[ks], s[st]);
            }
          } else {
#pragma unroll
            for (int G = 0; G < D / 8; ++G) {
              f32x4_t ka = *(const f32x4_t*)(krow + 8 * G + 4 * hh);
#pragma unroll
              for (int j = 0; j < 4; ++j) s[st] = mfma32_f32(ka[j], qff[4 * G + j], s[st]);
            }
          }
        }
        // ---- scale, bias, mask (log2 domain)
        const bool need_mask = (kb < 0) || (kb + BN > kv_hi) ||
                               (CAUSAL && (kb + BN - 1 > w0 + off));
        float x[16 * NS];
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = kb + 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
            float v = s[st][i] * a.scale_log2;
            if constexpr (HAS_BIAS) {
              if (row_ok && kj >= 0 && kj < Lk) {
                T bv = bias_bh[(int64_t)kj * a.bs3];
                float bf;
                if constexpr (BF16) bf = bf16_to_f32(bv); else bf = bv;
                v = __builtin_fmaf(bf, kLog2e, v);
              }
            }
            if (need_mask) {
              bool ok = kj >= 0 && kj < kv_hi && (!CAUSAL || kj <= rq + off);
              v = ok ? v : -INFINITY;
            }
            x[16 * st + i] = v;
          }
        // ---- online softmax
        float mx = x[0];
#pragma unroll
        for (int i = 1; i < 16 * NS; ++i) mx = fmaxf(mx, x[i]);
        mx = fmaxf(mx, xor32(mx));
        const float m_new = fmaxf(m_run, mx);
        const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
        const float alpha = fast_exp2(m_run - m_use);
        m_run = m_new;
        float psum = 0.f;
#pragma unroll
        for (int i = 0; i < 16 * NS; ++i) {
          x[i] = fast_exp2(x[i] - m_use);
          psum += x[i];
        }
        l_run = l_run * alpha + psum;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
        // ---- O^T += V^T P^T
        if constexpr (BF16) {
#pragma unroll
          for (int kc = 0; kc < 2 * NS; ++kc) {  // 16-key chunks
            u32x4_t pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) pb[e] = pack_bf16x2(x[8 * kc + 2 * e], x[8 * kc + 2 * e + 1]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              u32x4_t va = *(const u32x4_t*)(&sm.v[buf][(32 * dt + r32) * S::VP + 16 * kc + 8 * hh]);
              acc[dt] = mfma32_bf16(va, pb, acc[dt]);
            }
          }
        } else {
#pragma unroll
          for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) {
                float va = sm.v[buf][key * S::VP + 32 * dt + r32];
                acc[dt] = mfma32_f32(va, x[16 * st + i], acc[dt]);
              }
            }
        }
      }
      if (n + 1 < nblk) ld.store(sm, buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2
    const float l_tot = l_run + xor32(l_run);
    const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
    if (row_ok) {
      T* orow = og + (size_t)(q0 + rq) * qstride + (size_t)h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt + 8 * a4 + 4 * hh;
          float o0 = acc[dt][4 * a4 + 0] * inv_l, o1 = acc[dt][4 * a4 + 1] * inv_l;
          float o2 = acc[dt][4 * a4 + 2] * inv_l, o3 = acc[dt][4 * a4 + 3] * inv_l;
          if constexpr (BF16) {
            u32x2_t w = {pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
            *(u32x2_t*)(orow + d0) = w;
          } else {
            *(f32x4_t*)(orow + d0) = (f32x4_t){o0, o1, o2, o3};
          }
        }
      if (hh == 0) {
        const float lse = l_tot > 0.f ? (m_run + __builtin_log2f(l_tot)) * kLn2 : -INFINITY;
        a.lse[(size_t)h * a.total_q + q0 + rq] = lse;
      }
    }
  }
}

}  // namespace

template <bool BF16, int D, bool CAUSAL, bool HAS_BIAS>
static hipError_t launch_fwd_t(const FwdArgs& a, int64_t items, hipStream_t st) {
  auto kern = fwd_kernel<BF16, D, CAUSAL, HAS_BIAS>;
  const int grid = resident_grid((const void*)kern, NT, items);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  timing_before(st, BF16 ? "fwd_bf16" : "fwd_f32");
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a);
  timing_after(st);
  return hipGetLastError();
}

template <bool BF16, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, int64_t grid, hipStream_t st) {
  const bool has_bias = a.bias != nullptr;
  if (a.causal)
    return has_bias ? launch_fwd_t<BF16, D, true, true>(a, grid, st)
                    : launch_fwd_t<BF16, D, true, false>(a, grid, st);
  return has_bias ? launch_fwd_t<BF16, D, false, true>(a, grid, st)
                  : launch_fwd_t<BF16, D, false, false>(a, grid, st);
}

int fwd_block_m() { return BM; }

hipError_t launch_fwd(const FwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.bf16) return a.d == 64 ? launch_fwd_d<true, 64>(a, grid, st) : launch_fwd_d<true, 128>(a, grid, st);
  return a.d == 64 ? launch_fwd_d<false, 64>(a, grid, st) : launch_fwd_d<false, 128>(a, grid, st);
}

}  // namespace va
