// Backward kernels: dQ, dK, dV of exact packed varlen attention, recomputing
// the softmax from the forward's log-sum-exp instead of storing it.
//
//   D_i = sum_d dO_i,d O_i,d                      (preprocess)
//   P   = exp(scale * Q K^T + bias - LSE)         (masked entries 0)
//   dP  = dO V^T,  dS = P * (dP - D)
//   dV  = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K
//
// dK/dV kernel: a workgroup owns 128 keys (32 per wave) of one sequence and
// KV head; K and V stay in registers, and the workgroup walks the query
// blocks (and the query heads of its GQA group) that see those keys, staging
// Q and dO in LDS both as rows and transposed (for the contractions over
// queries).  When the group's heads are split over several workgroups, each
// writes float32 partial sums to the workspace and a reduce kernel adds them
// in a fixed order, so results never depend on scheduling.
//
// dQ kernel: shaped like the forward.  A workgroup owns 128 query rows of one
// head; Q and dO stay in registers; the score tile is computed transposed
// (keys x queries) so each lane holds one query row, and dS^T feeds the dQ^T
// contraction straight from registers.
#include "va_common.h"
#include "va_kernels.h"

namespace va {

namespace {

constexpr int NT = 256;
constexpr int BNK = 128;  // keys per dK/dV workgroup
constexpr int BMQ_DQ = 128;  // query rows per dQ workgroup

template <bool BF16>
using elem_t = typename std::conditional<BF16, uint16_t, float>::type;

// Row r (0..) position inside a transposed bf16 LDS row: bits 2 and 3 of r
// swapped, so the 8 k-slots of a lane half are contiguous (see va_fwd.hip).
__device__ __forceinline__ int tpos(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

// Stages a [ROWS][D] block of a token-major tensor into LDS: as rows
// ([ROWS][D + pad]) and, for bf16, transposed ([D][ROWS + pad], rows permuted
// by tpos).  Each thread owns pairs of consecutive rows of one 16-byte column
// chunk so the transposed store can pair them.
template <bool BF16, int ROWS, int D, bool TRANS>
struct Stager {
  using T = elem_t<BF16>;
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int CH = D / EPV;                 // 16-byte chunks per row
  static constexpr int PAIRS = (ROWS / 2) * CH;      // tasks
  static constexpr int TPT = (PAIRS + NT - 1) / NT;  // tasks per thread
  static constexpr int NP = D + 16 / (int)sizeof(T);     // row pitch (elements)
  static constexpr int TP = ROWS + 16 / (int)sizeof(T);  // transposed pitch
  u32x4_t r[2 * TPT];

  __device__ __forceinline__ void load(const T* __restrict__ base, size_t row_stride, int row0,
                                       int rhi) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int c = u % CH, p = u / CH;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        const int row = row0 + 2 * p + e;
        u32x4_t z = {0, 0, 0, 0};
        if (u < PAIRS && row >= 0 && row < rhi)
          z = *(const u32x4_t*)(base + (size_t)row * row_stride + c * EPV);
        r[2 * i + e] = z;
      }
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ dn, T* __restrict__ dt) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int u = threadIdx.x + i * NT;
      if (u >= PAIRS) continue;
      const int c = u % CH, p = u / CH;
      *(u32x4_t*)(dn + (2 * p) * NP + c * EPV) = r[2 * i];
      *(u32x4_t*)(dn + (2 * p + 1) * NP + c * EPV) = r[2 * i + 1];
      if constexpr (BF16 && TRANS) {
        const int pos = tpos(2 * p);
        const u32x4_t a = r[2 * i], b = r[2 * i + 1];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          uint32_t lo = (a[e] & 0xFFFFu) | (b[e] << 16);
          uint32_t hi = (a[e] >> 16) | (b[e] & 0xFFFF0000u);
          *(uint32_t*)(dt + (c * 8 + 2 * e) * TP + pos) = lo;
          *(uint32_t*)(dt + (c * 8 + 2 * e + 1) * TP + pos) = hi;
        }
      }
    }
  }
};

// Register fragment of one row (this lane's row) for the "other" operand of
// a 32x32 MFMA contracting over head_dim: bf16 -> D/16 vectors of 8; f32 ->
// D/2 scalars with k-slot (group G, step j) of lane half hh = dim 8G+4hh+j.
template <bool BF16, int D>
struct RowFrag {
  static constexpr int N = BF16 ? D / 16 : D / 2;
  u32x4_t b[BF16 ? N : 1];
  float f[BF16 ? 1 : N];
  __device__ __forceinline__ void load(const elem_t<BF16>* row, bool ok, int hh) {
    if constexpr (BF16) {
#pragma unroll
      for (int ks = 0; ks < N; ++ks) {
        u32x4_t z = {0, 0, 0, 0};
        if (ok) z = *(const u32x4_t*)(row + 16 * ks + 8 * hh);
        b[ks] = z;
      }
    } else {
#pragma unroll
      for (int G = 0; G < D / 8; ++G) {
        f32x4_t z = {0.f, 0.f, 0.f, 0.f};
        if (ok) z = *(const f32x4_t*)(row + 8 * G + 4 * hh);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * G + j] = z[j];
      }
    }
  }
};

// acc += (32 rows of an LDS row-major tile, from `lrow` = this lane's row) x
// frag^T, contracting over head_dim.  Result: C[lds row][fragment row].
template <bool BF16, int D>
__device__ __forceinline__ f32x16_t mm_rows(const elem_t<BF16>* lrow, const RowFrag<BF16, D>& fr,
                                            f32x16_t acc, int hh) {
  if constexpr (BF16) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4_t a = *(const u32x4_t*)(lrow + 16 * ks + 8 * hh);
      acc = mfma32_bf16(a, fr.b[ks], acc);
    }
  } else {
#pragma unroll
    for (int G = 0; G < D / 8; ++G) {
      f32x4_t a = *(const f32x4_t*)(lrow + 8 * G + 4 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma32_f32(a[j], fr.f[4 * G + j], acc);
    }
  }
  return acc;
}

__device__ __forceinline__ float ld_bias(const uint16_t* p) { return bf16_to_f32(*p); }
__device__ __forceinline__ float ld_bias(const float* p) { return *p; }

// ---------------------------------------------------------------- preprocess
template <bool BF16, int D>
__global__ __launch_bounds__(NT) void dsum_kernel(BwdArgs a) {
  using T = elem_t<BF16>;
  constexpr int EPV = 16 / sizeof(T);
  constexpr int TPR = D / EPV;  // threads per (token, head) row
  const int64_t rows = (int64_t)a.total_q * a.hq;
  const int64_t row = ((int64_t)blockIdx.x * NT + threadIdx.x) / TPR;
  const int c = threadIdx.x % TPR;
  float s = 0.f;
  if (row < rows) {
    const T* o = (const T*)a.out + row * D + c * EPV;
    const T* g = (const T*)a.dout + row * D + c * EPV;
    if constexpr (BF16) {
      const u32x4_t x = *(const u32x4_t*)o, y = *(const u32x4_t*)g;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = __builtin_fmaf(bf16_to_f32(x[e] & 0xFFFF), bf16_to_f32(y[e] & 0xFFFF), s);
        s = __builtin_fmaf(bf16_to_f32(x[e] >> 16), bf16_to_f32(y[e] >> 16), s);
      }
    } else {
      // float vectors are loaded as such (no bit casts of vector elements)
      const f32x4_t x = *(const f32x4_t*)o, y = *(const f32x4_t*)g;
#pragma unroll
      for (int e = 0; e < 4; ++e) s = __builtin_fmaf(x[e], y[e], s);
    }
  }
#pragma unroll
  for (int o = TPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
  if (row < rows && c == 0) {
    const int t = (int)(row / a.hq), h = (int)(row % a.hq);
    a.dsum[(size_t)h * a.total_q + t] = s;
  }
}

// ---------------------------------------------------------------- dK / dV
template <bool BF16, int D>
struct DkdvSmem {
  using T = elem_t<BF16>;
  static constexpr int BMQ = D == 128 ? 32 : 64;
  using St = Stager<BF16, BMQ, D, true>;
  T qn[2][BMQ * St::NP];
  T dn[2][BMQ * St::NP];
  T qt[2][BF16 ? D * St::TP : 1];
  T dt[2][BF16 ? D * St::TP : 1];
  float lse2[2][BMQ];
  float dsum[2][BMQ];
};

template <bool BF16, int D, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(NT, 1) void dkdv_kernel(BwdArgs a, int hsplit, float* part) {
  using T = elem_t<BF16>;
  using SM = DkdvSmem<BF16, D>;
  constexpr int BMQ = SM::BMQ;
  constexpr int NQ = BMQ / 32;  // 32-query score tiles per block
  constexpr int DT = D / 32;
  using St = typename SM::St;

  __shared__ SchedShared sched;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int hh = lane >> 5, r32 = lane & 31;

  sched_build(sched, a.cu_k, a.batch, a.total_k, BNK, a.tcap_k, a.stride_k, a.nlev_k);
  const int per_tile = a.hkv * hsplit;
  const int total_items = sched.total_tiles * per_tile;
  const size_t qstride = (size_t)a.hq * D, kstride = (size_t)a.hkv * D;
  const int hpw = a.n_rep / hsplit;  // query heads per workgroup

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int tile = item / per_tile;
    const int rem = item - tile * per_tile;
    const int g = rem / hsplit, sp = rem - g * hsplit;
    int b, t;
    sched_find(sched, a.cu_k, a.batch, a.total_k, BNK, a.tcap_k, a.stride_k, a.nlev_k, tile, b, t);
    int q0, q1, k0, k1;
    seq_bounds(a.cu_q, b, a.total_q, q0, q1);
    seq_bounds(a.cu_k, b, a.total_k, k0, k1);
    q0 = uniform(q0); q1 = uniform(q1); k0 = uniform(k0); k1 = uniform(k1);
    const int Lq = q1 - q0, Lk = k1 - k0, off = Lk - Lq;
    const int kt0 = t * BNK;
    const int wk0 = kt0 + 32 * wid;  // first key of this wave
    const int kj = wk0 + r32;        // this lane's key (columns of the score tile)
    const bool key_ok = kj < Lk;
    const bool wave_keys = wk0 < Lk;

    RowFrag<BF16, D> kf, vf;
    {
      const T* krow = (const T*)a.k + (size_t)(k0 + min(kj, max(Lk - 1, 0))) * kstride + (size_t)g * D;
      const T* vrow = (const T*)a.v + (size_t)(k0 + min(kj, max(Lk - 1, 0))) * kstride + (size_t)g * D;
      kf.load(krow, key_ok, hh);
      vf.load(vrow, key_ok, hh);
    }
    f32x16_t dk[DT], dv[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) { dk[i] = (f32x16_t){}; dv[i] = (f32x16_t){}; }

    // queries that can see key kt0: i + off >= kt0
    const int qs = CAUSAL ? max(0, kt0 - off) : 0;
    const int nqb = qs < Lq ? (Lq - qs + BMQ - 1) / BMQ : 0;
    const int niter = nqb * hpw;
    const int h_first = g * a.n_rep + sp * hpw;

    St sq, sd;
    float pl = 0.f, pd = 0.f;  // staged lse2 / dsum for thread tid < BMQ
    auto issue = [&](int it) {
      const int r = it / nqb, n = it - r * nqb;
      const int h = h_first + r;
      const int qb = qs + n * BMQ;
      sq.load((const T*)a.q + (size_t)q0 * qstride + (size_t)h * D, qstride, qb, Lq);
      sd.load((const T*)a.dout + (size_t)q0 * qstride + (size_t)h * D, qstride, qb, Lq);
      if (tid < BMQ) {
        const int i = qb + tid;
        pl = 0.f; pd = 0.f;
        if (i < Lq) {
          pl = a.lse[(size_t)h * a.total_q + q0 + i] * kLog2e;
          pd = a.dsum[(size_t)h * a.total_q + q0 + i];
        }
      }
    };
    auto commit = [&](int buf) {
      sq.store(sm.qn[buf], sm.qt[buf]);
      sd.store(sm.dn[buf], sm.dt[buf]);
      if (tid < BMQ) { sm.lse2[buf][tid] = pl; sm.dsum[buf][tid] = pd; }
    };

    if (niter > 0) { issue(0); commit(0); }
    __syncthreads();
    for (int it = 0; it < niter; ++it) {
      const int buf = it & 1;
      const int r = it / nqb, n = it - r * nqb;
      const int h = h_first + r;
      const int qb = qs + n * BMQ;
      if (it + 1 < niter) issue(it + 1);
      // this wave's keys are seen by queries i >= wk0 - off
      const bool active = wave_keys && (!CAUSAL || qb + BMQ - 1 + off >= wk0);
      if (active) {
        const bool need_mask = (qb + BMQ > Lq) || (wk0 + 32 > Lk) || (CAUSAL && qb + off < wk0 + 31);
        const T* bias_h = nullptr;
        if constexpr (HAS_BIAS)
          bias_h = (const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1 + (int64_t)kj * a.bs3;
        f32x16_t p[NQ], ds[NQ];
#pragma unroll
        for (int qt = 0; qt < NQ; ++qt) {
          // S = Q K^T and dP = dO V^T: C[query][key], lane = key
          f32x16_t s = mm_rows<BF16, D>(&sm.qn[buf][(32 * qt + r32) * St::NP], kf, (f32x16_t){}, hh);
          f32x16_t dp = mm_rows<BF16, D>(&sm.dn[buf][(32 * qt + r32) * St::NP], vf, (f32x16_t){}, hh);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = 32 * qt + 8 * (i >> 2) + 4 * hh + (i & 3);  // query inside block
            const int qi = qb + ql;
            float x = s[i] * a.scale_log2;
            if constexpr (HAS_BIAS) {
              if (qi < Lq && key_ok) x = __builtin_fmaf(ld_bias(bias_h + (int64_t)qi * a.bs2), kLog2e, x);
            }
            float pv = fast_exp2(x - sm.lse2[buf][ql]);
            if (need_mask) {
              const bool ok = qi < Lq && key_ok && (!CAUSAL || kj <= qi + off);
              pv = ok ? pv : 0.f;
            }
            p[qt][i] = pv;
            ds[qt][i] = pv * (dp[i] - sm.dsum[buf][ql]);
          }
        }
        // dV += P^T dO, dK += dS^T Q: C[key][d], lane = d
        if constexpr (BF16) {
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              u32x4_t pa, da;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                pa[e] = pack_bf16x2(p[qt][8 * c + 2 * e], p[qt][8 * c + 2 * e + 1]);
                da[e] = pack_bf16x2(ds[qt][8 * c + 2 * e], ds[qt][8 * c + 2 * e + 1]);
              }
              const int col = 32 * qt + 16 * c + 8 * hh;
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) {
                u32x4_t ob = *(const u32x4_t*)(&sm.dt[buf][(32 * dt + r32) * St::TP + col]);
                u32x4_t qb4 = *(const u32x4_t*)(&sm.qt[buf][(32 * dt + r32) * St::TP + col]);
                dv[dt] = mfma32_bf16(pa, ob, dv[dt]);
                dk[dt] = mfma32_bf16(da, qb4, dk[dt]);
              }
            }
        } else {
#pragma unroll
          for (int qt = 0; qt < NQ; ++qt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int ql = 32 * qt + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) {
                const float ob = sm.dn[buf][ql * St::NP + 32 * dt + r32];
                const float qv = sm.qn[buf][ql * St::NP + 32 * dt + r32];
                dv[dt] = mfma32_f32(p[qt][i], ob, dv[dt]);
                dk[dt] = mfma32_f32(ds[qt][i], qv, dk[dt]);
              }
            }
        }
      }
      if (it + 1 < niter) commit(buf ^ 1);
      __syncthreads();
    }

    // ---- epilogue: rows = keys 8(i/4)+4hh+i%4 of the wave, column d = 32dt + r32
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int key = wk0 + 8 * (i >> 2) + 4 * hh + (i & 3);
        if (key >= Lk) continue;
        const size_t o = (size_t)(k0 + key) * kstride + (size_t)g * D + 32 * dt + r32;
        const float kv = dk[dt][i], vv = dv[dt][i];
        if (hsplit > 1) {
          const size_t plane = (size_t)a.total_k * kstride;
          part[(size_t)(2 * sp) * plane + o] = kv;
          part[(size_t)(2 * sp + 1) * plane + o] = vv;
        } else if (a.grad_bf16) {
          ((uint16_t*)a.dk)[o] = (uint16_t)(pack_bf16x2(kv * a.scale, 0.f) & 0xFFFF);
          ((uint16_t*)a.dv)[o] = (uint16_t)(pack_bf16x2(vv, 0.f) & 0xFFFF);
        } else {
          ((float*)a.dk)[o] = kv * a.scale;
          ((float*)a.dv)[o] = vv;
        }
      }
  }
}

// Adds the head-split partial sums of dK and dV in a fixed order.
__global__ __launch_bounds__(NT) void dkdv_reduce_kernel(BwdArgs a, int hsplit, const float* part) {
  const size_t plane = (size_t)a.total_k * a.hkv * a.d;
  const size_t n4 = plane / 4;
  for (size_t i = (size_t)blockIdx.x * NT + threadIdx.x; i < n4; i += (size_t)gridDim.x * NT) {
    f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = {0.f, 0.f, 0.f, 0.f};
    for (int s = 0; s < hsplit; ++s) {
      sk += ((const f32x4_t*)(part + (size_t)(2 * s) * plane))[i];
      sv += ((const f32x4_t*)(part + (size_t)(2 * s + 1) * plane))[i];
    }
    sk *= a.scale;
    if (a.grad_bf16) {
      ((u32x2_t*)a.dk)[i] = (u32x2_t){pack_bf16x2(sk[0], sk[1]), pack_bf16x2(sk[2], sk[3])};
      ((u32x2_t*)a.dv)[i] = (u32x2_t){pack_bf16x2(sv[0], sv[1]), pack_bf16x2(sv[2], sv[3])};
    } else {
      ((f32x4_t*)a.dk)[i] = sk;
      ((f32x4_t*)a.dv)[i] = sv;
    }
  }
}

// ---------------------------------------------------------------- dQ
template <bool BF16, int D>
struct DqSmem {
  using T = elem_t<BF16>;
  static constexpr int BN = (BF16 && D == 64) ? 64 : 32;
  using St = Stager<BF16, BN, D, true>;
  using Sv = Stager<BF16, BN, D, false>;
  T kn[2][BN * St::NP];
  T kt[2][BF16 ? D * St::TP : 1];
  T vn[2][BN * St::NP];
};

template <bool BF16, int D, bool CAUSAL, bool HAS_BIAS>
__global__ __launch_bounds__(NT, 2) void dq_kernel(BwdArgs a) {
  using T = elem_t<BF16>;
  using SM = DqSmem<BF16, D>;
  constexpr int BN = SM::BN;
  constexpr int NS = BN / 32;
  constexpr int DT = D / 32;
  using St = typename SM::St;
  using Sv = typename SM::Sv;

  __shared__ SchedShared sched;
  __shared__ SM sm;

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int hh = lane >> 5, r32 = lane & 31;

  sched_build(sched, a.cu_q, a.batch, a.total_q, BMQ_DQ, a.tcap_q, a.stride_q, a.nlev_q);
  const int total_items = sched.total_tiles * a.hq;
  const size_t qstride = (size_t)a.hq * D, kstride = (size_t)a.hkv * D;

  for (int item = blockIdx.x; item < total_items; item += gridDim.x) {
    const int tile = item / a.hq;
    const int h = item - tile * a.hq;
    int b, t;
    sched_find(sched, a.cu_q, a.batch, a.total_q, BMQ_DQ, a.tcap_q, a.stride_q, a.nlev_q, tile, b, t);
    int q0, q1, k0, k1;
    seq_bounds(a.cu_q, b, a.total_q, q0, q1);
    seq_bounds(a.cu_k, b, a.total_k, k0, k1);
    q0 = uniform(q0); q1 = uniform(q1); k0 = uniform(k0); k1 = uniform(k1);
    const int Lq = q1 - q0, Lk = k1 - k0, off = Lk - Lq;
    const int g = h / a.n_rep;
    const int r1 = Lq - t * BMQ_DQ;
    const int w0 = r1 - BMQ_DQ + 32 * wid;
    const int rq = w0 + r32;
    const bool row_ok = rq >= 0;
    const int kv_hi = CAUSAL ? min(Lk, r1 + off) : Lk;
    const int wave_hi = CAUSAL ? min(Lk, w0 + 32 + off) : Lk;
    const bool wave_on = (w0 + 31 >= 0) && wave_hi > 0;
    const int nblk = kv_hi > 0 ? (kv_hi + BN - 1) / BN : 0;
    const int kb0 = CAUSAL ? kv_hi - nblk * BN : 0;

    RowFrag<BF16, D> qf, of;
    {
      const size_t ro = (size_t)(q0 + max(rq, 0)) * qstride + (size_t)h * D;
      qf.load((const T*)a.q + ro, row_ok, hh);
      of.load((const T*)a.dout + ro, row_ok, hh);
    }
    float lse2 = 0.f, dsum = 0.f;
    if (row_ok) {
      lse2 = a.lse[(size_t)h * a.total_q + q0 + rq] * kLog2e;
      dsum = a.dsum[(size_t)h * a.total_q + q0 + rq];
    }
    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = (f32x16_t){};

    const T* kbase = (const T*)a.k + (size_t)k0 * kstride + (size_t)g * D;
    const T* vbase = (const T*)a.v + (size_t)k0 * kstride + (size_t)g * D;
    const T* bias_bh = nullptr;
    if constexpr (HAS_BIAS)
      bias_bh = (const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1 + (int64_t)max(rq, 0) * a.bs2;

    St sk;
    Sv sv;
    if (nblk > 0) {
      sk.load(kbase, kstride, kb0, kv_hi);
      sv.load(vbase, kstride, kb0, kv_hi);
      sk.store(sm.kn[0], sm.kt[0]);
      sv.store(sm.vn[0], nullptr);
    }
    __syncthreads();
    for (int n = 0; n < nblk; ++n) {
      const int kb = kb0 + n * BN;
      const int buf = n & 1;
      if (n + 1 < nblk) {
        sk.load(kbase, kstride, kb + BN, kv_hi);
        sv.load(vbase, kstride, kb + BN, kv_hi);
      }
      if (wave_on && kb < wave_hi) {
        const bool need_mask = (kb < 0) || (kb + BN > kv_hi) || (CAUSAL && (kb + BN - 1 > w0 + off));
        float dsv[16 * NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          // S^T = K Q^T, dP^T = V dO^T: C[key][query], lane = query
          f32x16_t s = mm_rows<BF16, D>(&sm.kn[buf][(32 * st + r32) * St::NP], qf, (f32x16_t){}, hh);
          f32x16_t dp = mm_rows<BF16, D>(&sm.vn[buf][(32 * st + r32) * St::NP], of, (f32x16_t){}, hh);
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int kj = kb + 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
            float x = s[i] * a.scale_log2;
            if constexpr (HAS_BIAS) {
              if (row_ok && kj >= 0 && kj < Lk) x = __builtin_fmaf(ld_bias(bias_bh + (int64_t)kj * a.bs3), kLog2e, x);
            }
            float pv = fast_exp2(x - lse2);
            if (need_mask) {
              const bool ok = row_ok && kj >= 0 && kj < kv_hi && (!CAUSAL || kj <= rq + off);
              pv = ok ? pv : 0.f;
            }
            dsv[16 * st + i] = pv * (dp[i] - dsum);
          }
        }
        // dQ^T += K^T dS^T
        if constexpr (BF16) {
#pragma unroll
          for (int kc = 0; kc < 2 * NS; ++kc) {
            u32x4_t pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) pb[e] = pack_bf16x2(dsv[8 * kc + 2 * e], dsv[8 * kc + 2 * e + 1]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) {
              u32x4_t ka = *(const u32x4_t*)(&sm.kt[buf][(32 * dt + r32) * St::TP + 16 * kc + 8 * hh]);
              acc[dt] = mfma32_bf16(ka, pb, acc[dt]);
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
                const float ka = sm.kn[buf][key * St::NP + 32 * dt + r32];
                acc[dt] = mfma32_f32(ka, dsv[16 * st + i], acc[dt]);
              }
            }
        }
      }
      if (n + 1 < nblk) {
        sk.store(sm.kn[buf ^ 1], sm.kt[buf ^ 1]);
        sv.store(sm.vn[buf ^ 1], nullptr);
      }
      __syncthreads();
    }

    if (row_ok) {
      const size_t ro = (size_t)(q0 + rq) * qstride + (size_t)h * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt + 8 * a4 + 4 * hh;
          const float o0 = acc[dt][4 * a4 + 0] * a.scale, o1 = acc[dt][4 * a4 + 1] * a.scale;
          const float o2 = acc[dt][4 * a4 + 2] * a.scale, o3 = acc[dt][4 * a4 + 3] * a.scale;
          if (a.grad_bf16) {
            *(u32x2_t*)((uint16_t*)a.dq + ro + d0) = (u32x2_t){pack_bf16x2(o0, o1), pack_bf16x2(o2, o3)};
          } else {
            *(f32x4_t*)((float*)a.dq + ro + d0) = (f32x4_t){o0, o1, o2, o3};
          }
        }
    }
  }
}

template <bool BF16, int D, bool CAUSAL, bool HAS_BIAS>
hipError_t launch_bwd_t(const BwdArgs& a, int64_t q_items, int64_t k_items, hipStream_t st) {
  {
    constexpr int EPV = BF16 ? 8 : 4;
    const int64_t threads = (int64_t)a.total_q * a.hq * (D / EPV);
    const int64_t grid = (threads + NT - 1) / NT;
    timing_before(st, "bwd_dsum");
    hipLaunchKernelGGL((dsum_kernel<BF16, D>), dim3((unsigned)grid), dim3(NT), 0, st, a);
    timing_after(st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    auto kern = dkdv_kernel<BF16, D, CAUSAL, HAS_BIAS>;
    const int hsplit = a.hsplit;
    const int grid = resident_grid((const void*)kern, NT, k_items * hsplit);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    timing_before(st, BF16 ? "bwd_dkdv_bf16" : "bwd_dkdv_f32");
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a, hsplit, a.part);
    timing_after(st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    if (hsplit > 1) {
      const size_t n4 = (size_t)a.total_k * a.hkv * D / 4;
      int64_t g = (int64_t)((n4 + NT - 1) / NT);
      if (g > 4096) g = 4096;
      timing_before(st, "bwd_dkdv_reduce");
      hipLaunchKernelGGL(dkdv_reduce_kernel, dim3((unsigned)g), dim3(NT), 0, st, a, hsplit,
                         (const float*)a.part);
      timing_after(st);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  {
    auto kern = dq_kernel<BF16, D, CAUSAL, HAS_BIAS>;
    const int grid = resident_grid((const void*)kern, NT, q_items);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    timing_before(st, BF16 ? "bwd_dq_bf16" : "bwd_dq_f32");
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a);
    timing_after(st);
  }
  return hipGetLastError();
}

template <bool BF16, int D>
hipError_t launch_bwd_d(const BwdArgs& a, int64_t q_items, int64_t k_items, hipStream_t st) {
  const bool hb = a.bias != nullptr;
  if (a.causal)
    return hb ? launch_bwd_t<BF16, D, true, true>(a, q_items, k_items, st)
              : launch_bwd_t<BF16, D, true, false>(a, q_items, k_items, st);
  return hb ? launch_bwd_t<BF16, D, false, true>(a, q_items, k_items, st)
            : launch_bwd_t<BF16, D, false, false>(a, q_items, k_items, st);
}

}  // namespace

int bwd_block_q() { return BMQ_DQ; }
int bwd_block_k() { return BNK; }

hipError_t launch_bwd(const BwdArgs& a, int64_t q_items, int64_t k_items, hipStream_t st) {
  if (a.bf16)
    return a.d == 64 ? launch_bwd_d<true, 64>(a, q_items, k_items, st)
                     : launch_bwd_d<true, 128>(a, q_items, k_items, st);
  return a.d == 64 ? launch_bwd_d<false, 64>(a, q_items, k_items, st)
                   : launch_bwd_d<false, 128>(a, q_items, k_items, st);
}

}  // namespace va
