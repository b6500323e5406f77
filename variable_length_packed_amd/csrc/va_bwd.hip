// Backward kernels: dQ, dK, dV of exact packed varlen attention, recomputing
// the softmax from the forward's log-sum-exp instead of storing it.
//
//   D_i = sum_d dO_i,d O_i,d                      (preprocess)
//   P   = exp(scale * Q K^T + bias - LSE)         (masked entries 0)
//   dP  = dO V^T,  dS = P * (dP - D)
//   dV  = P^T dO,  dK = scale * dS^T Q,  dQ = scale * dS K
//
// dK/dV kernel: a work unit is 128 keys (32 per wave) of one sequence and KV
// head; K and V stay in registers while the workgroup walks the 32-query
// blocks that see those keys, for every query head of the GQA group, staging
// Q and dO in LDS as rows: read as rows for S and dP, and with transposing LDS
// reads for the contractions over queries.  A key tile seen by many query
// blocks is split into units over ranges of query blocks; those write float32
// partial sums that the dQ pass, after its own items, adds in chunk order, so
// results never depend on scheduling.
//
// dQ kernel: shaped like the forward.  A unit is 128 query rows of one head
// (or a range of key blocks of them, whose last chunk to finish adds the
// chunks' float32 partial sums in chunk order); Q and dO stay in
// registers; score tiles are computed transposed (keys x queries) so each
// lane holds one query row and dS^T feeds the dQ^T contraction straight from
// registers.
//
// Both take their units from the planner's list, heaviest first: workgroup w
// starts with item w and takes each later item from the list's cursor near
// the end of its current one (NextItem).
//
// No mask is needed for a key past the sequence (its K and V read as zero and
// its dK/dV row is never stored; in dQ its zero K row adds nothing) or for a
// query row past it (its staged LSE is +inf, so its P is 0).  Only tiles that
// cross the causal diagonal take the masked path, in a loop of their own.
//
// bf16: P and dS are rounded to bf16 for the MFMA.  For dK the rounding error
// of dS is carried by a second bf16 operand (the residual dS - bf16(dS)), so
// that contraction is exact to float32 accumulation; dV (P >= 0, errors of
// both signs cancel) and dQ use the plain rounding.
#include "va_common.h"
#include "va_kernels.h"
#include "va_plan.h"

namespace va {

namespace {

constexpr int NT = 256;
constexpr int BNK = 128;     // keys per dK/dV workgroup
// query heads per KV head with a per-key bias gradient (an LDS accumulator per
// head; fewer at head_dim 256, whose Q/dO staging fills most of the LDS)
template <int D>
constexpr int dbias_max_heads() { return D <= 128 ? 32 : 8; }
constexpr int BMQ_DQ = 128;  // query rows per dQ workgroup

template <int H16>
using elem_t = typename std::conditional<(H16 != 0), uint16_t, float>::type;

// Stages a [ROWS][D] block (rows row0 .. of a buffer resource; rows outside
// read as zero) into LDS rows ([ROWS][D + pad]), one 16-byte piece per task,
// consecutive threads along a row.  The 16-bit operands that contract over
// the rows (dO^T and Q^T in dK/dV, K^T in dQ) are read from these rows with
// transposing LDS reads (tr_frag), so no transposed copy is ever written.
template <int H16, int ROWS, int D>
struct Stager {
  using T = elem_t<H16>;
  static constexpr int EPV = 16 / sizeof(T);
  static constexpr int CH = D / EPV;                  // 16-byte pieces per row
  static constexpr int TASKS = ROWS * CH;
  static constexpr int TPT = (TASKS + NT - 1) / NT;   // pieces per thread
  static constexpr int NP = D + 16 / (int)sizeof(T);  // row pitch (elements)
  u32x4_t r[TPT];

  __device__ __forceinline__ void load(rsrc_t res, int row_bytes, int row0) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int u = threadIdx.x + i * NT;
      if (TASKS % NT != 0 && u >= TASKS) continue;  // a partial last round
      const int c = u % CH, row = u / CH;
      r[i] = buf_load16(res, (row0 + row) * row_bytes + c * 16);
    }
  }

  __device__ __forceinline__ void store(T* __restrict__ dn) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int u = threadIdx.x + i * NT;
      if (TASKS % NT != 0 && u >= TASKS) continue;  // a partial last round
      const int c = u % CH, row = u / CH;
      *(u32x4_t*)(dn + row * NP + c * EPV) = r[i];
    }
  }
  // the same rows unpadded, in the swizzled order of swz()
  __device__ __forceinline__ void store_swz(T* __restrict__ dn) {
#pragma unroll
    for (int i = 0; i < TPT; ++i) {
      const int u = threadIdx.x + i * NT;
      if (TASKS % NT != 0 && u >= TASKS) continue;
      const int c = u % CH, row = u / CH;
      *(u32x4_t*)(dn + swz<D>(row, c * EPV)) = r[i];
    }
  }
};

// Register fragment of this lane's row for the "other" operand of a 32x32
// MFMA contracting over head_dim: bf16 -> D/16 vectors of 8; f32 -> D/2
// scalars with k-slot (group G, step j) of lane half hh = dim 8G+4hh+j.
template <int H16, int D>
struct RowFrag {
  static constexpr int N = H16 ? D / 16 : D / 2;
  u32x4_t b[H16 ? N : 1];
  float f[H16 ? 1 : N];
  __device__ __forceinline__ void load(rsrc_t res, int row_bytes, int row, int hh) {
    if constexpr (H16) {
#pragma unroll
      for (int ks = 0; ks < N; ++ks) b[ks] = buf_load16(res, row * row_bytes + (16 * ks + 8 * hh) * 2);
    } else {
#pragma unroll
      for (int G = 0; G < D / 8; ++G) {
        const u32x4_t z = buf_load16(res, row * row_bytes + (8 * G + 4 * hh) * 4);
#pragma unroll
        for (int j = 0; j < 4; ++j) f[4 * G + j] = __uint_as_float(z[j]);
      }
    }
  }
};

// acc += (32 rows of an LDS row-major tile, from `lrow` = this lane's row) x
// frag^T, contracting over head_dim.  Result: C[lds row][fragment row].
template <int H16, int D>
__device__ __forceinline__ f32x16_t mm_rows(const elem_t<H16>* lrow, const RowFrag<H16, D>& fr,
                                            f32x16_t acc, int hh) {
  if constexpr (H16) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const u32x4_t a = *(const u32x4_t*)(lrow + 16 * ks + 8 * hh);
      acc = mfma16<H16>(a, fr.b[ks], acc);
    }
  } else {
#pragma unroll
    for (int G = 0; G < D / 8; ++G) {
      const f32x4_t a = *(const f32x4_t*)(lrow + 8 * G + 4 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc = mfma32_f32(a[j], fr.f[4 * G + j], acc);
    }
  }
  return acc;
}


// 16-bit operand of 8 values and, optionally, the 16-bit residual of the same 8.
template <int H16>
__device__ __forceinline__ void pack8(const float* v, u32x4_t& hi, u32x4_t* lo) {
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    hi[e] = pack16<H16>(v[2 * e], v[2 * e + 1]);
    if (lo) {
      const float r0 = v[2 * e] - lo16<H16>(hi[e]);
      const float r1 = v[2 * e + 1] - hi16<H16>(hi[e]);
      (*lo)[e] = pack16<H16>(r0, r1);
    }
  }
}

// ---------------------------------------------------------------- preprocess
// One launch: workgroups 0 and 1 build the dK/dV and dQ work plans while the
// others compute D = rowsum(dO * O) for every (query row, head); with plans
// the forward already built (va_varlen_bwd_planned), every workgroup computes D.
// Threads per (token, head) row of the D pass: one per 16-byte piece, padded
// to a power of two so the row's sum is a butterfly inside an aligned group.
template <int H16, int D>
constexpr int dsum_tpr() {
  constexpr int n = D / (H16 ? 8 : 4);
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// D pass: the rows are cut into equal contiguous ranges, one per workgroup,
// and with the planners the launch holds DSUM_WG workgroups (one per CU: no
// CU gets a second round while others idle); a group of TPR threads takes every GPW-th row of its range, DSUM_R
// rows at a time with all their loads issued before the first sum.
constexpr int DSUM_R = 4;
constexpr int DSUM_WG = 256;

template <int H16, int D>
__global__ __launch_bounds__(plan::PT) void plan_dsum_kernel(BwdArgs a, PlanSet ps) {
  __shared__ plan::PlanShared sh;
  const int np = ps.nplans;  // 2, or 0 when the forward built the plans
  if ((int)blockIdx.x < np) {
    plan::plan_body(ps.p[blockIdx.x], sh);
    return;
  }
  using T = elem_t<H16>;
  using V = std::conditional_t<H16 != 0, u32x4_t, f32x4_t>;  // float vectors are loaded as such
  constexpr int EPV = 16 / sizeof(T);
  constexpr int TPR = dsum_tpr<H16, D>();  // threads per (token, head) row; the first D / EPV load
  constexpr int GPW = plan::PT / TPR;      // row groups per workgroup
  static_assert(plan::PT % TPR == 0, "rows must not straddle workgroups");
  // rows are numbered head-major (r = h * total_q + t), so the groups of a wave
  // take consecutive tokens of one head and their D stores are contiguous
  const int64_t rows = (int64_t)a.total_q * a.hq;
  const int64_t nwg = (int64_t)gridDim.x - np, w = (int64_t)blockIdx.x - np;
  const int64_t lo = rows * w / nwg, hi = rows * (w + 1) / nwg;
  const int c = threadIdx.x % TPR;
  const bool small = rows < ((int64_t)1 << 31);  // uniform: 32-bit division where the count allows
  for (int64_t r0 = lo + threadIdx.x / TPR; r0 < hi; r0 += (int64_t)GPW * DSUM_R) {
    V x[DSUM_R], y[DSUM_R];
#pragma unroll
    for (int j = 0; j < DSUM_R; ++j) {
      const int64_t r = r0 + (int64_t)j * GPW;
      if (r < hi && c < D / EPV) {
        int64_t t, h;
        if (small) {
          t = (uint32_t)r % (uint32_t)a.total_q;
          h = (uint32_t)r / (uint32_t)a.total_q;
        } else {
          t = r % a.total_q;
          h = r / a.total_q;
        }
        const int64_t e = (t * a.hq + h) * D + c * EPV;
        x[j] = *(const V*)((const T*)a.out + e);
        y[j] = *(const V*)((const T*)a.dout + e);
      }
    }
#pragma unroll
    for (int j = 0; j < DSUM_R; ++j) {
      const int64_t r = r0 + (int64_t)j * GPW;
      float s = 0.f;
      if (r < hi && c < D / EPV) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if constexpr (H16) {
            s = __builtin_fmaf(lo16<H16>(x[j][e]), lo16<H16>(y[j][e]), s);
            s = __builtin_fmaf(hi16<H16>(x[j][e]), hi16<H16>(y[j][e]), s);
          } else {
            s = __builtin_fmaf(x[j][e], y[j][e], s);
          }
        }
      }
#pragma unroll
      for (int o = TPR / 2; o > 0; o >>= 1) s += __shfl_xor(s, o, 64);
      if (r < hi && c == 0) a.dsum[r] = s;  // D is [Hq][total_q]: element h * total_q + t = r
    }
  }
}

// ---------------------------------------------------------------- dK / dV
constexpr int BMQ = 32;  // queries per dK/dV block

template <int H16, int D>
struct DkdvSmem {
  using T = elem_t<H16>;
  using St = Stager<H16, BMQ, D>;
  T qn[2][BMQ * St::NP];
  T dn[2][BMQ * St::NP];
  float lse2[2][BMQ];
  float ndsum[2][BMQ];  // -D of each query (the dP accumulators start from it)
};

// The direct-staged layout (16-bit inputs without a bias, head_dim 64 or 128):
// Q and dO blocks, and the raw LSE and dsum of their queries, load straight
// into LDS two blocks ahead of the block computed, so three buffers; rows
// unpadded in the swizzled order of swz().  The LSE and dsum are converted in
// place (base 2, -D, rows past the sequence) once they have landed.
template <int H16, int D>
struct DkdvSmemDirect {
  using T = elem_t<H16>;
  __attribute__((aligned(16))) T qn[3][BMQ * D];
  __attribute__((aligned(16))) T dn[3][BMQ * D];
  __attribute__((aligned(16))) float lse2[3][BMQ];
  __attribute__((aligned(16))) float ndsum[3][BMQ];
};

template <int H16, int D>
constexpr int dkdv_min_blocks() { return D <= 64 ? 2 : 1; }

// BIAS: 0 none; 1 any layout (one element per load); 2 contiguous keys in 16-byte
// aligned rows (the step's tile staged in LDS with Q and dO)
template <int H16, int D, bool CAUSAL, int BIAS>
__global__ __launch_bounds__(NT, (dkdv_min_blocks<H16, D>())) void dkdv_kernel(BwdArgs a) {
  using T = elem_t<H16>;
  constexpr bool HAS_BIAS = BIAS != 0;
  constexpr bool DIRECT = H16 != 0 && !HAS_BIAS && (D == 64 || D == 128);
  using SM = typename std::conditional<DIRECT, DkdvSmemDirect<H16, D>, DkdvSmem<H16, D>>::type;
  using St = Stager<H16, BMQ, D>;
  constexpr int DT = D / 32;
  // head_dim 256: each unit runs as two items, each accumulating dK and dV for
  // half of the dims (S and dP computed in both), so the accumulators fit
  constexpr int HS = D > 128 ? 2 : 1;  // items per unit and KV head
  constexpr int DTO = DT / HS;         // 32-wide output tiles per item
  constexpr int ELT = (int)sizeof(T);

  __shared__ SM sm;
  __shared__ __attribute__((aligned(16))) int s_info[2][kItemInts];
  // per-key bias gradient sums [head of the group][key of the tile] (bias kernels only)
  __shared__ float db_acc[HAS_BIAS ? dbias_max_heads<D>() * BNK : 1];
  // a bias with contiguous keys and 16-byte aligned rows comes a step ahead, with
  // Q and dO, as [BMQ rows][BNK keys] tiles (double-buffered), loaded straight
  // into LDS: each wave load fills 64 x 16 consecutive bytes
  constexpr bool btile = BIAS == 2;
  constexpr int BTP = BNK;
  constexpr int BCH = BNK * ELT / 16;     // 16-byte pieces per tile row
  constexpr int BTT = BMQ * BCH / NT;     // per thread
  static_assert(BMQ * BCH % NT == 0, "bias tile loads must tile the workgroup");
  __shared__ __attribute__((aligned(16))) T bias_t[btile ? 2 * BMQ * BTP : 1];

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int hh = lane >> 5, r32 = lane & 31;

  const int per_unit = a.hkv * HS;
  const int total_items = uniform(a.plan_k.hdr[1]) * per_unit;
  // token strides (elements): Q, K, V as the caller lays them out; dO, dK, dV dense
  const size_t qstride = (size_t)a.q_rs, dostride = (size_t)a.hq * D;
  const size_t kstride = (size_t)a.k_rs, vstride = (size_t)a.v_rs, gstride = (size_t)a.hkv * D;
  const int qrow_bytes = (int)(qstride * ELT), dorow_bytes = (int)(dostride * ELT);
  const int krow_bytes = (int)(kstride * ELT), vrow_bytes = (int)(vstride * ELT);
  const int hpw = a.n_rep;  // every query head of the group

  int kth = 0;  // items this workgroup has run
  if (tid == 0) item_store(s_info[0], item_load(a.plan_k, (int)blockIdx.x, per_unit, total_items));
  __syncthreads();
  for (int cur = 0;; cur ^= 1) {
    const int* inf = s_info[cur];
    const int item = uniform(inf[kInfItem]);
    if (item >= total_items) break;
    const int unit = item / per_unit;
    const int rem = uniform(item - unit * per_unit);  // the division runs on the vector ALU
    const int g = rem / HS;
    const int hb = rem - g * HS;  // which half of the dims (head_dim 256)
    const int b = uniform(inf[kInfUnit]), t = uniform(inf[kInfUnit + 1]);
    const int u0 = uniform(inf[kInfUnit + 2]), u1 = uniform(inf[kInfUnit + 3]);
    const int k0 = uniform(inf[kInfRows]), k1 = uniform(inf[kInfRows + 1]), q0 = uniform(inf[kInfRows + 2]),
              q1 = uniform(inf[kInfRows + 3]);
    const int slot = uniform(inf[kInfSlot]);  // >= 0: a chunk of a split tile
    const int Lq = q1 - q0, Lk = k1 - k0, off = Lk - Lq;
    const int kt0 = t * BNK;
    const int wk0 = kt0 + 32 * wid;  // first key of this wave
    const int kj = wk0 + r32;        // this lane's key (columns of the score tile)
    const bool wave_keys = wk0 < Lk;

    RowFrag<H16, D> kf, vf;
    kf.load(make_rsrc((const T*)a.k + (size_t)k0 * kstride + (size_t)g * D,
                      Lk > 0 ? (int64_t)(Lk - 1) * krow_bytes + D * ELT : 0), krow_bytes, kj, hh);
    vf.load(make_rsrc((const T*)a.v + (size_t)k0 * vstride + (size_t)g * D,
                      Lk > 0 ? (int64_t)(Lk - 1) * vrow_bytes + D * ELT : 0), vrow_bytes, kj, hh);
    const size_t koff = (size_t)k0 * gstride + (size_t)g * D;  // this tile's dK / dV rows
    f32x16_t dk[DTO], dv[DTO];
#pragma unroll
    for (int i = 0; i < DTO; ++i) { dk[i] = (f32x16_t){}; dv[i] = (f32x16_t){}; }

    // query blocks that can see a key of the tile: i + off >= kt0 (causal);
    // this unit runs blocks [u0, u1) of them, for every head of the group
    const int qs = CAUSAL ? max(0, kt0 - off) : 0;
    const int nqb = qs < Lq ? (Lq - qs + BMQ - 1) / BMQ : 0;
    // blocks crossing the diagonal for some wave: qb + off < kt0 + BNK - 1
    const int n_diag = CAUSAL ? min(nqb, max(0, (kt0 + BNK - 1 - off - qs + BMQ - 1) / BMQ)) : 0;
    const int nb = u1 - u0;
    const int nm = min(max(n_diag - u0, 0), nb);  // masked blocks of the unit (its first ones)
    const int k_masked = hpw * nm, k_total = hpw * nb;
    const int h_first = uniform(g * a.n_rep);
    // block k of the unit is (head r, query block n): the masked blocks first
    // (heads outer), then the unmasked ones; next_of() gives block k from
    // block k - 1 (values only, so the cursor stays in scalar registers)
    auto next_of = [&](int k, int2 c) -> int2 {
      if (k == k_masked) return make_int2(0, u0 + nm);
      int r = c.x, n = c.y + 1;
      if (k < k_masked) {
        if (n == u0 + nm) { n = u0; ++r; }
      } else if (n == u1) {
        n = u0 + nm;
        ++r;
      }
      return make_int2(r, n);
    };

    St sq, sd;
    float pl = 0.f, pd = 0.f;  // staged LSE / dsum of query pi
    int pi = 0;
    // the bias view of head h (element (r, c) at r*bs2 + c*bs3) through a resource
    // that ends after the last element a valid (row, key) reads, rounded up to a
    // dword; rows past the sequence read 0 or are zeroed where used
    auto bias_res = [&](int h) {
      const int64_t last = ((int64_t)(Lq - 1) * a.bs2 + (int64_t)(Lk - 1) * a.bs3 + 1) * ELT;
      return make_rsrc((const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1, (last + 3) & ~(int64_t)3);
    };
    auto issue = [&](int2 rn, int tbuf) {
      const int r = uniform(rn.x), n = uniform(rn.y);
      const int h = h_first + r;
      const int qb = qs + n * BMQ;
      if constexpr (HAS_BIAS) {
        if constexpr (btile) {
          const rsrc_t br = bias_res(h);
#pragma unroll
          for (int i = 0; i < BTT; ++i) {
            const int u = tid + i * NT, row = u / BCH, ch = u % BCH;
            const int64_t o = ((int64_t)(qb + row) * a.bs2 + kt0) * ELT + 16 * ch;
            T* dst = bias_t + tbuf * BMQ * BTP + (i * NT + 64 * wid) * (16 / ELT);
            __builtin_amdgcn_raw_ptr_buffer_load_lds(br, (__attribute__((address_space(3))) void*)dst, 16,
                                                     (int)(o < 0x7FFFFFF0 ? o : 0x7FFFFFF0), 0, 0, 0);
          }
        }
      }
      sq.load(make_rsrc((const T*)a.q + (size_t)q0 * qstride + (size_t)h * D,
                        Lq > 0 ? (int64_t)(Lq - 1) * qrow_bytes + D * ELT : 0), qrow_bytes, qb);
      sd.load(make_rsrc((const T*)a.dout + (size_t)q0 * dostride + (size_t)h * D,
                        Lq > 0 ? (int64_t)(Lq - 1) * dorow_bytes + D * ELT : 0), dorow_bytes, qb);
      // the raw LSE and dsum of query qb + tid % BMQ (rows past the sequence read 0);
      // commit() converts them, so nothing here waits for the loads above
      {
        const size_t rb = (size_t)h * a.total_q + q0;
        pi = qb + (tid & (BMQ - 1));
        pl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.lse + rb, (int64_t)Lq * 4), pi * 4, 0, 0));
        pd = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(make_rsrc(a.dsum + rb, (int64_t)Lq * 4), pi * 4, 0, 0));
      }
    };
    // direct staging: block rn's Q and dO rows into buffer b3 (wave w's load i fills
    // slots (i * 4 + w) * 64 .. +63 of the tile: row = slot / PR, its piece
    // (slot % PR) ^ swz_key(row)), and the raw LSE (wave 0) and dsum (wave 1) of its
    // queries; each wave issues NI_D loads per tensor, waves 0 and 1 one more
    constexpr int PR = D * 2 / 16;      // 16-byte pieces per row
    constexpr int NI_D = BMQ * PR / NT;  // loads per thread per tensor
    static_assert(!DIRECT || BMQ * PR % NT == 0, "direct loads must tile the workgroup");
    auto issue_direct = [&](int2 rn, int b3) {
      if constexpr (DIRECT) {
        const int r = uniform(rn.x), n = uniform(rn.y);
        const int h = h_first + r;
        const int qb = qs + n * BMQ;
        const rsrc_t qres = make_rsrc((const T*)a.q + (size_t)q0 * qstride + (size_t)h * D,
                                      Lq > 0 ? (int64_t)(Lq - 1) * qrow_bytes + D * ELT : 0);
        const rsrc_t dres = make_rsrc((const T*)a.dout + (size_t)q0 * dostride + (size_t)h * D,
                                      Lq > 0 ? (int64_t)(Lq - 1) * dorow_bytes + D * ELT : 0);
#pragma unroll
        for (int i = 0; i < NI_D; ++i) {
          const int base = (i * (NT / 64) + wid) * 64;  // first slot of this wave's load
          const int u = base + lane, row = u / PR, piece = (u % PR) ^ swz_key<D>(row);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              qres, (__attribute__((address_space(3))) void*)(sm.qn[b3] + base * 8), 16,
              (qb + row) * qrow_bytes + piece * 16, 0, 0, 0);
          __builtin_amdgcn_raw_ptr_buffer_load_lds(
              dres, (__attribute__((address_space(3))) void*)(sm.dn[b3] + base * 8), 16,
              (qb + row) * dorow_bytes + piece * 16, 0, 0, 0);
        }
        if (wid < 2) {
          const size_t rb = (size_t)h * a.total_q + q0;
          const rsrc_t res = make_rsrc((wid == 0 ? a.lse : a.dsum) + rb, (int64_t)Lq * 4);
          float* dst = wid == 0 ? sm.lse2[b3] : sm.ndsum[b3];
          if (lane < BMQ)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(res, (__attribute__((address_space(3))) void*)dst, 4,
                                                     (qb + lane) * 4, 0, 0, 0);
        }
      }
    };
    // once block rn's direct loads have landed: its LSE to base 2 (+inf for rows
    // past the sequence or that see nothing, so their P is 0) and its dsum to -D
    // (0 past the sequence), by the waves that loaded them
    auto fixup_direct = [&](int2 rn, int b3) {
      if constexpr (DIRECT) {
        const int qb = qs + uniform(rn.y) * BMQ;
        const int pi_ = qb + lane;
        if (wid == 0 && lane < BMQ) {
          const float l = sm.lse2[b3][lane];
          sm.lse2[b3][lane] = pi_ < Lq && l != -INFINITY ? l * kLog2e : INFINITY;
        } else if (wid == 1 && lane < BMQ) {
          sm.ndsum[b3][lane] = pi_ < Lq ? -sm.ndsum[b3][lane] : 0.f;
        }
      }
    };
    auto commit = [&](int buf) {
      // the bias tile's direct loads were issued before Q and dO: wait for all of them
      // so the barrier after this publishes the tile
      if constexpr (btile) __builtin_amdgcn_s_waitcnt(kWaitVm0);
      sq.store(sm.qn[buf]);
      sd.store(sm.dn[buf]);
      if (tid < BMQ) {
        // rows past the sequence get P = exp2(x - inf) = 0, and so does a row that sees nothing
        sm.lse2[buf][tid] = pi < Lq && pl != -INFINITY ? pl * kLog2e : INFINITY;
        sm.ndsum[buf][tid] = pi < Lq ? -pd : 0.f;
      }
    };

    // rn, rn_next, rn_next2: blocks k, k + 1, k + 2
    auto step = [&](auto mask_tag, int k, int2 rn, int2 rn_next, int2 rn_next2) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int buf = DIRECT ? k % 3 : k & 1;
      const int r = uniform(rn.x), n = uniform(rn.y);
      const int h = h_first + r;
      const int qb = qs + n * BMQ;
      if constexpr (DIRECT) {
        if (k + 2 < k_total) issue_direct(rn_next2, (k + 2) % 3);
      } else {
        if (k + 1 < k_total) issue(rn_next, buf ^ 1);
      }
      // this wave's keys are seen by queries i >= wk0 - off
      const bool active = wave_keys && (!CAUSAL || qb + BMQ - 1 + off >= wk0);
      if (active) {
        // S = Q K^T and dP - D = dO V^T - D: C[query][key], lane = key.  Register i
        // holds query 8 (i / 4) + 4 hh + i % 4, so the LSE and -D of a lane's 16 queries
        // are four 16-byte LDS reads, and -D starts the dP accumulators.
        f32x4_t lq[4], nd[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          lq[j] = *(const f32x4_t*)&sm.lse2[buf][8 * j + 4 * hh];
          nd[j] = *(const f32x4_t*)&sm.ndsum[buf][8 * j + 4 * hh];
        }
        const f32x16_t nd16 = {nd[0][0], nd[0][1], nd[0][2], nd[0][3], nd[1][0], nd[1][1], nd[1][2], nd[1][3],
                               nd[2][0], nd[2][1], nd[2][2], nd[2][3], nd[3][0], nd[3][1], nd[3][2], nd[3][3]};
        f32x16_t s, dp;
        if constexpr (DIRECT) {
          s = (f32x16_t){};
          dp = nd16;
#pragma unroll
          for (int ks = 0; ks < D / 16; ++ks) {
            const int o = swz<D>(r32, 16 * ks + 8 * hh);
            s = mfma16<H16>(*(const u32x4_t*)&sm.qn[buf][o], kf.b[ks], s);
            dp = mfma16<H16>(*(const u32x4_t*)&sm.dn[buf][o], vf.b[ks], dp);
          }
        } else {
          s = mm_rows<H16, D>(&sm.qn[buf][r32 * St::NP], kf, (f32x16_t){}, hh);
          dp = mm_rows<H16, D>(&sm.dn[buf][r32 * St::NP], vf, nd16, hh);
        }
        // the bias of head h through a resource that ends after the last element a valid
        // (row, key) reads (rounded up to a dword); rows past the sequence read 0 or are
        // zeroed below, so garbage never meets a row whose P must be 0
        rsrc_t bres = make_rsrc(a.bias, 0);
        int brow = 0;
        if constexpr (HAS_BIAS) {
          if constexpr (!btile) {
            bres = bias_res(h);
            brow = (int)(((int64_t)kj * a.bs3 + (int64_t)(qb + 4 * hh) * a.bs2) * ELT);
          }
        }
        const T* bt_lane = bias_t + (btile ? (buf * BMQ + 4 * hh) * BTP + 32 * wid + r32 : 0);  // staged tile
        // causal: key kj is visible to query qb + ql iff ql >= kj - off - qb
        const int thr = kj - off - qb - 4 * hh;
        float p[16], ds[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int cl = 8 * (i >> 2) + (i & 3);  // query inside the block is cl + 4*hh
          const int ql = cl + 4 * hh;
          float x = s[i] * a.scale_log2;
          if constexpr (HAS_BIAS) {
            float bf;
            if constexpr (btile) {
              if constexpr (H16) bf = lo16<H16>((uint32_t)bt_lane[cl * BTP]);
              else bf = bt_lane[cl * BTP];
            } else {
              const int off = brow + cl * (int)a.bs2 * ELT;
              if constexpr (H16) bf = lo16<H16>(__builtin_amdgcn_raw_buffer_load_b16(bres, off, 0, 0));
              else bf = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, off, 0, 0));
            }
            x = __builtin_fmaf(qb + ql < Lq ? bf : 0.f, kLog2e, x);
          }
          float pv = fast_exp2(x - lq[i >> 2][i & 3]);
          if constexpr (MASK) pv = cl >= thr ? pv : 0.f;
          p[i] = pv;
          ds[i] = pv * dp[i];
        }
        if constexpr (HAS_BIAS) {
          // bias gradient = dS (the bias enters the logits additively)
          if (a.dbias_mode == 1) {
            if (kj < Lk && hb == 0) {  // both halves hold the same dS
              float* db = a.dbias + (int64_t)b * a.ds0 + (int64_t)h * a.ds1 + (int64_t)kj * a.ds3;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int qi = qb + 8 * (i >> 2) + 4 * hh + (i & 3);
                if (qi < Lq) db[(int64_t)qi * a.ds2] = ds[i];
              }
            }
          } else if (a.dbias_mode == 2) {
            float cs = 0.f;  // this lane's key over its 16 rows, then over both lane halves
#pragma unroll
            for (int i = 0; i < 16; ++i) cs += ds[i];
            cs += xor32(cs);
            if (hh == 0) db_acc[(a.ds1 == 0 ? 0 : r) * BNK + 32 * wid + r32] += cs;
          }
        }
        // dV += P^T dO, dK += dS^T Q: C[key][d], lane = d
        if constexpr (H16) {
#pragma unroll
          for (int c = 0; c < 2; ++c) {
            u32x4_t pa, da, da_lo;
            pack8<H16>(&p[8 * c], pa, nullptr);
            pack8<H16>(&ds[8 * c], da, &da_lo);
#pragma unroll
            for (int dt_ = 0; dt_ < DTO; ++dt_) {
              // dims 32 (dt_ + hb DTO) + r32 of the queries of P's chunk c, from the rows
              const int c0 = 32 * (dt_ + hb * DTO);
              u32x4_t ob, qb4;
              if constexpr (DIRECT) {
                ob = tr_frag_swz<D>(sm.dn[buf], c, c0);
                qb4 = tr_frag_swz<D>(sm.qn[buf], c, c0);
              } else {
                ob = tr_frag(sm.dn[buf], St::NP, c, c0);
                qb4 = tr_frag(sm.qn[buf], St::NP, c, c0);
              }
              dv[dt_] = mfma16<H16>(pa, ob, dv[dt_]);
              dk[dt_] = mfma16<H16>(da, qb4, dk[dt_]);
              dk[dt_] = mfma16<H16>(da_lo, qb4, dk[dt_]);
            }
          }
        } else {
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ql = 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
            for (int dt_ = 0; dt_ < DTO; ++dt_) {
              const float ob = sm.dn[buf][ql * St::NP + 32 * (dt_ + hb * DTO) + r32];
              const float qv = sm.qn[buf][ql * St::NP + 32 * (dt_ + hb * DTO) + r32];
              dv[dt_] = mfma32_f32(p[i], ob, dv[dt_]);
              dk[dt_] = mfma32_f32(ds[i], qv, dk[dt_]);
            }
          }
        }
      }
      if constexpr (HAS_BIAS) {
        // per-pair bias gradient of a query block that sees none of this wave's keys: 0
        if (!active && a.dbias_mode == 1 && hb == 0 && kj < Lk) {
          float* db = a.dbias + (int64_t)b * a.ds0 + (int64_t)h * a.ds1 + (int64_t)kj * a.ds3;
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int qi = qb + 8 * (i >> 2) + 4 * hh + (i & 3);
            if (qi < Lq) db[(int64_t)qi * a.ds2] = 0.f;
          }
        }
      }
      if constexpr (DIRECT) {
        // block k + 1's loads (issued a step ago) have landed; block k + 2's stay in flight
        if (k + 2 < k_total) {
          if (wid < 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * NI_D + 1));
          else __builtin_amdgcn_s_waitcnt(wait_vm(2 * NI_D));
        } else {
          __builtin_amdgcn_s_waitcnt(kWaitVm0);
        }
        if (k + 1 < k_total) fixup_direct(rn_next, (k + 1) % 3);
      } else {
        if (k + 1 < k_total) commit(buf ^ 1);
      }
      lds_barrier();
    };

    if constexpr (HAS_BIAS) {
      // per-key bias gradient: each wave sums into its own 32 columns (no barrier needed)
      if (a.dbias_mode == 2 && hh == 0)
        for (int r = 0; r < (a.ds1 == 0 ? 1 : hpw); ++r) db_acc[r * BNK + 32 * wid + r32] = 0.f;
      // per-pair bias gradient of the rows before the first query that sees the tile
      // (causal): 0, written once per (tile, head) by the tile's first chunk, the two
      // lane halves taking alternate rows
      if (a.dbias_mode == 1 && hb == 0 && u0 == 0 && kj < Lk && qs > 0) {
        for (int r = 0; r < hpw; ++r) {
          float* db = a.dbias + (int64_t)b * a.ds0 + (int64_t)(h_first + r) * a.ds1 + (int64_t)kj * a.ds3;
          for (int qi = hh; qi < min(qs, Lq); qi += 2) db[(int64_t)qi * a.ds2] = 0.f;
        }
      }
    }
    int2 rn = make_int2(0, u0);
    int2 rn1 = next_of(1, rn);  // block k + 1
    if constexpr (DIRECT) {
      if (k_total > 0) issue_direct(rn, 0);
      if (k_total > 1) issue_direct(rn1, 1);
      // block 0 and every load before it (K and V fragments included) have landed
      if (k_total > 1) {
        if (wid < 2) __builtin_amdgcn_s_waitcnt(wait_vm(2 * NI_D + 1));
        else __builtin_amdgcn_s_waitcnt(wait_vm(2 * NI_D));
      } else {
        __builtin_amdgcn_s_waitcnt(kWaitVm0);
      }
      if (k_total > 0) fixup_direct(rn, 0);
    } else {
      if (k_total > 0) { issue(rn, 0); commit(0); }
      // every load so far (K and V fragments included) has landed: the steps below then
      // wait only for their own prefetches
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
    lds_barrier();
    // the next item: a ticket taken at the start of this item's second-to-last
    // step, its plan entries loaded during the last (thread 0)
    NextItem<Plan> next_item{a.plan_k, per_unit, total_items, s_info[cur ^ 1]};
    int k = 0;
    for (; k < k_masked; ++k) {
      const int2 nx2 = next_of(k + 2, rn1);
      next_item.at(k, k_total);
      step(std::integral_constant<bool, true>(), k, rn, rn1, nx2);
      rn = rn1;
      rn1 = nx2;
    }
    for (; k < k_total; ++k) {
      const int2 nx2 = next_of(k + 2, rn1);
      next_item.at(k, k_total);
      step(std::integral_constant<bool, false>(), k, rn, rn1, nx2);
      rn = rn1;
      rn1 = nx2;
    }
    next_item.finish(k_total);
    ++kth;

    if constexpr (HAS_BIAS) {
      if (a.dbias_mode == 2 && hh == 0 && hb == 0) {
        const int nacc = a.ds1 == 0 ? 1 : hpw;
        if (slot < 0) {
          if (kj < Lk)
            for (int r = 0; r < nacc; ++r)
              a.dbias[(int64_t)b * a.ds0 + (int64_t)(h_first + r) * a.ds1 + (int64_t)kj * a.ds3] =
                  db_acc[r * BNK + 32 * wid + r32];
        } else {
          float* pd = a.part_db + ((size_t)slot * a.hkv + g) * hpw * BNK;
          for (int r = 0; r < nacc; ++r) pd[r * BNK + 32 * wid + r32] = db_acc[r * BNK + 32 * wid + r32];
        }
      }
    }

    // ---- epilogue.  Register i of tile dt holds key wk0 + 8(i/4) + 4hh + i%4,
    // dim 32dt + r32.  Whole tiles: buffer stores whose resource ends at the
    // sequence's last key (rows past it are dropped).  A chunk of a split tile
    // stores the registers as they lie (16 bytes per lane, [dt][i/4][lane][4])
    // into its slot; the merge in the dQ pass undoes the layout.
    if (slot < 0) {
      const int gelt = a.grad_bf16 ? 2 : 4;
      const int krow = (int)gstride * gelt;
      const size_t base = (koff + (size_t)max(wk0, 0) * gstride) * gelt;
      const int64_t nbytes = Lk > wk0 ? (int64_t)(Lk - wk0 - 1) * krow + D * gelt : 0;
      const rsrc_t rk = make_rsrc((const uint8_t*)a.dk + base, nbytes);
      const rsrc_t rv = make_rsrc((const uint8_t*)a.dv + base, nbytes);
      const int lane_off = 4 * hh * krow + r32 * gelt;
#pragma unroll
      for (int dt_ = 0; dt_ < DTO; ++dt_)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int off = lane_off + (8 * (i >> 2) + (i & 3)) * krow + 32 * (dt_ + hb * DTO) * gelt;
          const float kv = dk[dt_][i] * a.scale, vv = dv[dt_][i];
          if (a.grad_bf16) {
            buf_store2((uint16_t)(pack16<H16>(kv, 0.f) & 0xFFFF), rk, off);
            buf_store2((uint16_t)(pack16<H16>(vv, 0.f) & 0xFFFF), rv, off);
          } else {
            buf_store4(__float_as_uint(kv), rk, off);
            buf_store4(__float_as_uint(vv), rv, off);
          }
        }
    } else {
      float* pk = a.part_kv + ((size_t)slot * a.hkv + g) * 2 * BNK * D + (size_t)wid * 32 * D;
      float* pv = pk + BNK * D;
#pragma unroll
      for (int dt_ = 0; dt_ < DTO; ++dt_)
#pragma unroll
        for (int i4 = 0; i4 < 4; ++i4) {
          const int o = (((dt_ + hb * DTO) * 4 + i4) * 64 + lane) * 4;
          *(f32x4_t*)(pk + o) = (f32x4_t){dk[dt_][4 * i4], dk[dt_][4 * i4 + 1], dk[dt_][4 * i4 + 2], dk[dt_][4 * i4 + 3]};
          *(f32x4_t*)(pv + o) = (f32x4_t){dv[dt_][4 * i4], dv[dt_][4 * i4 + 1], dv[dt_][4 * i4 + 2], dv[dt_][4 * i4 + 3]};
        }
    }
    lds_barrier();
  }
}

// Sums the chunks of split dK/dV tiles in chunk order (deterministic) and
// writes the gradients.  A work item is one wave's 32 keys of one (split
// tile, KV head); a thread owns 16-byte pieces of the partials' register
// layout [dt][i/4][lane][4], i.e. 4 consecutive keys of one dim.
template <int D>
__device__ __forceinline__ void dkdv_merge_item(const BwdArgs& a, int it) {
  constexpr int DT = D / 32;
  constexpr int PIECES = DT * 4 * 64;       // 16-byte pieces per wave block
  constexpr int PPT = PIECES / NT;          // per thread
  {
    const int w = it & 3, sg = it >> 2;
    const int si = sg / a.hkv, g = sg - si * a.hkv;
    const int4 sp = a.plan_k.splits[si];
    const int b = uniform(sp.x), t = uniform(sp.y), sb = uniform(sp.z), nch = uniform(sp.w);
    int k0, k1;
    seq_bounds(a.cu_k, b, a.total_k, k0, k1);
    const int Lk = k1 - k0;
#pragma unroll
    for (int pp = 0; pp < PPT; ++pp) {
      const int piece = threadIdx.x + pp * NT;
      const int lane = piece & 63, i4 = (piece >> 6) & 3, dt = piece >> 8;
      const int hh = lane >> 5, r32 = lane & 31;
      f32x4_t sk = {0.f, 0.f, 0.f, 0.f}, sv = sk;
#pragma unroll 4
      for (int c = 0; c < nch; ++c) {
        const float* pk = a.part_kv + ((size_t)(sb + c) * a.hkv + g) * 2 * BNK * D + (size_t)w * 32 * D;
        sk += *(const f32x4_t*)(pk + piece * 4);
        sv += *(const f32x4_t*)(pk + BNK * D + piece * 4);
      }
      const int key0 = t * BNK + 32 * w + 8 * i4 + 4 * hh;  // keys key0 .. key0+3
      const int d = 32 * dt + r32;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (key0 + j >= Lk) break;
        const size_t o = ((size_t)(k0 + key0 + j) * a.hkv + g) * D + d;
        const float kv = sk[j] * a.scale, vv = sv[j];
        if (a.grad_bf16) {
          ((uint16_t*)a.dk)[o] = (uint16_t)(pack16_rt(kv, 0.f, a.grad_bf16) & 0xFFFF);
          ((uint16_t*)a.dv)[o] = (uint16_t)(pack16_rt(vv, 0.f, a.grad_bf16) & 0xFFFF);
        } else {
          ((float*)a.dk)[o] = kv;
          ((float*)a.dv)[o] = vv;
        }
      }
    }
    if (a.dbias_mode == 2) {  // per-key bias gradient: chunk sums in chunk order
      const int nacc = a.ds1 == 0 ? 1 : a.n_rep;
      for (int e = threadIdx.x; e < nacc * 32; e += NT) {
        const int r = e >> 5, kk = 32 * w + (e & 31), key = t * BNK + kk;
        if (key >= Lk) continue;
        float s = 0.f;
        for (int c = 0; c < nch; ++c) s += a.part_db[(((size_t)(sb + c) * a.hkv + g) * a.n_rep + r) * BNK + kk];
        a.dbias[(int64_t)b * a.ds0 + (int64_t)(g * a.n_rep + r) * a.ds1 + (int64_t)key * a.ds3] = s;
      }
    }
  }
}

// ---------------------------------------------------------------- dQ
// Two workgroups per CU (256 registers per lane) up to head_dim 128; one at 256,
// whose accumulators and Q/dO fragments alone take about that many.
template <int D>
constexpr int dq_min_blocks() { return D <= 128 ? 2 : 1; }

template <int H16, int D>
struct DqSmem {
  using T = elem_t<H16>;
  static constexpr int BN = (H16 && D <= 64) ? 64 : 32;
  using St = Stager<H16, BN, D>;
  using Sv = Stager<H16, BN, D>;
  T kn[2][BN * St::NP];
  T vn[2][BN * St::NP];
};

// BIAS: 0 none; 1 any layout (one element per load); 2 contiguous keys (four per load)
template <int H16, int D, bool CAUSAL, int BIAS>
__global__ __launch_bounds__(NT, (dq_min_blocks<D>())) void dq_kernel(BwdArgs a) {
  constexpr bool HAS_BIAS = BIAS != 0;
  using T = elem_t<H16>;
  using SM = DqSmem<H16, D>;
  constexpr int BN = SM::BN;
  constexpr int NS = BN / 32;
  // 16-bit, no bias, two 32-key score tiles per block: the explicit-order step (FAST);
  // at head_dim 64 its K tiles are staged swizzled, conflict-free for both the row
  // reads of S and the transposing reads of dQ += dS K
  constexpr bool FAST = H16 && !HAS_BIAS && NS == 2;
  constexpr bool KSWZ = FAST && D == 64;
  constexpr int DT = D / 32;
  constexpr int ELT = (int)sizeof(T);
  using St = typename SM::St;
  using Sv = typename SM::Sv;

  __shared__ SM sm;
  __shared__ __attribute__((aligned(16))) int s_info[2][kItemInts];
  __shared__ int s_last;  // this chunk of a split tile finished last

  const int tid = threadIdx.x, lane = tid & 63, wid = uniform(tid >> 6);
  const int hh = lane >> 5, r32 = lane & 31;

  const int total_items = uniform(a.plan_q.hdr[1]) * a.hq;
  // token strides (elements): Q, K, V as the caller lays them out; dO and dQ dense
  const size_t qstride = (size_t)a.q_rs, dostride = (size_t)a.hq * D;
  const size_t kstride = (size_t)a.k_rs, vstride = (size_t)a.v_rs;
  const int qrow_bytes = (int)(qstride * ELT), dorow_bytes = (int)(dostride * ELT);
  const int krow_bytes = (int)(kstride * ELT), vrow_bytes = (int)(vstride * ELT);
  const int gelt = a.grad_bf16 ? 2 : 4;

  int kth = 0;  // items this workgroup has run
  if (tid == 0) item_store(s_info[0], item_load(a.plan_q, (int)blockIdx.x, a.hq, total_items));
  __syncthreads();
  for (int cur = 0;; cur ^= 1) {
    const int* inf = s_info[cur];
    const int item = uniform(inf[kInfItem]);
    if (item >= total_items) break;
    const int unit = item / a.hq;
    const int h = item - unit * a.hq;
    const int b = uniform(inf[kInfUnit]), t = uniform(inf[kInfUnit + 1]);
    const int n0 = uniform(inf[kInfUnit + 2]), n1 = uniform(inf[kInfUnit + 3]);
    const int q0 = uniform(inf[kInfRows]), q1 = uniform(inf[kInfRows + 1]), k0 = uniform(inf[kInfRows + 2]),
              k1 = uniform(inf[kInfRows + 3]);
    const int slot = uniform(inf[kInfSlot]);  // >= 0: a chunk of a split tile
    const int si = uniform(inf[kInfSplit]);  // that split tile
    const int Lq = q1 - q0, Lk = k1 - k0, off = Lk - Lq;
    const int g = h / a.n_rep;
    const int r1 = Lq - t * BMQ_DQ;
    const int w0 = r1 - BMQ_DQ + 32 * wid;
    const int rq = w0 + r32;
    const bool row_ok = rq >= 0;
    const int kv_hi = CAUSAL ? min(Lk, r1 + off) : Lk;
    const int wave_hi = CAUSAL ? min(Lk, w0 + 32 + off) : Lk;
    const bool wave_on = (w0 + 31 >= 0) && wave_hi > 0;
    // blocks start at key 0; those before n_plain are fully visible to every
    // row of the tile (the smallest row sees keys <= r1 - BMQ_DQ + off); this
    // unit runs blocks [n0, n1)
    const int n_plain = CAUSAL ? max(r1 - BMQ_DQ + off + 1, 0) / BN : kv_hi / BN;
    const int kv_end = min(kv_hi, n1 * BN);  // keys this unit may read

    const size_t qoff = (size_t)q0 * dostride + (size_t)h * D;  // dO and dQ rows
    RowFrag<H16, D> qf, of;
    qf.load(make_rsrc((const T*)a.q + (size_t)q0 * qstride + (size_t)h * D,
                      Lq > 0 ? (int64_t)(Lq - 1) * qrow_bytes + D * ELT : 0), qrow_bytes, rq, hh);
    of.load(make_rsrc((const T*)a.dout + qoff, Lq > 0 ? (int64_t)(Lq - 1) * dorow_bytes + D * ELT : 0),
            dorow_bytes, rq, hh);
    float lse2 = 0.f, dsum = 0.f;
    if (row_ok) {
      const float l = a.lse[(size_t)h * a.total_q + q0 + rq];
      lse2 = l == -INFINITY ? INFINITY : l * kLog2e;  // a row that sees nothing adds nothing
      dsum = a.dsum[(size_t)h * a.total_q + q0 + rq];
    }
    f32x16_t ndsum16;  // -D of this lane's row in every register: the dP^T accumulators start from it
#pragma unroll
    for (int i = 0; i < 16; ++i) ndsum16[i] = -dsum;
    f32x16_t acc[DT];
#pragma unroll
    for (int i = 0; i < DT; ++i) acc[i] = (f32x16_t){};

    const rsrc_t kres = make_rsrc((const T*)a.k + (size_t)k0 * kstride + (size_t)g * D,
                                  kv_end > 0 ? (int64_t)(kv_end - 1) * krow_bytes + D * ELT : 0);
    const rsrc_t vres = make_rsrc((const T*)a.v + (size_t)k0 * vstride + (size_t)g * D,
                                  kv_end > 0 ? (int64_t)(kv_end - 1) * vrow_bytes + D * ELT : 0);
    // this (sequence, head)'s bias view (element (r, c) at r*bs2 + c*bs3), ending after the
    // last element a valid (row, key) reads; rows before the sequence read 0, keys past
    // it are masked
    rsrc_t bres = make_rsrc(a.bias, 0);
    int boff = 0;
    if constexpr (HAS_BIAS) {
      const int64_t last = Lq > 0 && Lk > 0 ? ((int64_t)(Lq - 1) * a.bs2 + (int64_t)(Lk - 1) * a.bs3 + 1) * ELT : 0;
      bres = make_rsrc((const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1, (last + 3) & ~(int64_t)3);
      boff = (int)(((int64_t)rq * a.bs2 + 4 * hh * a.bs3) * ELT);
    }
    const int hi_row = CAUSAL ? min(kv_hi - 1, rq + off) : kv_hi - 1;

    St sk;
    Sv sv;
    auto step = [&](auto mask_tag, int n) {
      constexpr bool MASK = decltype(mask_tag)::value;
      const int kb = n * BN;
      const int buf = (n - n0) & 1;
      // a 16-bit bias with contiguous keys: this step's values are loaded before the
      // next step's K/V prefetch, so waiting for them does not wait for the prefetch
      // (vector loads retire in order); register e holds keys kb + 32(e/4) + 8(e%4)
      // + 4hh .. +3.  (float32 keeps its loads in the step: its registers are full.)
      constexpr bool EARLY = BIAS == 2 && H16 != 0;
      u32x2_t braw[EARLY ? 4 * NS : 1];
      if constexpr (EARLY) {
        if (wave_on && kb < wave_hi) {
#pragma unroll
          for (int e = 0; e < 4 * NS; ++e) braw[e] = buf_load8(bres, boff + (kb + 32 * (e >> 2) + 8 * (e & 3)) * ELT);
        }
      }
      if (n + 1 < n1) {
        sk.load(kres, krow_bytes, kb + BN);
        sv.load(vres, vrow_bytes, kb + BN);
      }
      // FAST: the tiles' MFMAs and the vector work of the softmax gradient in an
      // explicit order -- the fragments of tile 1 are read under tile 0's MFMAs, tile
      // 1's MFMAs run under tile 0's exponentials, and the dQ MFMAs of tile 0's keys
      // under tile 1's
      if constexpr (FAST) {
        if (wave_on && kb < wave_hi) {
          constexpr int KS = D / 16;  // k-steps over head_dim
          // K rows: swizzled (head_dim 64) or padded; row r32 (+32 for tile 1), piece 2 ks + hh
          auto kfrag = [&](int row, int ks) __attribute__((always_inline)) {
            if constexpr (KSWZ) return *(const u32x4_t*)&sm.kn[buf][swz<D>(row, 16 * ks + 8 * hh)];
            else return *(const u32x4_t*)&sm.kn[buf][row * St::NP + 16 * ks + 8 * hh];
          };
          const T* vr = &sm.vn[buf][r32 * St::NP + 8 * hh];
          u32x4_t kf[2][KS], vf[2][KS];
          f32x16_t s2[2] = {(f32x16_t){}, (f32x16_t){}}, dp2[2] = {ndsum16, ndsum16};
          float dsv[32];
          u32x4_t pbs[4];
          // softmax gradient of tile st (lane = query, registers = keys), packed for dQ
          auto grad = [&](int st) __attribute__((always_inline)) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int kj = kb + 32 * st + 8 * (i >> 2) + (i & 3) + 4 * hh;
              float pv = fast_exp2(__builtin_fmaf(s2[st][i], a.scale_log2, -lse2));
              if constexpr (MASK) pv = kj <= hi_row ? pv : 0.f;
              dsv[16 * st + i] = pv * dp2[st][i];
            }
#pragma unroll
            for (int c = 0; c < 2; ++c) pack8<H16>(&dsv[16 * st + 8 * c], pbs[2 * st + c], nullptr);
          };
          auto dq_mma = [&](int kc) __attribute__((always_inline)) {
#pragma unroll
            for (int dt_ = 0; dt_ < DT; ++dt_) {
              u32x4_t kt;
              if constexpr (KSWZ) kt = tr_frag_swz<D>(sm.kn[buf], kc, 32 * dt_);
              else kt = tr_frag(sm.kn[buf], St::NP, kc, 32 * dt_);
              acc[dt_] = mfma16<H16>(kt, pbs[kc], acc[dt_]);
            }
          };
          // tile 0's fragments
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            kf[0][ks] = kfrag(r32, ks);
            vf[0][ks] = *(const u32x4_t*)(vr + 16 * ks);
          }
          __builtin_amdgcn_sched_barrier(0);
          // tile 0's S^T and dP^T - D, tile 1's fragments read under them
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s2[0] = mfma16<H16>(kf[0][ks], qf.b[ks], s2[0]);
            kf[1][ks] = kfrag(32 + r32, ks);
            dp2[0] = mfma16<H16>(vf[0][ks], of.b[ks], dp2[0]);
            vf[1][ks] = *(const u32x4_t*)(vr + 32 * St::NP + 16 * ks);
          }
          __builtin_amdgcn_sched_barrier(0);
          // tile 1's MFMAs, each with a share of tile 0's vector work
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            s2[1] = mfma16<H16>(kf[1][ks], qf.b[ks], s2[1]);
            dp2[1] = mfma16<H16>(vf[1][ks], of.b[ks], dp2[1]);
          }
          grad(0);
#pragma unroll
          for (int i = 0; i < 2 * KS; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // exponentials
            __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);  // other vector work
          }
          __builtin_amdgcn_sched_barrier(0);
          // tile 0's dQ MFMAs under tile 1's vector work
          dq_mma(0);
          dq_mma(1);
          grad(1);
#pragma unroll
          for (int i = 0; i < 2 * DT; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);  // transposing reads
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
            __builtin_amdgcn_sched_group_barrier(0x400, 4, 0);  // exponentials
            __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);  // other vector work
          }
          __builtin_amdgcn_sched_barrier(0);
          dq_mma(2);
          dq_mma(3);
        }
      } else if (wave_on && kb < wave_hi) {
        float dsv[16 * NS];
#pragma unroll
        for (int st = 0; st < NS; ++st) {
          // S^T = K Q^T, dP^T = V dO^T: C[key][query], lane = query
          const f32x16_t s = mm_rows<H16, D>(&sm.kn[buf][(32 * st + r32) * St::NP], qf, (f32x16_t){}, hh);
          // dP^T - D (the no-bias kernels start the accumulators from -D, kept in registers)
          const f32x16_t dp = mm_rows<H16, D>(&sm.vn[buf][(32 * st + r32) * St::NP], of,
                                              HAS_BIAS ? (f32x16_t){} : ndsum16, hh);
          float bv[HAS_BIAS ? 16 : 1];
          if constexpr (HAS_BIAS) {
            // registers 4j .. 4j+3 are 4 consecutive keys: one load each when keys are
            // contiguous, else four element loads packed the same way
#pragma unroll
            for (int j = 0; j < 4; ++j) {
              const int key = kb + 32 * st + 8 * j;
              if constexpr (H16) {
                u32x2_t x;
                if constexpr (BIAS == 2) {
                  x = braw[4 * st + j];
                } else {
                  uint32_t e[4];
#pragma unroll
                  for (int c = 0; c < 4; ++c)
                    e[c] = __builtin_amdgcn_raw_buffer_load_b16(bres, boff + (key + c) * (int)a.bs3 * ELT, 0, 0);
                  x = (u32x2_t){e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
                }
                bv[4 * j + 0] = lo16<H16>(x[0]);
                bv[4 * j + 1] = hi16<H16>(x[0]);
                bv[4 * j + 2] = lo16<H16>(x[1]);
                bv[4 * j + 3] = hi16<H16>(x[1]);
              } else {
                u32x4_t x;
                if constexpr (BIAS == 2) {
                  x = buf_load16(bres, boff + key * ELT);
                } else {
#pragma unroll
                  for (int c = 0; c < 4; ++c)
                    x[c] = __builtin_amdgcn_raw_buffer_load_b32(bres, boff + (key + c) * (int)a.bs3 * ELT, 0, 0);
                }
#pragma unroll
                for (int e = 0; e < 4; ++e) bv[4 * j + e] = __uint_as_float(x[e]);
              }
            }
          }
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ci = 32 * st + 8 * (i >> 2) + (i & 3);
            const int kj = kb + ci + 4 * hh;
            float x = s[i] * a.scale_log2;
            if constexpr (HAS_BIAS) x = __builtin_fmaf(bv[i], kLog2e, x);
            float pv = fast_exp2(x - lse2);
            if constexpr (MASK) pv = kj <= hi_row ? pv : 0.f;
            dsv[16 * st + i] = pv * (HAS_BIAS ? dp[i] - dsum : dp[i]);
          }
        }
        // dQ^T += K^T dS^T
        if constexpr (H16) {
#pragma unroll
          for (int kc = 0; kc < 2 * NS; ++kc) {
            u32x4_t pb;
            pack8<H16>(&dsv[8 * kc], pb, nullptr);
#pragma unroll
            for (int dt_ = 0; dt_ < DT; ++dt_)
              acc[dt_] = mfma16<H16>(tr_frag(sm.kn[buf], St::NP, kc, 32 * dt_), pb, acc[dt_]);
          }
        } else {
#pragma unroll
          for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
              for (int dt_ = 0; dt_ < DT; ++dt_) {
                const float ka = sm.kn[buf][key * St::NP + 32 * dt_ + r32];
                acc[dt_] = mfma32_f32(ka, dsv[16 * st + i], acc[dt_]);
              }
            }
        }
      }
      if (n + 1 < n1) {
        if constexpr (KSWZ) sk.store_swz(sm.kn[buf ^ 1]);
        else sk.store(sm.kn[buf ^ 1]);
        sv.store(sm.vn[buf ^ 1]);
      }
      lds_barrier();
    };

    if (n1 > n0) {
      sk.load(kres, krow_bytes, n0 * BN);
      sv.load(vres, vrow_bytes, n0 * BN);
      if constexpr (KSWZ) sk.store_swz(sm.kn[0]);
      else sk.store(sm.kn[0]);
      sv.store(sm.vn[0]);
    }
    // every load so far (Q and dO fragments included) has landed: the steps below then
    // wait only for their own prefetches
    __builtin_amdgcn_s_waitcnt(kWaitVm0);
    lds_barrier();
    NextItem<Plan> next_item{a.plan_q, a.hq, total_items, s_info[cur ^ 1]};
    int n = n0;
    for (; n < min(n_plain, n1); ++n) {
      next_item.at(n - n0, n1 - n0);
      step(std::integral_constant<bool, false>(), n);
    }
    for (; n < n1; ++n) {
      next_item.at(n - n0, n1 - n0);
      step(std::integral_constant<bool, true>(), n);
    }
    next_item.finish(n1 - n0);
    ++kth;

    // dQ = scale * acc.  A chunk of a split tile stores acc in float32 to its
    // slot instead, and the chunk that finishes last sums the tile's chunks in
    // chunk order, its own from registers (the same values it stored).
    auto write_dq = [&]() __attribute__((always_inline)) {
      // rows < 0 fall outside the resource: their stores are dropped
      const int dq_row_bytes = (int)dostride * gelt;
      const rsrc_t dqres = make_rsrc((uint8_t*)a.dq + qoff * gelt,
                                     Lq > 0 ? (int64_t)(Lq - 1) * dq_row_bytes + D * gelt : 0);
#pragma unroll
      for (int dt_ = 0; dt_ < DT; ++dt_)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt_ + 8 * a4 + 4 * hh;
          const float o0 = acc[dt_][4 * a4 + 0] * a.scale, o1 = acc[dt_][4 * a4 + 1] * a.scale;
          const float o2 = acc[dt_][4 * a4 + 2] * a.scale, o3 = acc[dt_][4 * a4 + 3] * a.scale;
          if (a.grad_bf16) {
            buf_store8((u32x2_t){pack16<H16>(o0, o1), pack16<H16>(o2, o3)}, dqres, rq * dq_row_bytes + d0 * 2);
          } else {
            buf_store16((u32x4_t){__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2),
                                  __float_as_uint(o3)}, dqres, rq * dq_row_bytes + d0 * 4);
          }
        }
    };
    if (slot < 0) {
      write_dq();
    } else {
      constexpr int SLOT_Q = BMQ_DQ * D;  // floats of one (slot, head) block
      const int rl = rq - (r1 - BMQ_DQ);  // 0 .. BMQ_DQ-1
      const rsrc_t pres = make_rsrc(a.part_q + ((size_t)slot * a.hq + h) * SLOT_Q, (int64_t)SLOT_Q * 4);
#pragma unroll
      for (int dt_ = 0; dt_ < DT; ++dt_)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const f32x4_t o = {acc[dt_][4 * a4], acc[dt_][4 * a4 + 1], acc[dt_][4 * a4 + 2], acc[dt_][4 * a4 + 3]};
          buf_store16_dev(as_u32x4(o), pres, (rl * D + 32 * dt_ + 8 * a4 + 4 * hh) * 4);
        }
      if (split_done_last(&a.plan_q.left[si * a.hq + h], &s_last)) {
        const int4 sp = a.plan_q.splits[si];
        const int sb = uniform(sp.z), nch = uniform(sp.w), me = slot - sb;  // first slot, chunks, this chunk
        constexpr int G = D <= 128 ? DT : 1;  // output tiles summed per pass (bounds the registers)
#pragma unroll
        for (int g0 = 0; g0 < DT; g0 += G) {
          f32x4_t sum[G][4];
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4) sum[j][a4] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
          for (int c = 0; c < nch; ++c) {
            if (c == me) {
#pragma unroll
              for (int j = 0; j < G; ++j)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                  sum[j][a4] += (f32x4_t){acc[g0 + j][4 * a4], acc[g0 + j][4 * a4 + 1], acc[g0 + j][4 * a4 + 2],
                                          acc[g0 + j][4 * a4 + 3]};
            } else {
              const rsrc_t cres =
                  make_rsrc(a.part_q + ((size_t)(sb + c) * a.hq + h) * SLOT_Q, (int64_t)SLOT_Q * 4);
#pragma unroll
              for (int j = 0; j < G; ++j)
#pragma unroll
                for (int a4 = 0; a4 < 4; ++a4)
                  sum[j][a4] += buf_load16_dev(cres, (rl * D + 32 * (g0 + j) + 8 * a4 + 4 * hh) * 4);
            }
          }
#pragma unroll
          for (int j = 0; j < G; ++j)
#pragma unroll
            for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
              for (int e = 0; e < 4; ++e) acc[g0 + j][4 * a4 + e] = sum[j][a4][e];
        }
        write_dq();
      }
    }
    lds_barrier();
  }
  // then the merge slabs of split dK/dV tiles (the dK/dV pass has finished),
  // round robin over the workgroups
  const int merge_items = uniform(a.plan_k.hdr[2]) * a.hkv * 4;
  for (int m = blockIdx.x; m < merge_items; m += gridDim.x) dkdv_merge_item<D>(a, m);
}

template <int H16, int D, bool CAUSAL, bool HAS_BIAS>
hipError_t launch_bwd_t(const BwdArgs& a, const PlanSet& ps, int64_t q_items, int64_t k_items,
                        hipStream_t st) {
  {
    // D workgroups: DSUM_WG less the planners (the launch then fits one round of
    // one workgroup per CU), or fewer when there are fewer rows than row groups
    const int64_t rows = (int64_t)a.total_q * a.hq, gpw = plan::PT / dsum_tpr<H16, D>();
    const int64_t grid = ps.nplans + std::min<int64_t>(DSUM_WG - ps.nplans, (rows + gpw - 1) / gpw);
    timing_before(st, "bwd_plan_dsum");
    hipLaunchKernelGGL((plan_dsum_kernel<H16, D>), dim3((unsigned)grid), dim3(plan::PT), 0, st, a, ps);
    timing_after(st);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  {
    auto kern = dkdv_kernel<H16, D, CAUSAL, 0>;
    if constexpr (HAS_BIAS) {
      kern = dkdv_kernel<H16, D, CAUSAL, 1>;
      if constexpr (D <= 128)  // at 256 the staged Q/dO leave no room for a bias tile
        if (a.bias_tile) kern = dkdv_kernel<H16, D, CAUSAL, 2>;
    }
    const int grid = resident_grid((const void*)kern, NT, k_items * (D > 128 ? 2 : 1));  // two items per unit at 256
    if (grid <= 0) return hipErrorInvalidConfiguration;
    timing_before(st, H16 == 2 ? "bwd_dkdv_f16" : H16 ? "bwd_dkdv_bf16" : "bwd_dkdv_f32");
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a);
    timing_after(st);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    auto kern = !HAS_BIAS ? dq_kernel<H16, D, CAUSAL, 0>
                          : (a.bias_vec ? dq_kernel<H16, D, CAUSAL, 2> : dq_kernel<H16, D, CAUSAL, 1>);
    const int grid = resident_grid((const void*)kern, NT, q_items);
    if (grid <= 0) return hipErrorInvalidConfiguration;
    timing_before(st, H16 == 2 ? "bwd_dq_f16" : H16 ? "bwd_dq_bf16" : "bwd_dq_f32");
    hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a);
    timing_after(st);
    e = hipGetLastError();
  }
  return e;
}

template <int H16, int D>
hipError_t launch_bwd_d(const BwdArgs& a, const PlanSet& ps, int64_t q_items, int64_t k_items,
                        hipStream_t st) {
  const bool hb = a.bias != nullptr;
  if (a.causal)
    return hb ? launch_bwd_t<H16, D, true, true>(a, ps, q_items, k_items, st)
              : launch_bwd_t<H16, D, true, false>(a, ps, q_items, k_items, st);
  return hb ? launch_bwd_t<H16, D, false, true>(a, ps, q_items, k_items, st)
            : launch_bwd_t<H16, D, false, false>(a, ps, q_items, k_items, st);
}

}  // namespace

int bwd_block_q() { return BMQ_DQ; }
int bwd_block_k() { return BNK; }
int bwd_dkdv_block_q() { return BMQ; }
int bwd_dq_block_n(bool bf16, int d) {
  if (bf16) return d <= 64 ? DqSmem<1, 64>::BN : DqSmem<1, 128>::BN;
  return DqSmem<0, 64>::BN;
}

template <int H16>
static hipError_t launch_bwd_h(const BwdArgs& a, const PlanSet& ps, int64_t q_items, int64_t k_items,
                               hipStream_t st) {
  switch (a.d) {
    case 32: return launch_bwd_d<H16, 32>(a, ps, q_items, k_items, st);
    case 64: return launch_bwd_d<H16, 64>(a, ps, q_items, k_items, st);
    case 96: return launch_bwd_d<H16, 96>(a, ps, q_items, k_items, st);
    case 128: return launch_bwd_d<H16, 128>(a, ps, q_items, k_items, st);
    case 256: return launch_bwd_d<H16, 256>(a, ps, q_items, k_items, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_bwd(const BwdArgs& a, const PlanSet& ps, int64_t q_items, int64_t k_items,
                      hipStream_t st) {
  if (a.bf16 == 2) return launch_bwd_h<2>(a, ps, q_items, k_items, st);
  if (a.bf16) return launch_bwd_h<1>(a, ps, q_items, k_items, st);
  return launch_bwd_h<0>(a, ps, q_items, k_items, st);
}

}  // namespace va
