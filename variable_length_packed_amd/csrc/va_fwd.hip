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

constexpr int NT = 256;  // threads per workgroup

// keys per block: 64 for bf16 (two 32-key score tiles), 32 for f32 (LDS size)
template <int H16, int D>
struct BlockN {
  static constexpr int value = H16 && D <= 128 ? 64 : 32;
};

template <int H16, int D>
struct FwdSmem {
  static constexpr int BN = BlockN<H16, D>::value;
  using T = typename std::conditional<(H16 != 0), uint16_t, float>::type;
  // K and V blocks: [BN][D] row-major as in memory, row pitch padded by 16
  // bytes.  bf16 V^T fragments come from transposing LDS reads.
  static constexpr int KP = D + 16 / (int)sizeof(T);
  // V rows: the pitch that keeps the transposing V^T reads of a wave on
  // distinct banks (head_dim a multiple of 64: 64 bytes of padding; 32, 96: none)
  static constexpr int VP = H16 ? D + (D % 64 == 0 ? 32 : 0) : KP;
  T k[2][BN * KP];
  T v[2][BN * VP];
};

template <int H16, int D>
struct Loader {
  static constexpr int BN = BlockN<H16, D>::value;
  using T = typename std::conditional<(H16 != 0), uint16_t, float>::type;
  static constexpr int EPV = 16 / sizeof(T);           // elements per 16-byte vector
  static constexpr int KVEC = BN * D / EPV;            // 16-byte vectors per K block
  static constexpr int KPT = (KVEC + NT - 1) / NT;     // per thread
  u32x4_t kr[KPT];
  u32x4_t vr[KPT];

  // Block of keys kb .. kb+BN-1 of one (sequence, KV head).  The resources
  // cover keys [0, kv_hi); other rows (negative offsets included) read 0.
  __device__ __forceinline__ void load_k(rsrc_t kres, int row_bytes, int kb) {
    static_assert(KVEC % NT == 0, "loader tasks must tile the workgroup");
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int key = u / (D / EPV), c = u % (D / EPV);
      kr[i] = buf_load16(kres, (kb + key) * row_bytes + c * 16);
    }
  }
  __device__ __forceinline__ void load_v(rsrc_t vres, int row_bytes, int kb) {
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int key = u / (D / EPV), c = u % (D / EPV);
      vr[i] = buf_load16(vres, (kb + key) * row_bytes + c * 16);
    }
  }

  __device__ __forceinline__ void store_k(FwdSmem<H16, D>& sm, int buf) {
    using S = FwdSmem<H16, D>;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int key = u / (D / EPV), c = u % (D / EPV);
      *(u32x4_t*)(&sm.k[buf][key * S::KP + c * EPV]) = kr[i];
    }
  }
  __device__ __forceinline__ void store_v(FwdSmem<H16, D>& sm, int buf) {
    using S = FwdSmem<H16, D>;
#pragma unroll
    for (int i = 0; i < KPT; ++i) {
      const int u = threadIdx.x + i * NT;
      const int key = u / (D / EPV), c = u % (D / EPV);
      *(u32x4_t*)(&sm.v[buf][key * S::VP + c * EPV]) = vr[i];
    }
  }
};

// Query tiles of 32 rows per wave.  Two tiles halve LDS reads per MFMA (each
// K and V^T fragment feeds two MFMAs) but need the whole register file, i.e.
// one wave per SIMD; measured on gfx950 that loses more to exposed latency
// than it saves, so one tile per wave (two waves per SIMD) is used.
template <int H16, int D>
struct WaveTiles {
  static constexpr int value = 1;
};
template <int H16, int D>
constexpr int block_m() { return 4 * 32 * WaveTiles<H16, D>::value; }

// d <= 64: two workgroups per CU (256 registers per lane); d = 96, 128: one,
// with the accumulators free to use the whole 512-entry register file.
template <int H16, int D>
constexpr int min_blocks() { return D <= 64 ? 2 : 1; }

// BIAS: 0 none; 1 loaded per step (vector loads for contiguous keys, else one
// element per load); 2 (16-bit only) contiguous keys in 16-byte aligned rows, the
// tile of a block staged in LDS a block ahead
template <int H16, int D, bool CAUSAL, int BIAS>
__global__ __launch_bounds__(NT, (min_blocks<H16, D>())) void fwd_kernel(FwdArgs a) {
  using T = typename std::conditional<(H16 != 0), uint16_t, float>::type;
  using S = FwdSmem<H16, D>;
  constexpr int BN = BlockN<H16, D>::value;
  constexpr int NS = BN / 32;                // 32-key score tiles per block
  constexpr int DT = D / 32;                 // 32-wide output tiles along head_dim
  constexpr int QF = H16 ? D / 16 : D / 2;  // Q fragments (MFMA k-steps) per lane
  constexpr int QT = WaveTiles<H16, D>::value;  // 32-row query tiles per wave
  constexpr int BM = block_m<H16, D>();
  constexpr int WR = 32 * QT;                 // rows per wave

  __shared__ S sm;
  __shared__ __attribute__((aligned(16))) int s_info[2][kItemInts];
  __shared__ int s_last;  // this chunk of a split tile finished last
  // 16-bit bias with contiguous keys: the [BM rows][BN keys] tile of a block, loaded
  // a block ahead straight into LDS (double-buffered).  Row r keeps its 16-byte
  // piece c (keys 8c .. 8c+7) in slot c ^ (r % 8), so the 32 rows a wave reads at
  // once spread over the banks.
  constexpr bool HAS_BIAS = BIAS != 0;
  constexpr bool BTILE = BIAS == 2;
  static_assert(!BTILE || H16 != 0, "the staged bias tile is 16-bit");
  constexpr int BPR = BN * 2 / 16;  // 16-byte pieces per tile row
  static_assert(!BTILE || BPR == 8, "the slot swizzle assumes 8 pieces per row");
  static_assert(!BTILE || BM * BPR % NT == 0, "bias tile loads must tile the workgroup");
  __shared__ __attribute__((aligned(16))) uint16_t fbias[BTILE ? 2 * BM * BN : 1];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = uniform(tid >> 6);
  const int hh = lane >> 5;
  const int r32 = lane & 31;

  const int total_items = uniform(a.plan.hdr[1]) * a.hq;

  const T* __restrict__ qg = (const T*)a.q;
  const T* __restrict__ kg = (const T*)a.k;
  const T* __restrict__ vg = (const T*)a.v;
  T* __restrict__ og = (T*)a.out;
  // token strides (elements): Q, K and V as the caller lays them out (a fused
  // QKV projection interleaves them), O dense
  const size_t qstride = (size_t)a.q_rs, ostride = (size_t)a.hq * D;
  const size_t kstride = (size_t)a.k_rs, vstride = (size_t)a.v_rs;

  int kth = 0;  // items this workgroup has run
  if (tid == 0) item_store(s_info[0], item_load(a.plan, (int)blockIdx.x, a.hq, total_items));
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
    const int Lq = q1 - q0, Lk = k1 - k0;
    const int off = Lk - Lq;
    const int g = h / a.n_rep;
    const int r1 = Lq - t * BM;
    const int w0 = r1 - BM + WR * wid;  // first row of this wave
    int rq[QT];                          // this lane's query row in each query tile
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) rq[qt] = w0 + 32 * qt + r32;
    // keys the whole tile may see, and this wave's last visible key + 1
    const int kv_hi = CAUSAL ? min(Lk, r1 + off) : Lk;
    const int wave_hi = CAUSAL ? min(Lk, w0 + WR + off) : Lk;
    const bool wave_on = (w0 + WR - 1 >= 0) && wave_hi > 0;
    // blocks start at key 0; the ragged block (if any) is the last, and with a
    // causal mask the blocks crossing the diagonal are the last ones too, so
    // every masked block comes after every unmasked one.  Blocks before
    // n_plain are unmasked for every wave of the workgroup: the smallest row
    // of the tile sees keys <= r1 - BM + off.  This unit runs blocks
    // [n0, n1) of the tile's ceil(kv_hi / BN).
    const int kb0 = n0 * BN;
    const int nb = n1 - n0;
    const int n_plain = CAUSAL ? min(max(r1 - BM + off + 1, 0) / BN, kv_hi / BN) : kv_hi / BN;
    const int j_plain = min(max(n_plain - n0, 0), nb);
    const int kv_end = min(kv_hi, n1 * BN);  // keys this unit may read

    // ---- resources: this sequence's rows of Q/O for head h and of K/V for head g
    constexpr int ELT = (int)sizeof(T);
    const int qrow_bytes = (int)(qstride * ELT), orow_bytes = (int)(ostride * ELT);
    const int krow_bytes = (int)(kstride * ELT), vrow_bytes = (int)(vstride * ELT);
    const rsrc_t qres = make_rsrc(qg + (size_t)q0 * qstride + (size_t)h * D,
                                  Lq > 0 ? (int64_t)(Lq - 1) * qrow_bytes + D * ELT : 0);
    const rsrc_t ores = make_rsrc(og + (size_t)q0 * ostride + (size_t)h * D,
                                  Lq > 0 ? (int64_t)(Lq - 1) * orow_bytes + D * ELT : 0);
    const rsrc_t kres = make_rsrc(kg + (size_t)k0 * kstride + (size_t)g * D,
                                  kv_end > 0 ? (int64_t)(kv_end - 1) * krow_bytes + D * ELT : 0);
    const rsrc_t vres = make_rsrc(vg + (size_t)k0 * vstride + (size_t)g * D,
                                  kv_end > 0 ? (int64_t)(kv_end - 1) * vrow_bytes + D * ELT : 0);

    // ---- Q fragments (B operand of S^T = K Q^T); rows < 0 read as zero
    u32x4_t qf4[QT][H16 ? QF : 1];
    float qff[QT][H16 ? 1 : QF];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      if constexpr (H16) {
#pragma unroll
        for (int ks = 0; ks < QF; ++ks)
          qf4[qt][ks] = buf_load16(qres, rq[qt] * qrow_bytes + (16 * ks + 8 * hh) * 2);
      } else {
        // k-slot (group G, step j) of lane half hh reads dim 8G + 4hh + j
#pragma unroll
        for (int G = 0; G < D / 8; ++G) {
          const u32x4_t z = buf_load16(qres, rq[qt] * qrow_bytes + (8 * G + 4 * hh) * 4);
#pragma unroll
          for (int j = 0; j < 4; ++j) qff[qt][4 * G + j] = __uint_as_float(z[j]);
        }
      }
    }

    f32x16_t acc[QT][DT];
    float m_run[QT], l_run[QT];  // running max (log2 units) and this half's partial row sum
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
#pragma unroll
      for (int i = 0; i < DT; ++i) acc[qt][i] = (f32x16_t){};
      m_run[qt] = -INFINITY;
      l_run[qt] = 0.f;
    }

    // this (sequence, head)'s bias view (element (r, c) at r*bs2 + c*bs3) and the byte
    // offset of this lane's row and key half in it
    rsrc_t bres = make_rsrc(a.bias, 0);
    int boff[QT];
    if constexpr (HAS_BIAS) {
      // the resource ends after the last element a valid (r, c) reads, rounded up to a
      // whole dword; loads past it (rows before the sequence, keys past its end) read 0
      const int64_t last = Lq > 0 && Lk > 0 ? ((int64_t)(Lq - 1) * a.bs2 + (int64_t)(Lk - 1) * a.bs3 + 1) * ELT : 0;
      bres = make_rsrc((const T*)a.bias + (int64_t)b * a.bs0 + (int64_t)h * a.bs1, (last + 3) & ~(int64_t)3);
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) boff[qt] = (int)(((int64_t)rq[qt] * a.bs2 + 4 * hh * a.bs3) * ELT);
    }
    constexpr bool btile = BTILE;
    // loads block kb's bias tile into buffer tb: wave load i fills 64 consecutive
    // slots (8 rows); slot s of tile row r takes piece s ^ (r % 8)
    auto bias_dma = [&](int kb, int tb) __attribute__((always_inline)) {
      if constexpr (BTILE) {
#pragma unroll
        for (int i = 0; i < BM * BPR / NT; ++i) {
          const int u = (i * (NT / 64) + wid) * 64 + lane;  // slot index in the tile
          const int row = u / BPR, piece = (u % BPR) ^ (row & 7);
          const int64_t o = ((int64_t)(r1 - BM + row) * a.bs2 + kb + 8 * piece) * 2;
          uint16_t* dst = fbias + tb * BM * BN + (i * (NT / 64) + wid) * 64 * 8;
          __builtin_amdgcn_raw_ptr_buffer_load_lds(bres, (__attribute__((address_space(3))) void*)dst, 16,
                                                   (int)(o < 0 ? 0x7FFFFFF0 : (o < 0x7FFFFFF0 ? o : 0x7FFFFFF0)),
                                                   0, 0, 0);
        }
      }
    };

    Loader<H16, D> ld;

    // Visible keys of a row: kj in [0, hi_row]; kj is kb + c_i + 4*hh with
    // c_i = 32*st + 8*(i/4) + i%4 a compile-time constant, so the mask of a
    // score is one unsigned range test on c_i.
    int hi_row[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) hi_row[qt] = CAUSAL ? min(kv_hi - 1, rq[qt] + off) : kv_hi - 1;

    // ---- S^T = K Q^T of the block in K buffer `kbuf`: each K fragment read
    // from LDS feeds the QT query tiles
    // bf16: the K fragments of a block, read from LDS ahead of their MFMAs
    constexpr int KFN = H16 ? QF * NS : 1;
    auto read_k = [&](int kbuf, u32x4_t (&kfr)[KFN]) __attribute__((always_inline)) {
      if constexpr (H16) {
#pragma unroll
        for (int ks = 0; ks < QF; ++ks)
#pragma unroll
          for (int st = 0; st < NS; ++st)
            kfr[ks * NS + st] = *(const u32x4_t*)(&sm.k[kbuf][(32 * st + r32) * S::KP + 16 * ks + 8 * hh]);
      }
    };
    auto qk_frag = [&](const u32x4_t (&kfr)[KFN], f32x16_t (&s)[QT][NS]) __attribute__((always_inline)) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int st = 0; st < NS; ++st) s[qt][st] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < QF; ++ks)
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) s[qt][st] = mfma16<H16>(kfr[ks * NS + st], qf4[qt][ks], s[qt][st]);
    };
    auto qk = [&](int kbuf, f32x16_t (&s)[QT][NS]) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int st = 0; st < NS; ++st) s[qt][st] = (f32x16_t){};
      if constexpr (H16) {
#pragma unroll
        for (int ks = 0; ks < QF; ++ks)
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const u32x4_t ka = *(const u32x4_t*)(&sm.k[kbuf][(32 * st + r32) * S::KP + 16 * ks + 8 * hh]);
#pragma unroll
            for (int qt = 0; qt < QT; ++qt) s[qt][st] = mfma16<H16>(ka, qf4[qt][ks], s[qt][st]);
          }
      } else {
#pragma unroll
        for (int G = 0; G < D / 8; ++G)
#pragma unroll
          for (int st = 0; st < NS; ++st) {
            const f32x4_t ka = *(const f32x4_t*)(&sm.k[kbuf][(32 * st + r32) * S::KP + 8 * G + 4 * hh]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
#pragma unroll
              for (int qt = 0; qt < QT; ++qt) s[qt][st] = mfma32_f32(ka[j], qff[qt][4 * G + j], s[qt][st]);
          }
      }
    };

    // bf16 V^T fragment of 16-key chunk kc (A operand of O^T += V^T P^T).  Its
    // k-slots must be the keys of the lane's P^T slots, i.e. of its score
    // registers: keys 4hh .. 4hh+3 and 8+4hh .. 8+4hh+3 of the chunk.  Lane l
    // holds dim 32*dt + l%32 of those keys, from two transposing reads of 4
    // keys each; in each group of 16 lanes, lane s points at key s/4 of the
    // four, dims 4*(s%4) .. +4 of the group's 16.
    const int vlane = (4 * hh + ((lane >> 2) & 3)) * S::VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
    auto read_vfrag = [&](int vbuf, int kc, u32x4_t (&dst)[DT]) __attribute__((always_inline)) {
      if constexpr (H16) {
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const T* p = &sm.v[vbuf][vlane + 16 * kc * S::VP + 32 * dt];
          const u32x2_t lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * S::VP);
          dst[dt] = (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
        }
      }
    };

    // ---- softmax of one block's scores, in two parts: mask / bias, row max
    // and the lazy rescale; then P and O^T += V^T P^T.  MASK: some score of
    // the wave's tile is invisible.  Scores are rewritten in place.
    auto softmax_max = [&](auto mask_tag, int kb, f32x16_t (&s)[QT][NS]) __attribute__((always_inline)) {
      constexpr bool MASK = decltype(mask_tag)::value;
      // bias (log2 units) and mask; without a bias the scores stay raw and the
      // scale is applied inside the exponent's FMA
      const int lo_rel = -kb - 4 * hh;  // c_i >= lo_rel  <=>  kj >= 0
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const unsigned span = (unsigned)max(hi_row[qt] + 1, 0);  // kj <= hi_row (none if < 0)
        float bv[HAS_BIAS ? NS : 1][16];
        if constexpr (HAS_BIAS) {
          if constexpr (BTILE) {
            // this lane's row of the staged tile: piece 4st + j, its half hh
            const int row = WR * wid + 32 * qt + r32;
            const uint16_t* rp = fbias + ((kb - kb0) / BN & 1) * BM * BN + row * BN + 4 * hh;
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const u32x2_t x = *(const u32x2_t*)(rp + 8 * ((4 * st + j) ^ (row & 7)));
                bv[st][4 * j + 0] = lo16<H16>(x[0]);
                bv[st][4 * j + 1] = hi16<H16>(x[0]);
                bv[st][4 * j + 2] = lo16<H16>(x[1]);
                bv[st][4 * j + 3] = hi16<H16>(x[1]);
              }
          } else if (a.bias_vec) {
            // registers 4j .. 4j+3 of a score tile are 4 consecutive keys: one 8-byte
            // (bf16) or 16-byte (f32) load each; keys past the sequence are masked
            // below, rows outside it are never stored
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                const int off = boff[qt] + (kb + 32 * st + 8 * j) * ELT;
                if constexpr (H16) {
                  const u32x2_t x = buf_load8(bres, off);
                  bv[st][4 * j + 0] = lo16<H16>(x[0]);
                  bv[st][4 * j + 1] = hi16<H16>(x[0]);
                  bv[st][4 * j + 2] = lo16<H16>(x[1]);
                  bv[st][4 * j + 3] = hi16<H16>(x[1]);
                } else {
                  const u32x4_t x = buf_load16(bres, off);
#pragma unroll
                  for (int e = 0; e < 4; ++e) bv[st][4 * j + e] = __uint_as_float(x[e]);
                }
              }
          } else {
            // any other layout: one element per load, same resource
#pragma unroll
            for (int st = 0; st < NS; ++st)
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                const int off = boff[qt] + (kb + 32 * st + 8 * (i >> 2) + (i & 3)) * (int)a.bs3 * ELT;
                if constexpr (H16)
                  bv[st][i] = lo16<H16>(__builtin_amdgcn_raw_buffer_load_b16(bres, off, 0, 0));
                else
                  bv[st][i] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(bres, off, 0, 0));
              }
          }
        }
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ci = 32 * st + 8 * (i >> 2) + (i & 3);
            float v = s[qt][st][i];
            if constexpr (HAS_BIAS) v = __builtin_fmaf(bv[st][i], kLog2e, v * a.scale_log2);
            if constexpr (MASK) v = ((unsigned)(ci - lo_rel) < span) ? v : -INFINITY;
            s[qt][st][i] = v;
          }
      }
      // online softmax with a lazily moved reference max (log2 units): keep the
      // reference unless a row's max exceeds it by more than 8 (then p <= 2^8:
      // exact algebra, no overflow); moving it rescales O
      float mx[QT];
      bool move = false;
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        float m = -INFINITY;
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 16; i += 2) m = max3f(m, s[qt][st][i], s[qt][st][i + 1]);
        m = fmaxf(m, xor32(m));
        if constexpr (!HAS_BIAS) m *= a.scale_log2;  // raw scores: scale the max once (scale > 0)
        mx[qt] = m;
        move = move || (m > m_run[qt] + 8.f);
      }
      if (__builtin_amdgcn_ballot_w64(move) != 0) {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const float m_new = fmaxf(m_run[qt], mx[qt]);
          const float alpha = fast_exp2(m_run[qt] - (m_new == -INFINITY ? 0.f : m_new));
          m_run[qt] = m_new;
          l_run[qt] *= alpha;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[qt][dt][i] *= alpha;
        }
      }
    };
    auto exp_pv = [&](int vbuf, f32x16_t (&s)[QT][NS]) __attribute__((always_inline)) {
      float m_use[QT], psum[QT];
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        m_use[qt] = m_run[qt] == -INFINITY ? 0.f : m_run[qt];
        psum[qt] = 0.f;
      }
      auto p_of = [&](float v, int qt) {
        if constexpr (HAS_BIAS) return fast_exp2(v - m_use[qt]);
        else return fast_exp2(__builtin_fmaf(v, a.scale_log2, -m_use[qt]));
      };
      if constexpr (H16) {
        // 16-key chunks kc: P^T chunk = registers 8*(kc%2) .. +8 of score tile kc/2.
        // The V^T fragments of chunk kc+1 are read while chunk kc computes.
        u32x4_t vnext[DT];
        auto read_v = [&](int kc, u32x4_t (&dst)[DT]) { read_vfrag(vbuf, kc, dst); };
        read_v(0, vnext);
#pragma unroll
        for (int kc = 0; kc < 2 * NS; ++kc) {
          u32x4_t vcur[DT];
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) vcur[dt] = vnext[dt];
          if (kc + 1 < 2 * NS) read_v(kc + 1, vnext);
#pragma unroll
          for (int qt = 0; qt < QT; ++qt) {
            u32x4_t pb;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float p0 = p_of(s[qt][kc >> 1][8 * (kc & 1) + 2 * e], qt);
              const float p1 = p_of(s[qt][kc >> 1][8 * (kc & 1) + 2 * e + 1], qt);
              psum[qt] += p0 + p1;
              pb[e] = pack16<H16>(p0, p1);
            }
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) acc[qt][dt] = mfma16<H16>(vcur[dt], pb, acc[qt][dt]);
          }
        }
      } else {
#pragma unroll
        for (int qt = 0; qt < QT; ++qt)
#pragma unroll
          for (int st = 0; st < NS; ++st)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const float p = p_of(s[qt][st][i], qt);
              psum[qt] += p;
              const int key = 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
              for (int dt = 0; dt < DT; ++dt) {
                const float va = sm.v[vbuf][key * S::VP + 32 * dt + r32];
                acc[qt][dt] = mfma32_f32(va, p, acc[qt][dt]);
              }
            }
      }
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) l_run[qt] += psum[qt];
    };

    // ---- bf16 without bias, a block every row of the wave sees in full: the
    // MFMAs of S(n+1) and PV(n) and the exponentials of block n in an explicit
    // order.  Round kc (one per 16-key chunk) issues the S(n+1) MFMAs of its
    // k-steps and the PV MFMAs of chunk kc-1, each followed by a share of the
    // vector work of chunk kc (exponentials, bf16 packing, row sums), so the
    // matrix unit and the vector unit of the SIMD both have work that waits
    // on neither.  The row sums add the bf16-rounded P that the PV MFMAs use.
    constexpr int NCH = 2 * NS;  // 16-key chunks per block
    // MASK: a block on the diagonal (or past a row's last key): the scores of
    // invisible keys become -inf before the row max, and a wave none of whose
    // rows sees the block skips the arithmetic (its later blocks are invisible
    // too, so the S it would compute is never used).
    // par: n & 1 (a literal where the caller knows it, so the buffer offsets fold)
    auto step_fast = [&](auto mask_tag, int n, int par, f32x16_t (&sc)[QT][NS], f32x16_t (&sn)[QT][NS])
                         __attribute__((always_inline)) {
      if constexpr (QT == 1 && H16 && !HAS_BIAS && QF % NCH == 0) {
      constexpr bool MASK = decltype(mask_tag)::value;
      constexpr int KPR = QF / NCH;  // S k-steps per round
      const int kb = kb0 + n * BN;
      const int kbuf = par ^ 1, vbuf = par;
      ld.load_k(kres, krow_bytes, kb + 2 * BN);  // past the last block every row reads as zero
      ld.load_v(vres, vrow_bytes, kb + BN);
      if (!MASK || (wave_on && kb < wave_hi)) {
      if constexpr (MASK) {
        const int lo_rel = -kb - 4 * hh;                         // c_i >= lo_rel  <=>  key >= 0
        const unsigned span = (unsigned)max(hi_row[0] + 1, 0);  // key <= hi_row
#pragma unroll
        for (int st = 0; st < NS; ++st)
#pragma unroll
          for (int i = 0; i < 16; ++i) {
            const int ci = 32 * st + 8 * (i >> 2) + (i & 3);
            sc[0][st][i] = ((unsigned)(ci - lo_rel) < span) ? sc[0][st][i] : -INFINITY;
          }
      }
      u32x4_t kfr[KFN];
      read_k(kbuf, kfr);
      u32x4_t vf[NCH][DT];
      read_vfrag(vbuf, 0, vf[0]);
      // row max of block n (raw scores, four independent chains)
      float m4[4] = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
      for (int st = 0; st < NS; ++st)
#pragma unroll
        for (int i = 0; i < 16; i += 2) {
          const int c = (8 * st + i / 2) & 3;
          m4[c] = max3f(m4[c], sc[0][st][i], sc[0][st][i + 1]);
        }
      float m = fmaxf(fmaxf(m4[0], m4[1]), fmaxf(m4[2], m4[3]));
      m = fmaxf(m, xor32(m)) * a.scale_log2;
      if (__builtin_amdgcn_ballot_w64(m > m_run[0] + 8.f) != 0) {
        const float m_new = fmaxf(m_run[0], m);
        const float alpha = fast_exp2(m_run[0] - (m_new == -INFINITY ? 0.f : m_new));
        m_run[0] = m_new;
        l_run[0] *= alpha;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int i = 0; i < 16; ++i) acc[0][dt][i] *= alpha;
      }
      const float nmu = m_run[0] == -INFINITY ? 0.f : -m_run[0];
#pragma unroll
      for (int st = 0; st < NS; ++st) sn[0][st] = (f32x16_t){};
      float ps0 = 0.f, ps1 = 0.f;
      u32x4_t pb[NCH];
#pragma unroll
      for (int kc = 0; kc <= NCH; ++kc) {
        __builtin_amdgcn_sched_barrier(0);
        if (kc < NCH) {
#pragma unroll
          for (int r = 0; r < KPR; ++r)
#pragma unroll
            for (int st = 0; st < NS; ++st) {
              const int ks = kc * KPR + r;
              sn[0][st] = mfma16<H16>(kfr[ks * NS + st], qf4[0][ks], sn[0][st]);
            }
        }
        if (kc > 0) {
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) acc[0][dt] = mfma16<H16>(vf[kc - 1][dt], pb[kc - 1], acc[0][dt]);
        }
        if (kc + 1 < NCH) read_vfrag(vbuf, kc + 1, vf[kc + 1]);
        if (kc < NCH) {
          const int st = kc >> 1, i0 = 8 * (kc & 1);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = fast_exp2(__builtin_fmaf(sc[0][st][i0 + 2 * e], a.scale_log2, nmu));
            const float p1 = fast_exp2(__builtin_fmaf(sc[0][st][i0 + 2 * e + 1], a.scale_log2, nmu));
            pb[kc][e] = pack16<H16>(p0, p1);
          }
          ps0 = sum16<H16>(pb[kc][0], ps0);
          ps1 = sum16<H16>(pb[kc][1], ps1);
          ps0 = sum16<H16>(pb[kc][2], ps0);
          ps1 = sum16<H16>(pb[kc][3], ps1);
          // one MFMA, then a share of the vector work, in turn
#pragma unroll
          for (int g = 0; g < (kc > 0 ? DT : 0) + KPR * NS; ++g) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 6, 0);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      l_run[0] += ps0 + ps1;
      }
      ld.store_k(sm, par);
      ld.store_v(sm, par ^ 1);
      lds_barrier();
      }
    };

    // Pipeline: K runs one block ahead of V.  Iteration n computes S of block
    // n+1 (MFMA) while it runs the softmax of block n (VALU), then PV of block
    // n; it stages K(n+2) into the K buffer block n used and V(n+1) into the V
    // buffer block n-1 used, so one barrier per block suffices.
    auto active = [&](int j) { return j < nb && wave_on && kb0 + j * BN < wave_hi; };
    {
      Loader<H16, D> ld1;  // K(1) in flight with K(0) and V(0)
      if (btile) bias_dma(kb0, 0);
      ld.load_k(kres, krow_bytes, kb0);
      ld.load_v(vres, vrow_bytes, kb0);
      ld1.load_k(kres, krow_bytes, kb0 + BN);
      ld.store_k(sm, 0);
      ld.store_v(sm, 0);
      ld1.store_k(sm, 1);
    }
    if (btile) __builtin_amdgcn_s_waitcnt(kWaitVm0);  // the bias tile, loaded straight into LDS
    lds_barrier();
    f32x16_t s_cur[QT][NS];
    if (active(0)) qk(0, s_cur);
    lds_barrier();  // every wave has read K(0) before K(2) replaces it
    // the next item: a ticket taken at the start of this item's second-to-last
    // block, its plan entries loaded during the last (thread 0)
    NextItem<Plan> next_item{a.plan, a.hq, total_items, s_info[cur ^ 1]};
    auto fetch_next = [&](int n) __attribute__((always_inline)) { next_item.at(n, nb); };

    auto step = [&](auto mask_tag, int n) {  // n: block index inside the unit
      constexpr bool MASK = decltype(mask_tag)::value;
      const int kb = kb0 + n * BN;
      if (btile && n + 1 < nb) bias_dma(kb + BN, (n + 1) & 1);  // before the K/V prefetch
      ld.load_k(kres, krow_bytes, kb + 2 * BN);  // past the last block every row reads as zero
      ld.load_v(vres, vrow_bytes, kb + BN);
      f32x16_t s_nxt[QT][NS];
      if constexpr (!MASK) {
        // every wave with rows in the sequence sees all of block n; S of
        // block n + 1 needs no guard either (a block past the unit reads as
        // zeros and is never used), so the MFMAs of S(n + 1) and the
        // exponentials and PV of block n share one straight-line region and
        // are interleaved there
        if constexpr (H16) {
          u32x4_t kfr[KFN];
          read_k((n + 1) & 1, kfr);  // in flight during the row max
          softmax_max(mask_tag, kb, s_cur);
          qk_frag(kfr, s_nxt);
          exp_pv(n & 1, s_cur);
          if constexpr (!HAS_BIAS) {
            // S(n + 1) MFMAs between the exponentials of block n, then the PV
            // MFMAs between the rest
#pragma unroll
            for (int i = 0; i < QF * NS * QT; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x400, 2, 0);  // transcendental
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
            }
#pragma unroll
            for (int i = 0; i < 2 * NS * DT * QT; ++i) {
              __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
              __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
              __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
            }
          }
        } else {
          softmax_max(mask_tag, kb, s_cur);
          qk((n + 1) & 1, s_nxt);
          exp_pv(n & 1, s_cur);
        }
      } else {
        if (active(n + 1)) qk((n + 1) & 1, s_nxt);
        if (active(n)) {
          softmax_max(mask_tag, kb, s_cur);
          exp_pv(n & 1, s_cur);
        }
      }
      ld.store_k(sm, n & 1);
      ld.store_v(sm, (n + 1) & 1);
      if (btile) __builtin_amdgcn_s_waitcnt(kWaitVm0);  // block n + 1's bias tile has landed
      lds_barrier();
#pragma unroll
      for (int qt = 0; qt < QT; ++qt)
#pragma unroll
        for (int st = 0; st < NS; ++st) s_cur[qt][st] = s_nxt[qt][st];
    };
    // unmasked blocks, then the (at most a few) masked ones: two loops, so the
    // accumulators never merge from two code paths inside a loop
    int j = 0;
    if constexpr (H16 && !HAS_BIAS && QT == 1 && QF % NCH == 0) {
      f32x16_t s_alt[QT][NS];
      const std::integral_constant<bool, false> plain;
      const std::integral_constant<bool, true> masked;
      // j is even here and in the single step after the pairs
      for (; j + 1 < j_plain; j += 2) {
        fetch_next(j);
        step_fast(plain, j, 0, s_cur, s_alt);
        fetch_next(j + 1);
        step_fast(plain, j + 1, 1, s_alt, s_cur);
      }
      if (j < j_plain) {
        fetch_next(j);
        step_fast(plain, j, 0, s_cur, s_alt);
#pragma unroll
        for (int st = 0; st < NS; ++st) s_cur[0][st] = s_alt[0][st];
        ++j;
      }
      if constexpr (D <= 128) {
        for (; j + 1 < nb; j += 2) {
          fetch_next(j);
          step_fast(masked, j, j & 1, s_cur, s_alt);
          fetch_next(j + 1);
          step_fast(masked, j + 1, (j + 1) & 1, s_alt, s_cur);
        }
        if (j < nb) {
          fetch_next(j);
          step_fast(masked, j, j & 1, s_cur, s_alt);
          ++j;
        }
      } else {
        // head_dim 256: the generic masked step (a second copy of the round
        // schedule would not fit the register file)
        for (; j < nb; ++j) {
          fetch_next(j);
          step(masked, j);
        }
      }
    } else {
      for (; j < j_plain; ++j) {
        fetch_next(j);
        step(std::integral_constant<bool, false>(), j);
      }
      for (; j < nb; ++j) {
        fetch_next(j);
        step(std::integral_constant<bool, true>(), j);
      }
    }
    next_item.finish(nb);
    ++kth;

    // ---- epilogue: O = acc / l, LSE = (m + log2 l) * ln 2.  A chunk of a split
    // tile stores O and the base-2 LSE in float32 to its slot instead, and the
    // chunk that finishes last merges the tile's chunks in chunk order, per row
    // LSE = log2 sum_c 2^LSE_c and O = sum_c 2^(LSE_c - LSE) O_c (accumulated
    // with a running max), taking its own O and LSE from registers (the same
    // values it stored), so the result does not depend on which chunk that is.
    const int row_base = r1 - BM;  // tile row 0
    float inv_v[QT], lse_v[QT];
#pragma unroll
    for (int qt = 0; qt < QT; ++qt) {
      const float l_tot = l_run[qt] + xor32(l_run[qt]);
      inv_v[qt] = l_tot > 0.f ? 1.f / l_tot : 0.f;
      lse_v[qt] = l_tot > 0.f ? m_run[qt] + __builtin_log2f(l_tot) : -INFINITY;
    }
    // O = acc * inv_l and the LSE of the rows >= 0
    auto write_out = [&](int qt, float inv_l, float lse2) __attribute__((always_inline)) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt + 8 * a4 + 4 * hh;
          const float o0 = acc[qt][dt][4 * a4 + 0] * inv_l, o1 = acc[qt][dt][4 * a4 + 1] * inv_l;
          const float o2 = acc[qt][dt][4 * a4 + 2] * inv_l, o3 = acc[qt][dt][4 * a4 + 3] * inv_l;
          // rows < 0 fall outside the resource: the store is dropped
          if constexpr (H16) {
            buf_store8((u32x2_t){pack16<H16>(o0, o1), pack16<H16>(o2, o3)}, ores, rq[qt] * orow_bytes + d0 * 2);
          } else {
            buf_store16((u32x4_t){__float_as_uint(o0), __float_as_uint(o1), __float_as_uint(o2),
                                  __float_as_uint(o3)}, ores, rq[qt] * orow_bytes + d0 * 4);
          }
        }
      if (rq[qt] >= 0 && hh == 0) a.lse[(size_t)h * a.total_q + q0 + rq[qt]] = lse2 * kLn2;
    };
    if (slot < 0) {
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) write_out(qt, inv_v[qt], lse_v[qt]);
    } else {
      constexpr int SLOT_O = BM * D;  // floats of one (slot, head) block of O
#pragma unroll
      for (int qt = 0; qt < QT; ++qt) {
        const int rl = rq[qt] - row_base;  // 0 .. BM-1
        const rsrc_t pres = make_rsrc(a.part_o + ((size_t)slot * a.hq + h) * SLOT_O, (int64_t)SLOT_O * 4);
#pragma unroll
        for (int dt = 0; dt < DT; ++dt)
#pragma unroll
          for (int a4 = 0; a4 < 4; ++a4) {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc[qt][dt][4 * a4 + e] *= inv_v[qt];
            const f32x4_t o = {acc[qt][dt][4 * a4], acc[qt][dt][4 * a4 + 1], acc[qt][dt][4 * a4 + 2],
                               acc[qt][dt][4 * a4 + 3]};
            buf_store16_dev(as_u32x4(o), pres, (rl * D + 32 * dt + 8 * a4 + 4 * hh) * 4);
          }
        if (hh == 0) st_dev(&a.part_lse[((size_t)slot * a.hq + h) * BM + rl], lse_v[qt]);
      }
      if (split_done_last(&a.plan.left[si * a.hq + h], &s_last)) {
        const int4 sp = a.plan.splits[si];
        const int sb = uniform(sp.z), nch = uniform(sp.w), me = slot - sb;  // first slot, chunks, this chunk
        // chunks in order with a running max (each chunk's LSE and O are loaded
        // together, so a chunk costs one round trip); at head dim 256 the output
        // tiles go one at a time to bound the registers
        constexpr int G = D <= 128 ? DT : 1;
#pragma unroll
        for (int qt = 0; qt < QT; ++qt) {
          const int rl = rq[qt] - row_base;
          const float* pl = a.part_lse + ((size_t)sb * a.hq + h) * BM + rl;  // chunk c: + c * hq * BM
          float mx = -INFINITY, wsum = 0.f;
#pragma unroll
          for (int g0 = 0; g0 < DT; g0 += G) {
            f32x4_t mo[G][4];
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
              for (int a4 = 0; a4 < 4; ++a4) mo[j][a4] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
            float m_run_c = -INFINITY, w_run = 0.f;
            for (int c = 0; c < nch; ++c) {
              const bool own = c == me;
              const float lc = own ? lse_v[qt] : ld_dev(pl + (size_t)c * a.hq * BM);
              const float m_new = fmaxf(m_run_c, lc);
              const float a_old = m_run_c == -INFINITY ? 0.f : fast_exp2(m_run_c - m_new);
              const float a_c = lc == -INFINITY ? 0.f : fast_exp2(lc - m_new);
              w_run = w_run * a_old + a_c;
              if (own) {
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                  for (int a4 = 0; a4 < 4; ++a4)
                    mo[j][a4] = mo[j][a4] * a_old +
                                a_c * (f32x4_t){acc[qt][g0 + j][4 * a4], acc[qt][g0 + j][4 * a4 + 1],
                                                acc[qt][g0 + j][4 * a4 + 2], acc[qt][g0 + j][4 * a4 + 3]};
              } else {
                const rsrc_t cres =
                    make_rsrc(a.part_o + ((size_t)(sb + c) * a.hq + h) * SLOT_O, (int64_t)SLOT_O * 4);
#pragma unroll
                for (int j = 0; j < G; ++j)
#pragma unroll
                  for (int a4 = 0; a4 < 4; ++a4)
                    mo[j][a4] = mo[j][a4] * a_old +
                                a_c * buf_load16_dev(cres, (rl * D + 32 * (g0 + j) + 8 * a4 + 4 * hh) * 4);
              }
              m_run_c = m_new;
            }
#pragma unroll
            for (int j = 0; j < G; ++j)
#pragma unroll
              for (int a4 = 0; a4 < 4; ++a4)
#pragma unroll
                for (int e = 0; e < 4; ++e) acc[qt][g0 + j][4 * a4 + e] = mo[j][a4][e];
            mx = m_run_c;
            wsum = w_run;
          }
          inv_v[qt] = wsum > 0.f ? 1.f / wsum : 0.f;
          lse_v[qt] = wsum > 0.f ? mx + __builtin_log2f(wsum) : -INFINITY;
          write_out(qt, inv_v[qt], lse_v[qt]);
        }
      }
    }
    lds_barrier();
  }
}

}  // namespace

template <int H16, int D, bool CAUSAL, bool HAS_BIAS>
static hipError_t launch_fwd_t(const FwdArgs& a, int64_t items, hipStream_t st) {
  auto kern = fwd_kernel<H16, D, CAUSAL, 0>;
  if constexpr (HAS_BIAS) {
    kern = fwd_kernel<H16, D, CAUSAL, 1>;
    // the staged tile: 16-bit, 64-key blocks
    if constexpr (H16 != 0 && BlockN<H16, D>::value == 64)
      if (a.bias_tile) kern = fwd_kernel<H16, D, CAUSAL, 2>;
  }
  const int grid = resident_grid((const void*)kern, NT, items);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  timing_before(st, H16 == 2 ? "fwd_f16" : H16 ? "fwd_bf16" : "fwd_f32");
  hipLaunchKernelGGL(kern, dim3(grid), dim3(NT), 0, st, a);
  timing_after(st);
  return hipGetLastError();
}

template <int H16, int D>
static hipError_t launch_fwd_d(const FwdArgs& a, int64_t grid, hipStream_t st) {
  const bool has_bias = a.bias != nullptr;
  if (a.causal)
    return has_bias ? launch_fwd_t<H16, D, true, true>(a, grid, st)
                    : launch_fwd_t<H16, D, true, false>(a, grid, st);
  return has_bias ? launch_fwd_t<H16, D, false, true>(a, grid, st)
                  : launch_fwd_t<H16, D, false, false>(a, grid, st);
}

int fwd_block_m() { return block_m<true, 64>(); }
int fwd_block_n(bool bf16, int d) {
  // keys per block: by element size, and 32 at head_dim 256 (LDS)
  if (d > 128) return bf16 ? BlockN<1, 256>::value : BlockN<0, 256>::value;
  return bf16 ? BlockN<1, 64>::value : BlockN<0, 64>::value;
}

template <int H16>
static hipError_t launch_fwd_h(const FwdArgs& a, int64_t grid, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_fwd_d<H16, 32>(a, grid, st);
    case 64: return launch_fwd_d<H16, 64>(a, grid, st);
    case 96: return launch_fwd_d<H16, 96>(a, grid, st);
    case 128: return launch_fwd_d<H16, 128>(a, grid, st);
    case 256: return launch_fwd_d<H16, 256>(a, grid, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int64_t grid, hipStream_t st) {
  if (a.bf16 == 2) return launch_fwd_h<2>(a, grid, st);
  if (a.bf16) return launch_fwd_h<1>(a, grid, st);
  return launch_fwd_h<0>(a, grid, st);
}

}  // namespace va
