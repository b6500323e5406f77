// Decode steps: attention of a few new query tokens per sequence against the
// sequence's paged KV cache.
//
// A decode step reads every cached key and value once and does little
// arithmetic per byte (2 * n_rep * q_len flops per byte of K/V at 16 bits), so
// this kernel is bound by HBM, not by the matrix cores.  Its shape follows
// from that:
//
// * A work item is ONE wave: 32 rows, each a (new token, query head) pair of
//   one KV head's GQA group, against a chunk of the sequence's keys.  The
//   n_rep query heads that share a KV head sit in one tile, so K and V are
//   read once per KV head, not once per query head.
// * Each lane owns one key of every 32-key score tile and loads that key's K
//   row straight into the A operand of S^T = K Q^T (no LDS), and the same
//   key's V row, which goes through a wave-private LDS slice so that the
//   transposing LDS read (ds_read_b64_tr_b16) can hand out V^T fragments for
//   O^T += V^T P^T, exactly as in the packed forward kernel.
// * The page of a key is one block-table lookup per lane and tile; the page
//   index is clamped into the pool and keys past the chunk's end are clamped
//   to its last key (their scores are masked), so no address ever leaves the
//   cache, whatever the table holds.
// * Long caches are split into chunks of `chunk` keys so that the grid has
//   thousands of waves; a chunk writes its normalised partial O and base-2
//   LSE, and a merge kernel combines a sequence's chunks in chunk order
//   (deterministic).
//
// The same kernels serve packed (ragged) K/V without a page table: key j of
// sequence b is then row cu_k[b] + j, read through the token strides.
//
// Semantics (the packed forward's): bottom-right causal alignment, so query
// i of Lq sees keys j <= i + Lk - Lq; a row with no visible key gives O = 0
// and LSE = -inf.
#include "va_common.h"
#include "va_kernels.h"

namespace va {

namespace {

constexpr int KNT = 256;  // 4 independent waves per workgroup

template <int D>
struct KvShape {
  // keys per step: 8 KB of K and 8 KB of V per wave at d = 64 and 128 (4 KB each
  // at d = 32, where 128-key steps would leave no room for two workgroups per
  // CU; 6 KB at d = 96, whose steps must stay whole 32-key tiles)
  static constexpr int KB = D == 32 ? 64 : D == 96 ? 32 : 4096 / D;
  static_assert(KB % 32 == 0 && KB * D / 8 % 64 == 0, "steps of whole tiles and whole wave loads");
  static constexpr int NS = KB / 32;   // 32-key score tiles per step
  // LDS row pitches (elements) of the staged K and V blocks: K is read by rows
  // (16-byte reads, conflict-free at D + 8), V by transposing 8-byte reads, whose
  // 32 lanes at a time touch four consecutive rows and are conflict-free on the 64
  // banks at pitch D for d = 32 and 96 and D + 32 for d = 128; at d = 64 the
  // conflict-free pitch (96) would not leave room for two workgroups per CU
  static constexpr int KP = D + 8;
  static constexpr int VP = D == 32 || D == 96 ? D : D == 128 ? D + 32 : D + 8;
  static constexpr int KS = D / 16;    // MFMA k-steps over head_dim
  static constexpr int DT = D / 32;    // 32-wide tiles of head_dim in O^T
};

// Key addressing of the decode kernel.
enum KvMode { kPagedSmall = 0, kPagedBig = 1, kRagged = 2 };

// A sequence's key count and the first row of its keys (ragged mode).  Paged
// lengths are clamped to max_k (the table's reach); ragged ones only to the
// rows of K and V, since max_seqlen_k is a hint there.
__device__ __forceinline__ int kv_len(const KvArgs& a, int b, int& k0) {
  if (a.cu_k) {
    int k1;
    seq_bounds(a.cu_k, b, a.total_k, k0, k1);
    return k1 - k0;
  }
  k0 = 0;
  return min(max(a.seqlens_k[b], 0), a.max_k);
}

// Keys per chunk of a sequence of Lk keys: `chunk`, or a multiple of it for
// a sequence longer than nchunk chunks (a ragged sequence past the hint), so
// no sequence has more chunks than the partial slots hold.
__device__ __forceinline__ int kv_chunk_of(const KvArgs& a, int Lk) {
  const int64_t cap = (int64_t)a.chunk * a.nchunk;
  return Lk <= cap ? a.chunk : a.chunk * (int)((Lk + cap - 1) / cap);
}

// The additive bias of the packed forward's short-query path (BIAS; ragged K/V
// only): this lane's (row, key) element b*bs0 + h*bs1 + qpos*bs2 + key*bs3,
// through a resource over the KV group's heads of the sequence that ends after
// the last element a valid (head, row, key) reads; rows past the sequence are
// never stored and keys past it are masked, whatever they read.
template <int H16, int NS>
struct KvBias {
  static constexpr int ELT = H16 ? 2 : 4;
  rsrc_t res;
  int off = 0;  // this lane's head, row and key half, bytes
  float v[NS][16];
  __device__ __forceinline__ void init(const KvArgs& a, int b, int g, int h, int qpos, int hh, int Lq, int Lk) {
    const int h0 = g * a.n_rep;
    const int64_t last = Lq > 0 && Lk > 0
                             ? ((int64_t)(a.n_rep - 1) * a.bs1 + (int64_t)(Lq - 1) * a.bs2 + (int64_t)(Lk - 1) * a.bs3 + 1) * ELT
                             : 0;
    res = make_rsrc((const uint8_t*)a.bias + ((int64_t)b * a.bs0 + (int64_t)h0 * a.bs1) * ELT, (last + 3) & ~(int64_t)3);
    off = (int)(((int64_t)(h - h0) * a.bs1 + (int64_t)qpos * a.bs2 + (int64_t)(4 * hh) * a.bs3) * ELT);
  }
  // the values of keys kb + 32 st + 8 (i / 4) + 4 hh + i % 4 (register i of tile st):
  // four consecutive keys per load when bias_vec, else one element per load
  __device__ __forceinline__ void load(const KvArgs& a, int kb) {
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (a.bias_vec) {
          const int o = off + (kb + 32 * st + 8 * j) * ELT;
          if constexpr (H16) {
            const u32x2_t x = buf_load8(res, o);
            v[st][4 * j + 0] = lo16<H16>(x[0]);
            v[st][4 * j + 1] = hi16<H16>(x[0]);
            v[st][4 * j + 2] = lo16<H16>(x[1]);
            v[st][4 * j + 3] = hi16<H16>(x[1]);
          } else {
            const u32x4_t x = buf_load16(res, o);
#pragma unroll
            for (int e = 0; e < 4; ++e) v[st][4 * j + e] = __uint_as_float(x[e]);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const int o = off + (int)((int64_t)(kb + 32 * st + 8 * j + e) * a.bs3 * ELT);
            if constexpr (H16) v[st][4 * j + e] = lo16<H16>(__builtin_amdgcn_raw_buffer_load_b16(res, o, 0, 0));
            else v[st][4 * j + e] = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(res, o, 0, 0));
          }
        }
      }
  }
};

template <int H16, int D, bool CAUSAL, int MODE, bool BIAS = false>
__global__ __launch_bounds__(KNT, 2) void kv_decode_kernel(KvArgs a) {
  constexpr bool BIGPAGE = MODE == kPagedBig, RAGGED = MODE == kRagged;
  using SH = KvShape<D>;
  constexpr int KB = SH::KB, NS = SH::NS, KP = SH::KP, VP = SH::VP, KS = SH::KS, DT = SH::DT;
  __shared__ uint16_t sk_all[4][KB * KP];
  __shared__ uint16_t sv_all[4][KB * VP];

  const int lane = threadIdx.x & 63;
  const int wid = uniform(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const int r32 = lane & 31;
  uint16_t* sk = sk_all[wid];
  uint16_t* sv = sv_all[wid];

  // ---- items: (entry of the planner's list, KV head), KV heads fastest, so
  // the waves of a workgroup read the same keys of neighbouring heads
  // (adjacent in each cache row) at the same time.  An entry is one
  // (sequence, 32-row block, key chunk) with work, so a static round robin
  // gives every wave nearly the same work; a wave prefetches its next item's
  // entry during the current one.  Waves never synchronise: each runs its
  // items alone.
  const int n_items = uniform(a.plan[0]) * a.hkv;
  const int n_waves = (int)gridDim.x * 4;
  auto entry = [&](int it) {
    return it < n_items ? a.chunks[it / a.hkv] : (KvChunk){0, 0, 0, 0, 0, 0, 0, 1};
  };
  KvChunk nxt = entry((int)blockIdx.x * 4 + wid);
  for (int item = (int)blockIdx.x * 4 + wid; item < n_items; item += n_waves) {
  const KvChunk ent = nxt;
  nxt = entry(item + n_waves);
  const int g = item % a.hkv;
  const int b = uniform(ent.b), rb = uniform(ent.rb), c = uniform(ent.c);
  const int q0 = uniform(ent.q0), q1 = uniform(ent.q1), Lk = uniform(ent.lk), k0 = uniform(ent.k0);
  const int chunk = uniform(ent.chunk);
  const size_t slot = (size_t)item;  // partial slot: (entry, KV head)
  const int Lq = q1 - q0;
  const int nch = max(1, (Lk + chunk - 1) / chunk);
  const int off = Lk - Lq;

  // this lane's row: new token qpos, query head h.  A row block is a.rows
  // (<= 32) rows; lanes past it compute a column that is never stored.
  const int r = rb * a.rows + r32;
  const int qpos = r / a.n_rep;
  const int h = g * a.n_rep + (r - qpos * a.n_rep);
  const bool row_ok = r32 < a.rows && qpos < Lq;
  // keys of the chunk that some row of the block sees, and the steps that
  // every valid row of the block sees in full
  const int qpos_first = (rb * a.rows) / a.n_rep;
  const int qpos_last = min(Lq - 1, (rb * a.rows + a.rows - 1) / a.n_rep);
  const int kbeg = c * chunk;
  int kend = min(Lk, kbeg + chunk);
  if (CAUSAL) kend = min(kend, qpos_last + off + 1);
  const int nsteps = kend > kbeg ? (kend - kbeg + KB - 1) / KB : 0;
  int plain_end = kend;
  if (CAUSAL) plain_end = min(plain_end, qpos_first + off + 1);
  const int nplain = plain_end > kbeg ? (plain_end - kbeg) / KB : 0;
  const int hi = !row_ok ? -1 : (CAUSAL ? min(kend - 1, qpos + off) : kend - 1);
  KvBias<H16, NS> bias;
  if constexpr (BIAS) bias.init(a, b, g, h, qpos, hh, Lq, Lk);

  // ---- Q fragments (B operand of S^T = K Q^T); rows past the sequence read 0
  constexpr int ELT = 2;
  const size_t qrow = (size_t)a.q_rs;
  const rsrc_t qres = make_rsrc((const uint16_t*)a.q + (size_t)q0 * qrow, (int64_t)Lq * qrow * ELT);
  u32x4_t qf[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qf[ks] = buf_load16(qres, (int)((qpos * qrow + h * D + 16 * ks + 8 * hh) * ELT));

  // ---- cache rows.  Loads are coalesced: a step's K (and V) block is KB rows of
  // LPR 16-byte pieces (this KV head's D * 2 bytes of a key), and load
  // instruction i reads pieces 64i .. 64i+63 in order, so consecutive lanes read
  // consecutive pieces of one row and the wave reads 64 / LPR rows per
  // instruction (a row may straddle two when LPR does not divide 64, d = 96).
  // Both go through the wave's LDS slices: K is read back in the MFMA operand
  // layout, V through the transposing read.
  constexpr int LPR = D / 8;          // 16-byte pieces per row
  constexpr int NI = KB * LPR / 64;   // load instructions per step and tensor
  auto prow = [&](int i) { return (64 * i + lane) / LPR; };       // row of load i's piece
  auto pcol = [&](int i) { return (64 * i + lane) % LPR * 8; };   // its first element
  const uint16_t* __restrict__ kc = (const uint16_t*)a.k_cache;
  const uint16_t* __restrict__ vc = (const uint16_t*)a.v_cache;
  const int32_t* __restrict__ bt = RAGGED ? nullptr : a.block_table + (size_t)b * a.bt_stride;
  const int pmask = (1 << a.page_shift) - 1;
  // key of load i of step n (clamped to the chunk's last key)
  auto key_of = [&](int n, int i) { return min(kbeg + n * KB + prow(i), kend - 1); };
  // pages of the next step to load, fetched a step ahead: with pages of at
  // least KB keys a step lies in one page (steps start at multiples of KB),
  // so one uniform lookup per step; otherwise one per load and lane
  constexpr int NPG = BIGPAGE || RAGGED ? 1 : NI;
  int pg[NPG];
  auto fetch_pages = [&](int n) __attribute__((always_inline)) {
    if constexpr (RAGGED) {
      pg[0] = 0;
    } else if constexpr (BIGPAGE) {
      pg[0] = bt[uniform(kbeg + n * KB) >> a.page_shift];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) pg[i] = bt[key_of(n, i) >> a.page_shift];
    }
  };
  u32x4_t kr[NI], vr[NI];
  auto load_kv = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t row;
      if constexpr (RAGGED) {
        row = (int64_t)k0 + key_of(n, i);
      } else {
        const int page = min(max(pg[BIGPAGE ? 0 : i], 0), a.num_pages - 1);
        row = ((int64_t)page << a.page_shift) + (key_of(n, i) & pmask);
      }
      kr[i] = __builtin_nontemporal_load((const u32x4_t*)(kc + row * a.k_rs + g * D + pcol(i)));
      vr[i] = __builtin_nontemporal_load((const u32x4_t*)(vc + row * a.v_rs + g * D + pcol(i)));
    }
  };

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x16_t){};
  float m_run = -INFINITY, l_run = 0.f;  // running max (log2 units), this lane's half of the row sum

  // V^T fragments: lane l reads dim 32 dt + l % 32 of the keys its P^T slots
  // hold (4hh .. 4hh+3 and 8+4hh .. 8+4hh+3 of each 16-key chunk), two
  // transposing reads of four keys each
  const int vlane = (4 * hh + ((lane >> 2) & 3)) * VP + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);

  if (nsteps > 0) {
    fetch_pages(0);
    load_kv(0);
  }
  if (nsteps > 1) fetch_pages(1);
  for (int n = 0; n < nsteps; ++n) {
    // K(n) and V(n) into the wave's LDS slices (the previous step's reads of
    // them are done: one wave's LDS operations complete in order)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      *(u32x4_t*)(sk + prow(i) * KP + pcol(i)) = kr[i];
      *(u32x4_t*)(sv + prow(i) * VP + pcol(i)) = vr[i];
    }
    // the next step's K and V are in flight during all of this step's work
    // (their pages were fetched a step ago); then the pages of the step after
    if (n + 1 < nsteps) load_kv(n + 1);
    if (n + 2 < nsteps) fetch_pages(n + 2);
    if constexpr (BIAS) bias.load(a, kbeg + n * KB);
    // S^T = K Q^T, K fragments from LDS
    f32x16_t s[NS];
#pragma unroll
    for (int st = 0; st < NS; ++st) {
      s[st] = (f32x16_t){};
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const u32x4_t kf = *(const u32x4_t*)(sk + (32 * st + r32) * KP + 16 * ks + 8 * hh);
        s[st] = mfma16<H16>(kf, qf[ks], s[st]);
      }
    }

    // ---- online softmax (base 2); masked steps test every key against the row's last
    const int kb = kbeg + n * KB;
    const bool masked = n >= nplain;
    float mx = -INFINITY;
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float v = s[st][i] * a.scale_log2;
        if constexpr (BIAS) v = __builtin_fmaf(bias.v[st][i], kLog2e, v);
        if (masked) {
          const int kj = kb + 32 * st + 8 * (i >> 2) + 4 * hh + (i & 3);
          v = kj <= hi ? v : -INFINITY;
        }
        s[st][i] = v;
        mx = fmaxf(mx, v);
      }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while m_run is -inf
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;

    // ---- P (rounded to the input kind) and O^T += V^T P^T, 16 keys at a time
#pragma unroll
    for (int st = 0; st < NS; ++st)
#pragma unroll
      for (int kc16 = 0; kc16 < 2; ++kc16) {
        uint32_t w[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float p0 = fast_exp2(s[st][8 * kc16 + 2 * j] - m_use);
          const float p1 = fast_exp2(s[st][8 * kc16 + 2 * j + 1] - m_use);
          w[j] = pack16<H16>(p0, p1);
          l_run = sum16<H16>(w[j], l_run);
        }
        const u32x4_t bop = (u32x4_t){w[0], w[1], w[2], w[3]};
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const uint16_t* p = sv + vlane + (32 * st + 16 * kc16) * VP + 32 * dt;
          const u32x2_t lo = lds_read_tr16(p), hi2 = lds_read_tr16(p + 8 * VP);
          acc[dt] = mfma16<H16>((u32x4_t){lo[0], lo[1], hi2[0], hi2[1]}, bop, acc[dt]);
        }
      }
  }

  // ---- epilogue: O = acc / l and LSE, or this chunk's partials
  const float l_tot = l_run + xor32(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __builtin_log2f(l_tot) : -INFINITY;
  if (nch == 1) {
    if (row_ok) {
      uint16_t* po = (uint16_t*)a.out + ((size_t)(q0 + qpos) * a.hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt + 8 * a4 + 4 * hh;
          const float o0 = acc[dt][4 * a4 + 0] * inv_l, o1 = acc[dt][4 * a4 + 1] * inv_l;
          const float o2 = acc[dt][4 * a4 + 2] * inv_l, o3 = acc[dt][4 * a4 + 3] * inv_l;
          *(u32x2_t*)(po + d0) = (u32x2_t){pack16<H16>(o0, o1), pack16<H16>(o2, o3)};
        }
      if (hh == 0) a.lse[(size_t)h * a.total_q + q0 + qpos] = lse2 * kLn2;
    }
  } else if (row_ok) {
    float* po = a.part_o + (slot * a.rows + r32) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hh;
        *(f32x4_t*)(po + d0) = (f32x4_t){acc[dt][4 * a4 + 0] * inv_l, acc[dt][4 * a4 + 1] * inv_l,
                                         acc[dt][4 * a4 + 2] * inv_l, acc[dt][4 * a4 + 3] * inv_l};
      }
    if (hh == 0) a.part_lse[slot * a.rows + r32] = lse2;
  }
  }
}

// The float32 decode kernel: the same items, paging, chunks and online softmax
// as kv_decode_kernel, on the float32 MFMA (32x32x2, two k-slots a lane).
//  - Q: lane l keeps dims 8G + 4hh + j of its row (k-slot (G, j)) in
//    registers; K rows are staged in the wave's LDS slice and read 16 bytes
//    at a time (dims 8G + 4hh .. +3 of key r32), so the two k-slots of one
//    MFMA are dims 8G + j and 8G + 4 + j for K and Q alike.
//  - P never leaves registers: register i of a score tile holds key
//    8(i/4) + 4hh + i%4 of the lane's row, which is the B operand of
//    O^T += V^T P^T with those two keys as k-slots; the A operand is one V
//    element per lane (dim 32 dt + r32 of that key) read from the V slice.
//  - 32-key steps; LDS pitches d + 4 (K: sixteen 16-byte row reads at a time
//    touch 64 distinct banks) and d + 8 (V: the two rows an element read
//    touches, k and k + 4, fall in opposite bank halves).  At d = 96 and 128
//    a workgroup's slices need more than half of the LDS and the staging
//    registers more than half of the register file: one workgroup per CU.
template <int D>
struct KvShapeF32 {
  static constexpr int KB = 32;
  static constexpr int KP = D + 4, VP = D + 8;
  static constexpr int G8 = D / 8;   // 8-dim groups of Q (4 k-slot pairs each)
  static constexpr int DT = D / 32;
  static constexpr int LPR = D / 4;  // 16-byte pieces per row
  static constexpr int NI = KB * LPR / 64;
  static_assert(KB * LPR % 64 == 0, "whole wave loads");
};
template <int D>
constexpr int kv_f32_blocks() { return D <= 64 ? 2 : 1; }

template <int D, bool CAUSAL, int MODE, bool BIAS = false>
__global__ __launch_bounds__(KNT, (kv_f32_blocks<D>())) void kv_decode_f32_kernel(KvArgs a) {
  constexpr bool BIGPAGE = MODE == kPagedBig, RAGGED = MODE == kRagged;
  using SH = KvShapeF32<D>;
  constexpr int KB = SH::KB, KP = SH::KP, VP = SH::VP, G8 = SH::G8, DT = SH::DT, LPR = SH::LPR, NI = SH::NI;
  __shared__ __attribute__((aligned(16))) float sk_all[4][KB * KP];
  __shared__ __attribute__((aligned(16))) float sv_all[4][KB * VP];

  const int lane = threadIdx.x & 63;
  const int wid = uniform(threadIdx.x >> 6);
  const int hh = lane >> 5;
  const int r32 = lane & 31;
  float* sk = sk_all[wid];
  float* sv = sv_all[wid];

  const int n_items = uniform(a.plan[0]) * a.hkv;
  const int n_waves = (int)gridDim.x * 4;
  auto entry = [&](int it) {
    return it < n_items ? a.chunks[it / a.hkv] : (KvChunk){0, 0, 0, 0, 0, 0, 0, 1};
  };
  KvChunk nxt = entry((int)blockIdx.x * 4 + wid);
  for (int item = (int)blockIdx.x * 4 + wid; item < n_items; item += n_waves) {
  const KvChunk ent = nxt;
  nxt = entry(item + n_waves);
  const int g = item % a.hkv;
  const int b = uniform(ent.b), rb = uniform(ent.rb), c = uniform(ent.c);
  const int q0 = uniform(ent.q0), q1 = uniform(ent.q1), Lk = uniform(ent.lk), k0 = uniform(ent.k0);
  const int chunk = uniform(ent.chunk);
  const size_t slot = (size_t)item;
  const int Lq = q1 - q0;
  const int nch = max(1, (Lk + chunk - 1) / chunk);
  const int off = Lk - Lq;

  const int r = rb * a.rows + r32;
  const int qpos = r / a.n_rep;
  const int h = g * a.n_rep + (r - qpos * a.n_rep);
  const bool row_ok = r32 < a.rows && qpos < Lq;
  const int qpos_first = (rb * a.rows) / a.n_rep;
  const int qpos_last = min(Lq - 1, (rb * a.rows + a.rows - 1) / a.n_rep);
  const int kbeg = c * chunk;
  int kend = min(Lk, kbeg + chunk);
  if (CAUSAL) kend = min(kend, qpos_last + off + 1);
  const int nsteps = kend > kbeg ? (kend - kbeg + KB - 1) / KB : 0;
  int plain_end = kend;
  if (CAUSAL) plain_end = min(plain_end, qpos_first + off + 1);
  const int nplain = plain_end > kbeg ? (plain_end - kbeg) / KB : 0;
  const int hi = !row_ok ? -1 : (CAUSAL ? min(kend - 1, qpos + off) : kend - 1);
  KvBias<0, 1> bias;
  if constexpr (BIAS) bias.init(a, b, g, h, qpos, hh, Lq, Lk);

  // ---- Q (the B operand of S^T = K Q^T); rows past the sequence read 0
  const size_t qrow = (size_t)a.q_rs;
  const rsrc_t qres = make_rsrc((const float*)a.q + (size_t)q0 * qrow, (int64_t)Lq * qrow * 4);
  float qf[4 * G8];
#pragma unroll
  for (int G = 0; G < G8; ++G) {
    const u32x4_t z = buf_load16(qres, (int)((qpos * qrow + h * D + 8 * G + 4 * hh) * 4));
#pragma unroll
    for (int j = 0; j < 4; ++j) qf[4 * G + j] = __uint_as_float(z[j]);
  }

  // ---- cache rows: coalesced 16-byte pieces, load i covering pieces 64i .. 64i+63
  auto prow = [&](int i) { return (64 * i + lane) / LPR; };
  auto pcol = [&](int i) { return (64 * i + lane) % LPR * 4; };
  const float* __restrict__ kc = (const float*)a.k_cache;
  const float* __restrict__ vc = (const float*)a.v_cache;
  const int32_t* __restrict__ bt = RAGGED ? nullptr : a.block_table + (size_t)b * a.bt_stride;
  const int pmask = (1 << a.page_shift) - 1;
  auto key_of = [&](int n, int i) { return min(kbeg + n * KB + prow(i), kend - 1); };
  constexpr int NPG = BIGPAGE || RAGGED ? 1 : NI;
  int pg[NPG];
  auto fetch_pages = [&](int n) __attribute__((always_inline)) {
    if constexpr (RAGGED) {
      pg[0] = 0;
    } else if constexpr (BIGPAGE) {
      pg[0] = bt[uniform(kbeg + n * KB) >> a.page_shift];
    } else {
#pragma unroll
      for (int i = 0; i < NI; ++i) pg[i] = bt[key_of(n, i) >> a.page_shift];
    }
  };
  u32x4_t kr[NI], vr[NI];
  auto load_kv = [&](int n) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      int64_t row;
      if constexpr (RAGGED) {
        row = (int64_t)k0 + key_of(n, i);
      } else {
        const int page = min(max(pg[BIGPAGE ? 0 : i], 0), a.num_pages - 1);
        row = ((int64_t)page << a.page_shift) + (key_of(n, i) & pmask);
      }
      kr[i] = __builtin_nontemporal_load((const u32x4_t*)(kc + row * a.k_rs + g * D + pcol(i)));
      vr[i] = __builtin_nontemporal_load((const u32x4_t*)(vc + row * a.v_rs + g * D + pcol(i)));
    }
  };

  f32x16_t acc[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) acc[dt] = (f32x16_t){};
  float m_run = -INFINITY, l_run = 0.f;

  if (nsteps > 0) {
    fetch_pages(0);
    load_kv(0);
  }
  if (nsteps > 1) fetch_pages(1);
  for (int n = 0; n < nsteps; ++n) {
    // K(n), V(n) into the wave's slices (its earlier reads of them are done:
    // one wave's LDS operations complete in order)
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      *(u32x4_t*)(sk + prow(i) * KP + pcol(i)) = kr[i];
      *(u32x4_t*)(sv + prow(i) * VP + pcol(i)) = vr[i];
    }
    if (n + 1 < nsteps) load_kv(n + 1);
    if (n + 2 < nsteps) fetch_pages(n + 2);
    if constexpr (BIAS) bias.load(a, kbeg + n * KB);
    // S^T = K Q^T
    f32x16_t s = (f32x16_t){};
#pragma unroll
    for (int G = 0; G < G8; ++G) {
      const f32x4_t ka = *(const f32x4_t*)(sk + r32 * KP + 8 * G + 4 * hh);
#pragma unroll
      for (int j = 0; j < 4; ++j) s = mfma32_f32(ka[j], qf[4 * G + j], s);
    }
    // ---- online softmax (base 2); masked steps test every key against the row's last
    const int kb = kbeg + n * KB;
    const bool masked = n >= nplain;
    float mx = -INFINITY;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float v = s[i] * a.scale_log2;
      if constexpr (BIAS) v = __builtin_fmaf(bias.v[0][i], kLog2e, v);
      if (masked) {
        const int kj = kb + 8 * (i >> 2) + 4 * hh + (i & 3);
        v = kj <= hi ? v : -INFINITY;
      }
      s[i] = v;
      mx = fmaxf(mx, v);
    }
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = m_new == -INFINITY ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);  // 0 while m_run is -inf
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int i = 0; i < 16; ++i) acc[dt][i] *= alpha;
    // ---- P and O^T += V^T P^T, two keys (k-slots) per MFMA
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const float p = fast_exp2(s[i] - m_use);
      l_run += p;
      const int key = 8 * (i >> 2) + 4 * hh + (i & 3);
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) acc[dt] = mfma32_f32(sv[key * VP + 32 * dt + r32], p, acc[dt]);
    }
  }

  // ---- epilogue: O = acc / l and LSE, or this chunk's partials
  const float l_tot = l_run + xor32(l_run);
  const float inv_l = l_tot > 0.f ? 1.f / l_tot : 0.f;
  const float lse2 = l_tot > 0.f ? m_run + __builtin_log2f(l_tot) : -INFINITY;
  if (nch == 1) {
    if (row_ok) {
      float* po = (float*)a.out + ((size_t)(q0 + qpos) * a.hq + h) * D;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int a4 = 0; a4 < 4; ++a4) {
          const int d0 = 32 * dt + 8 * a4 + 4 * hh;
          *(f32x4_t*)(po + d0) = (f32x4_t){acc[dt][4 * a4 + 0] * inv_l, acc[dt][4 * a4 + 1] * inv_l,
                                           acc[dt][4 * a4 + 2] * inv_l, acc[dt][4 * a4 + 3] * inv_l};
        }
      if (hh == 0) a.lse[(size_t)h * a.total_q + q0 + qpos] = lse2 * kLn2;
    }
  } else if (row_ok) {
    float* po = a.part_o + (slot * a.rows + r32) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = 32 * dt + 8 * a4 + 4 * hh;
        *(f32x4_t*)(po + d0) = (f32x4_t){acc[dt][4 * a4 + 0] * inv_l, acc[dt][4 * a4 + 1] * inv_l,
                                         acc[dt][4 * a4 + 2] * inv_l, acc[dt][4 * a4 + 3] * inv_l};
      }
    if (hh == 0) a.part_lse[slot * a.rows + r32] = lse2;
  }
  }
}

// The planner: one workgroup lists every (sequence, row block, key chunk)
// with work, in that order (chunks fastest), with the sequence's bounds
// (clamped as the decode kernel needs them), and stores the count in
// plan[0].  A sequence with Lq new tokens has ceil(Lq * n_rep / rows) row
// blocks of max(1, ceil(Lk / chunk)) chunks each (an empty cache still owes
// its rows O = 0 and LSE = -inf); one without new tokens has none.  The
// list never outgrows a.cap entries (the host's bound); entries past it are
// dropped, which only bad metadata can cause.
constexpr int kPlanThreads = 1024;
__global__ __launch_bounds__(kPlanThreads) void kv_plan_kernel(KvArgs a) {
  __shared__ int scan[kPlanThreads], mscan[kPlanThreads];
  __shared__ int s_base, s_mbase;
  const int tid = threadIdx.x;
  if (tid == 0) s_base = s_mbase = 0;
  __syncthreads();
  for (int b0 = 0; b0 < a.batch; b0 += kPlanThreads) {
    const int b = b0 + tid;
    int q0 = 0, q1 = 0, lk = 0, k0 = 0, ch = 1, nch = 0, nrb = 0;
    if (b < a.batch) {
      seq_bounds(a.cu_q, b, a.total_q, q0, q1);
      lk = kv_len(a, b, k0);
      ch = kv_chunk_of(a, lk);
      nch = max(1, (lk + ch - 1) / ch);
      nrb = (int)(((int64_t)(q1 - q0) * a.n_rep + a.rows - 1) / a.rows);
    }
    const int cnt = nrb * nch;                // list entries of the sequence
    const int mcnt = nch > 1 ? nrb : 0;        // its row blocks that need a merge
    // inclusive scans of both counts (Hillis-Steele over the workgroup)
    scan[tid] = cnt;
    mscan[tid] = mcnt;
    __syncthreads();
    for (int o = 1; o < kPlanThreads; o <<= 1) {
      const int add = tid >= o ? scan[tid - o] : 0, madd = tid >= o ? mscan[tid - o] : 0;
      __syncthreads();
      scan[tid] += add;
      mscan[tid] += madd;
      __syncthreads();
    }
    const int base = s_base + scan[tid] - cnt, mbase = s_mbase + mscan[tid] - mcnt;
    for (int e = 0; e < cnt; ++e)
      if (base + e < a.cap) a.chunks[base + e] = (KvChunk){b, e / nch, e % nch, q0, q1, lk, k0, ch};
    for (int r = 0; r < mcnt; ++r)
      if (mbase + r < a.cap_merge) a.merges[mbase + r] = base + r * nch;  // entry of chunk 0
    __syncthreads();
    if (tid == kPlanThreads - 1) {
      s_base += scan[tid];
      s_mbase += mscan[tid];
    }
    __syncthreads();
  }
  if (tid == 0) {
    a.plan[0] = min(s_base, a.cap);
    a.plan[1] = min(s_mbase, a.cap_merge);
  }
}

// Combines the chunks of every row block that has more than one:
// LSE = log2 sum_c 2^LSE_c and O = sum_c 2^(LSE_c - LSE) O_c, in chunk order.
// Work items are (row block of the planner's merge list, KV head); the list
// holds the entry of the block's chunk 0, and its other chunks are the
// entries that follow it.  Eight threads per row.
template <int H16, int D>
__global__ __launch_bounds__(KNT) void kv_merge_kernel(KvArgs a) {
  constexpr int TPR = 8, SEG = D / TPR;
  const int n_items = uniform(a.plan[1]) * a.hkv;
  const int row = threadIdx.x / TPR, seg = threadIdx.x % TPR;
  for (int item = (int)blockIdx.x; item < n_items; item += (int)gridDim.x) {
    const int e0 = uniform(a.merges[item / a.hkv]), g = item % a.hkv;
    const KvChunk ent = a.chunks[e0];
    const int rb = uniform(ent.rb);
    const int q0 = uniform(ent.q0), Lq = uniform(ent.q1) - q0;
    const int nch = max(1, (uniform(ent.lk) + uniform(ent.chunk) - 1) / uniform(ent.chunk));
    if (nch == 1 || e0 + nch > a.cap) continue;
    const int r = rb * a.rows + row;
    const int qpos = r / a.n_rep;
    if (qpos >= Lq || row >= a.rows) continue;
    const int h = g * a.n_rep + (r - qpos * a.n_rep);
    float mx = -INFINITY;
    for (int cc = 0; cc < nch; ++cc)
      mx = fmaxf(mx, a.part_lse[((size_t)(e0 + cc) * a.hkv + g) * a.rows + row]);
    f32x4_t acc[SEG / 4];
#pragma unroll
    for (int e = 0; e < SEG / 4; ++e) acc[e] = (f32x4_t){0.f, 0.f, 0.f, 0.f};
    float wsum = 0.f;
    if (mx != -INFINITY) {
      for (int cc = 0; cc < nch; ++cc) {
        const size_t sl = (size_t)(e0 + cc) * a.hkv + g;
        const float w = fast_exp2(a.part_lse[sl * a.rows + row] - mx);
        wsum += w;
        const f32x4_t* src = (const f32x4_t*)(a.part_o + (sl * a.rows + row) * D + seg * SEG);
#pragma unroll
        for (int e = 0; e < SEG / 4; ++e) acc[e] += w * src[e];
      }
    }
    const float inv = wsum > 0.f ? 1.f / wsum : 0.f;
    const size_t o0 = ((size_t)(q0 + qpos) * a.hq + h) * D + seg * SEG;
#pragma unroll
    for (int e = 0; e < SEG / 4; ++e) {
      const f32x4_t x = acc[e] * inv;
      if constexpr (H16) {
        *(u32x2_t*)((uint16_t*)a.out + o0 + 4 * e) = (u32x2_t){pack16<H16>(x[0], x[1]), pack16<H16>(x[2], x[3])};
      } else {
        *(f32x4_t*)((float*)a.out + o0 + 4 * e) = x;
      }
    }
    if (seg == 0)
      a.lse[(size_t)h * a.total_q + q0 + qpos] = wsum > 0.f ? (mx + __builtin_log2f(wsum)) * kLn2 : -INFINITY;
  }
}

template <int H16, int D, bool CAUSAL>
hipError_t launch_kv_t(const KvArgs& a, hipStream_t st) {
  const int64_t items = (int64_t)a.cap * a.hkv;
  void (*kern)(KvArgs);
  if (a.bias) {
    // the packed forward's short-query path (ragged K/V) with an additive bias
    if constexpr (H16 != 0) kern = kv_decode_kernel<H16, D, CAUSAL, kRagged, true>;
    else kern = kv_decode_f32_kernel<D, CAUSAL, kRagged, true>;
  } else if constexpr (H16 != 0) {
    kern = a.cu_k ? kv_decode_kernel<H16, D, CAUSAL, kRagged>
           : (1 << a.page_shift) >= KvShape<D>::KB ? kv_decode_kernel<H16, D, CAUSAL, kPagedBig>
                                                   : kv_decode_kernel<H16, D, CAUSAL, kPagedSmall>;
  } else {
    kern = a.cu_k ? kv_decode_f32_kernel<D, CAUSAL, kRagged>
           : (1 << a.page_shift) >= KvShapeF32<D>::KB ? kv_decode_f32_kernel<D, CAUSAL, kPagedBig>
                                                      : kv_decode_f32_kernel<D, CAUSAL, kPagedSmall>;
  }
  const int grid = resident_grid((const void*)kern, KNT, (items + 3) / 4);
  if (grid <= 0) return hipErrorInvalidConfiguration;
  timing_before(st, "kvcache_plan");
  hipLaunchKernelGGL(kv_plan_kernel, dim3(1), dim3(kPlanThreads), 0, st, a);
  timing_after(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_before(st, H16 == 2 ? "kvcache_f16" : H16 ? "kvcache_bf16" : "kvcache_f32");
  hipLaunchKernelGGL(kern, dim3(grid), dim3(KNT), 0, st, a);
  timing_after(st);
  e = hipGetLastError();
  if (e != hipSuccess || a.nchunk <= 1) return e;
  int64_t mg = (int64_t)a.cap_merge * a.hkv;
  if (mg > 2048) mg = 2048;
  if (mg < 1) mg = 1;
  timing_before(st, "kvcache_merge");
  hipLaunchKernelGGL((kv_merge_kernel<H16, D>), dim3((unsigned)mg), dim3(KNT), 0, st, a);
  timing_after(st);
  return hipGetLastError();
}

template <int H16, int D>
hipError_t launch_kv_d(const KvArgs& a, hipStream_t st) {
  return a.causal ? launch_kv_t<H16, D, true>(a, st) : launch_kv_t<H16, D, false>(a, st);
}

}  // namespace

int kv_block_n(int d) {
  return d == 32 ? KvShape<32>::KB : d == 64 ? KvShape<64>::KB : d == 96 ? KvShape<96>::KB : KvShape<128>::KB;
}

template <int H16>
hipError_t launch_kv_h(const KvArgs& a, hipStream_t st) {
  switch (a.d) {
    case 32: return launch_kv_d<H16, 32>(a, st);
    case 64: return launch_kv_d<H16, 64>(a, st);
    case 96: return launch_kv_d<H16, 96>(a, st);
    case 128: return launch_kv_d<H16, 128>(a, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_kvcache(const KvArgs& a, hipStream_t st) {
  if (a.h16 == 0) return launch_kv_h<0>(a, st);
  return a.h16 == 2 ? launch_kv_h<2>(a, st) : launch_kv_h<1>(a, st);
}

}  // namespace va
