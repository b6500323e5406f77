// Planner body (see va_plan.hip): device code shared by the forward's
// planner kernel and the backward's fused planner + preprocess kernel.  Must
// run in a workgroup of PT threads.
#pragma once
#include <limits.h>

#include "va_common.h"
#include "va_kernels.h"

namespace va {
namespace plan {

constexpr int PT = 1024;    // planner threads
constexpr int NBIN = 2048;  // step-count bins (larger counts share the last bin)

// Steps of tile t of a sequence (Lt rows on the tiled side, Lo on the other).
__device__ __forceinline__ int tile_steps(const PlanArgs& p, int Lt, int Lo, int t) {
  if (p.kside == 0) {
    // query tile t covers rows [Lq - (t+1)*tile, Lq - t*tile); with the
    // bottom-right causal mask its last row sees keys < r1 + Lk - Lq
    const int Lq = Lt, Lk = Lo;
    const int r1 = Lq - t * p.tile;
    int hi = p.causal ? min(Lk, r1 + (Lk - Lq)) : Lk;
    hi = max(hi, 0);
    return (hi + p.step - 1) / p.step;
  }
  // key tile t covers keys [t*tile, (t+1)*tile); causal: query i sees key j
  // iff j <= i + Lk - Lq, so the first query that sees the tile is kt0 - off
  const int Lk = Lt, Lq = Lo;
  const int kt0 = t * p.tile;
  const int qs = p.causal ? max(0, kt0 - (Lk - Lq)) : 0;
  return qs < Lq ? (Lq - qs + p.step - 1) / p.step : 0;
}

__device__ __forceinline__ int chunks_of(int steps, int chunk) {
  return steps > chunk ? (steps + chunk - 1) / chunk : 1;
}

// Chunk c of a tile of s = q * nch + r steps (0 <= r < nch): the first r
// chunks have q + 1 steps, the others q.
__device__ __forceinline__ void chunk_range(int q, int r, int c, int& n0, int& n1) {
  n0 = c * q + min(c, r);
  n1 = n0 + q + (c < r ? 1 : 0);
}


// Tiles are visited spread over the threads: the sequences are taken MAXB at
// a time, their tile counts scanned in LDS, and each thread finds the
// sequence of its tile by binary search.  When the batch fits one such
// block and has at most TPT * PT tiles (the usual case), every thread keeps
// its tiles (sequence, tile, steps) in registers, so the later passes
// neither reload cu_seqlens nor search again.
constexpr int MAXB = 2048;
constexpr int TPT = 4;    // cached tiles per thread
constexpr int NCAND = 6;  // chunk candidates: chunk << 0 .. chunk << 5

struct PlanShared {
  int bins[NBIN];
  int tstart[MAXB + 1];  // exclusive scan of the tile counts of the current block of sequences
  int st[MAXB];          // tiled-side first row
  int lt[MAXB];          // tiled-side length
  int so[MAXB];          // other-side first row
  int lo[MAXB];          // other-side length
  int wsum[PT / 64];
  int cnt[NCAND];        // partial slots per chunk candidate
  int slot_ctr, split_ctr;
};

// Block-wide exclusive scan of one int per thread; returns the total.
__device__ inline int block_scan(int x, int* wsum, int& excl) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) wsum[wid] = incl;
  __syncthreads();
  int before = 0, total = 0;
  for (int w = 0; w < PT / 64; ++w) {
    const int v = wsum[w];
    if (w < wid) before += v;
    total += v;
  }
  excl = before + incl - x;
  __syncthreads();
  return total;
}

// Loads the lengths of sequences b0 .. b0+nb-1 and scans their tile counts;
// returns the number of tiles.
__device__ inline int load_block(const PlanArgs& p, PlanShared& sh, int b0, int nb) {
  int cnt[2] = {0, 0};
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int i = 2 * threadIdx.x + e;
    if (i < nb) {
      int t0, t1, o0, o1;
      seq_bounds(p.cu_t, b0 + i, p.total_t, t0, t1);
      seq_bounds(p.cu_o, b0 + i, p.total_o, o0, o1);
      sh.st[i] = t0;
      sh.lt[i] = t1 - t0;
      sh.so[i] = o0;
      sh.lo[i] = o1 - o0;
      cnt[e] = (t1 - t0 + p.tile - 1) / p.tile;
    }
  }
  int excl;
  const int ntiles = block_scan(cnt[0] + cnt[1], sh.wsum, excl);
  if (2 * threadIdx.x < nb) sh.tstart[2 * threadIdx.x] = excl;
  if (2 * threadIdx.x + 1 < nb) sh.tstart[2 * threadIdx.x + 1] = excl + cnt[0];
  if (threadIdx.x == 0) sh.tstart[nb] = ntiles;
  __syncthreads();
  return ntiles;
}

// Sequence (inside the block) of tile i: the last one with tstart <= i.
__device__ __forceinline__ int find_seq(const PlanShared& sh, int nb, int i) {
  int lo_ = 0, hi_ = nb - 1;
  while (lo_ < hi_) {
    const int mid = (lo_ + hi_ + 1) >> 1;
    if (sh.tstart[mid] <= i) lo_ = mid; else hi_ = mid - 1;
  }
  return lo_;
}

// f(sequence, tile, steps, q) for every tile (the general path); q indexes
// the sequence's entries in sh during the call.
template <typename F>
__device__ void for_each_tile(const PlanArgs& p, PlanShared& sh, F&& f) {
  for (int b0 = 0; b0 < p.batch; b0 += MAXB) {
    const int nb = min(MAXB, p.batch - b0);
    const int ntiles = load_block(p, sh, b0, nb);
    for (int i = threadIdx.x; i < ntiles; i += PT) {
      const int q = find_seq(sh, nb, i);
      const int t = i - sh.tstart[q];
      f(b0 + q, t, tile_steps(p, sh.lt[q], sh.lo[q], t), q);
    }
    __syncthreads();
  }
}

__device__ __forceinline__ void plan_body(const PlanArgs& p, PlanShared& sh) {
  static_assert(2 * PT == MAXB, "two sequences per thread");
  static_assert(2 * PT == NBIN, "two bins per thread");
  const int tid = threadIdx.x;

  // tile cache (fast path)
  int cb[TPT], ct[TPT], cs[TPT];
  bool fast = p.batch <= MAXB;
  if (fast) {
    const int ntiles = load_block(p, sh, 0, p.batch);
    fast = ntiles <= TPT * PT;
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int i = tid + j * PT;
      cs[j] = -1;
      if (fast && i < ntiles) {
        const int q = find_seq(sh, p.batch, i);
        cb[j] = q;
        ct[j] = i - sh.tstart[q];
        cs[j] = tile_steps(p, sh.lt[q], sh.lo[q], ct[j]);
      }
    }
    __syncthreads();
  }
  auto visit = [&](auto&& f) {
    if (fast) {
#pragma unroll
      for (int j = 0; j < TPT; ++j)
        if (cs[j] >= 0) f(cb[j], ct[j], cs[j], cb[j]);
    } else {
      for_each_tile(p, sh, f);
    }
  };

  // (1) partial slots each chunk candidate needs (a split tile of nch chunks
  // takes nch slots)
  if (tid < NCAND) sh.cnt[tid] = 0;
  __syncthreads();
  const int chunk0 = max(p.chunk, 1);
  {
    int sl[NCAND];
#pragma unroll
    for (int j = 0; j < NCAND; ++j) sl[j] = 0;
    visit([&](int, int, int s, int) {
      // ceil(s / (chunk0 << j)) = ceil(ceil(s / chunk0) / 2^j): one division
      const int n = (s + chunk0 - 1) / chunk0;
#pragma unroll
      for (int j = 0; j < NCAND; ++j) {
        const int nch = (n + (1 << j) - 1) >> j;
        if (nch > 1) sl[j] += nch;
      }
    });
    // a wave with a split tile (candidate 0 splits whatever a larger one does)
    // sums every candidate with a butterfly of shuffles over all its lanes, the
    // candidates' shuffles of one distance issued together so their round trips
    // overlap, and lane 0 adds each sum with one LDS atomic; the other waves
    // skip the reduction
    if (__builtin_amdgcn_ballot_w64(sl[0] > 0) != 0) {
#pragma unroll
      for (int o = 32; o > 0; o >>= 1) {
        int t[NCAND];
#pragma unroll
        for (int j = 0; j < NCAND; ++j) t[j] = __shfl_xor(sl[j], o, 64);
#pragma unroll
        for (int j = 0; j < NCAND; ++j) sl[j] += t[j];
      }
      if ((threadIdx.x & 63) == 0) {
#pragma unroll
        for (int j = 0; j < NCAND; ++j)
          if (sl[j] > 0) atomicAdd(&sh.cnt[j], sl[j]);
      }
    }
  }
  __syncthreads();
  // the smallest chunk whose partial results fit the workspace (each split
  // tile takes >= 2 slots, so the split list fits too)
  int pick = NCAND;
  for (int j = NCAND - 1; j >= 0; --j)
    if (sh.cnt[j] <= p.slot_cap) pick = j;
  const int chunk = pick < NCAND ? chunk0 << pick : INT_MAX;

  // (2) histogram by step count, scanned from the top bin down: thread i
  // owns bins NBIN-1-2i and NBIN-2-2i
  for (int i = tid; i < NBIN; i += PT) sh.bins[i] = 0;
  __syncthreads();
  visit([&](int, int, int s, int) {
    const int nch = chunks_of(s, chunk);
    const int q = s / nch, r = s - q * nch;  // r chunks of q + 1 steps, nch - r of q
    if (r > 0) atomicAdd(&sh.bins[min(q + 1, NBIN - 1)], r);
    atomicAdd(&sh.bins[min(q, NBIN - 1)], nch - r);
  });
  __syncthreads();
  const int hiB = NBIN - 1 - 2 * tid, loB = hiB - 1;
  const int c_hi = sh.bins[hiB], c_lo = sh.bins[loB];
  int excl;
  const int n_units = block_scan(c_hi + c_lo, sh.wsum, excl);
  sh.bins[hiB] = excl;
  sh.bins[loB] = excl + c_hi;
  if (tid == 0) { sh.slot_ctr = 0; sh.split_ctr = 0; }
  __syncthreads();

  // (3) place
  visit([&](int b, int t, int s, int qs) {
    const int nch = chunks_of(s, chunk);
    const int4 bd = make_int4(sh.st[qs], sh.st[qs] + sh.lt[qs], sh.so[qs], sh.so[qs] + sh.lo[qs]);
    int sp = -1, sb = -1;
    if (nch > 1) {
      sp = atomicAdd(&sh.split_ctr, 1);
      sb = atomicAdd(&sh.slot_ctr, nch);
      if (sp < p.split_cap) {
        p.plan.splits[sp] = make_int4(b, t, sb, nch);
        for (int h = 0; h < p.heads; ++h) p.plan.left[sp * p.heads + h] = nch;
      }
    }
    const int q = s / nch, r = s - q * nch;
    int pos_hi = r > 0 ? atomicAdd(&sh.bins[min(q + 1, NBIN - 1)], r) : 0;
    int pos_lo = atomicAdd(&sh.bins[min(q, NBIN - 1)], nch - r);
    for (int c = 0; c < nch; ++c) {
      int n0, n1;
      chunk_range(q, r, c, n0, n1);
      const int pos = c < r ? pos_hi++ : pos_lo++;
      if (pos < p.unit_cap) {
        p.plan.units[pos] = make_int4(b, t, n0, n1);
        p.plan.bounds[pos] = bd;
        p.plan.slots[pos] = nch > 1 ? sb + c : -1;
        p.plan.sidx[pos] = sp;
      }
    }
  });
  __syncthreads();
  if (tid == 0) {
    p.plan.hdr[0] = 0;
    p.plan.hdr[1] = min(n_units, p.unit_cap);
    p.plan.hdr[2] = min(sh.split_ctr, p.split_cap);
  }
}

}  // namespace plan
}  // namespace va
