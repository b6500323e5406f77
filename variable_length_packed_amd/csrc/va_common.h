// Device helpers shared by the forward and backward kernels of the packed
// varlen attention library (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace va {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kWave = 64;

// D(32x32, f32) += A(32x16, bf16) * B(16x32, bf16).
// Lane l holds A[l % 32][8*(l/32) .. +8] and B[8*(l/32) .. +8][l % 32];
// result register i of lane l is D[8*(i/4) + 4*(l/32) + i%4][l % 32].
__device__ __forceinline__ f32x16_t mfma32_bf16(u32x4_t a, u32x4_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// D(32x32, f32) += A(32x2, f32) * B(2x32, f32).  Lane l holds A[l%32][l/32]
// and B[l/32][l%32]; result layout as above.
__device__ __forceinline__ f32x16_t mfma32_f32(float a, float b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// Two floats to two bf16 (round to nearest even), low half = lo.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2_t r = __builtin_convertvector((f32x2_t){lo, hi}, bf16x2_t);
  return __builtin_bit_cast(uint32_t, r);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// Raw buffer resources: loads past `bytes` (or at a negative offset, seen as
// a huge unsigned one) return zero and stores there are dropped, so ragged
// tiles need no branches.  Word 3 = 0x00020000: 32-bit data format, the
// setting for raw (unstructured) buffers on CDNA.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int n = bytes <= 0 ? 0 : (bytes >= 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, n, 0x00020000);
}
__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 0);
}
__device__ __forceinline__ u32x2_t buf_load8(rsrc_t r, int byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store16(u32x4_t v, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store8(u32x2_t v, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b64(v, r, byte_off, 0, 0);
}
__device__ __forceinline__ void buf_store4(uint32_t v, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b32(v, r, byte_off, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Value of the same register in lane l ^ 32 (v_permlane32_swap: a VALU op,
// no LDS round trip).  For lanes < 32 the partner's value is the second
// result, for lanes >= 32 the first.
__device__ __forceinline__ float xor32(float x) {
  const uint32_t u = __float_as_uint(x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __uint_as_float((threadIdx.x & 32) ? r[0] : r[1]);
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

__device__ __forceinline__ float max3f(float a, float b, float c) { return fmaxf(fmaxf(a, b), c); }

// Clamped sequence bounds: [s, e) inside [0, total).  Bad metadata can
// never produce an index outside the buffers.
__device__ __forceinline__ void seq_bounds(const int32_t* cu, int b, int total, int& s, int& e) {
  int a = cu[b], z = cu[b + 1];
  a = min(max(a, 0), total);
  z = min(max(z, a), total);
  s = a;
  e = z;
}

// ---------------------------------------------------------------------------
// Tile schedule over (sequence, q-tile, head), built on the device from
// cu_seqlens so no padded tile is computed and the host never reads device
// memory.  Tiles are end-aligned: tile t of sequence b covers query rows
// [Lq - (t+1)*BM, Lq - t*BM) (rows < 0 are absent), so the ragged tile holds
// the first rows, which see the fewest keys under a bottom-right causal mask.
// Tiles are ordered heaviest first: level t = 0 (the last rows of every
// sequence) first, then t = 1, ...; within a level by sequence.  With
// `stride` > 1, a level groups `stride` consecutive t of a sequence.  The
// work item index is tile * heads + head (heads fastest, so the query heads
// that share a KV head run together and share its K/V in L2).
// ---------------------------------------------------------------------------
constexpr int kMaxLevels = 512;
// Per-sequence tile counts cached in LDS when the batch fits (uint16 each).
constexpr int kMaxSeqCached = 2048;

struct SchedShared {
  int level_start[kMaxLevels + 1];
  int full[kMaxLevels + 1];
  int part[kMaxLevels + 1];
  uint16_t ntiles[kMaxSeqCached];
  int total_tiles;
};

__device__ __forceinline__ int seq_tiles(int len, int bm, int tcap) {
  int n = (len + bm - 1) / bm;
  return min(n, tcap);
}

// Called once per workgroup by all threads.
__device__ inline void sched_build(SchedShared& s, const int32_t* cu, int batch, int total,
                                   int bm, int tcap, int stride, int nlev) {
  const int tid = threadIdx.x;
  for (int i = tid; i <= nlev; i += blockDim.x) {
    s.full[i] = 0;
    s.part[i] = 0;
  }
  __syncthreads();
  for (int b = tid; b < batch; b += blockDim.x) {
    int q0, q1;
    seq_bounds(cu, b, total, q0, q1);
    const int n = seq_tiles(q1 - q0, bm, tcap);
    if (b < kMaxSeqCached) s.ntiles[b] = (uint16_t)min(n, 65535);
    const int f = n / stride, rem = n - f * stride;
    if (f > 0) atomicAdd(&s.full[f - 1], 1);
    if (rem > 0) atomicAdd(&s.part[f], rem);
  }
  __syncthreads();
  if (tid == 0) {
    // C(level) = stride * #{b : full levels of b > level} + partial(level)
    int above = 0;
    for (int l = nlev - 1; l >= 0; --l) {
      above += s.full[l];
      s.full[l] = above;  // now #{b : f_b > l}
    }
    int acc = 0;
    for (int l = 0; l < nlev; ++l) {
      s.level_start[l] = acc;
      acc += stride * s.full[l] + s.part[l];
    }
    s.level_start[nlev] = acc;
    s.total_tiles = acc;
  }
  __syncthreads();
}

__device__ __forceinline__ int sched_ntiles(const SchedShared& s, const int32_t* cu, int b,
                                            int total, int bm, int tcap) {
  if (b < kMaxSeqCached) return s.ntiles[b];
  int q0, q1;
  seq_bounds(cu, b, total, q0, q1);
  return seq_tiles(q1 - q0, bm, tcap);
}

// Maps a tile index to (sequence b, tile t).  Every wave decodes on its own
// (no barrier, nothing written): within level `lev` the tiles are ordered by
// sequence, so b is found by counting, 64 sequences per step, the sequences
// that own tiles in that level.
__device__ inline void sched_find(const SchedShared& s, const int32_t* cu, int batch, int total,
                                  int bm, int tcap, int stride, int nlev, int tile, int& b_out,
                                  int& t_out) {
  const int lane = threadIdx.x & 63;
  int lo = 0, hi = nlev - 1;  // largest lev with level_start[lev] <= tile
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (s.level_start[mid] <= tile) lo = mid; else hi = mid - 1;
  }
  const int lev = lo;
  const int u = tile - s.level_start[lev];
  const int lo_t = lev * stride;
  int base = 0, fb = 0, ft = lo_t;
  for (int chunk = 0; chunk < batch; chunk += 64) {
    const int b = chunk + lane;
    int c = 0;
    if (b < batch) c = min(max(sched_ntiles(s, cu, b, total, bm, tcap) - lo_t, 0), stride);
    if (stride == 1) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(c > 0);
      const int cnt = __builtin_popcountll(m);
      if (u < base + cnt) {
        // the (u - base)-th set bit of m
        const int excl = __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0));
        const uint64_t hit = __builtin_amdgcn_ballot_w64(c > 0 && excl == u - base);
        fb = chunk + (int)__builtin_ctzll(hit);
        ft = lo_t;
        break;
      }
      base += cnt;
    } else {
      int x = c;  // inclusive scan across the wave
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o, 64);
        if (lane >= o) x += y;
      }
      const int tot = __shfl(x, 63, 64);
      if (u < base + tot) {
        const int excl = base + x - c;
        const uint64_t hit = __builtin_amdgcn_ballot_w64(c > 0 && u >= excl && u < excl + c);
        const int l = (int)__builtin_ctzll(hit);
        fb = chunk + l;
        ft = lo_t + (u - (base + __shfl(x, l, 64) - __shfl(c, l, 64)));
        break;
      }
      base += tot;
    }
  }
  b_out = uniform(fb);
  t_out = uniform(ft);
}

}  // namespace va
