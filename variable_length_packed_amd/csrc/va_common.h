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

// acc + lo + hi of a packed bf16 pair (one v_dot2 against (1, 1)).
__device__ __forceinline__ float add_bf16x2(uint32_t pair, float acc) {
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair),
                                         __builtin_bit_cast(bf16x2_t, 0x3F803F80u), acc, false);
}

__device__ __forceinline__ float bf16_to_f32(uint16_t x) {
  return __builtin_bit_cast(float, (uint32_t)x << 16);
}

// ---------------------------------------------------------------------------
// 16-bit element kinds.  Kernels take H16 = 0 (float32), 1 (bfloat16) or
// 2 (float16); every 16-bit-path helper below picks the instruction of its
// kind.  Both kinds share one storage layout (16 bits per element) and one
// MFMA operand layout (v_mfma_f32_32x32x16_bf16 / _f16).
// ---------------------------------------------------------------------------
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

template <int H16>
__device__ __forceinline__ f32x16_t mfma16(u32x4_t a, u32x4_t b, f32x16_t c) {
  if constexpr (H16 == 2)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return mfma32_bf16(a, b, c);
}

// Two floats to two 16-bit values (round to nearest even), low half = lo.
template <int H16>
__device__ __forceinline__ uint32_t pack16(float lo, float hi) {
  if constexpr (H16 == 2)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){lo, hi}, f16x2_t));
  else
    return pack_bf16x2(lo, hi);
}

// acc + lo + hi of a packed pair.
template <int H16>
__device__ __forceinline__ float sum16(uint32_t pair, float acc) {
  if constexpr (H16 == 2)
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2_t, pair), __builtin_bit_cast(f16x2_t, 0x3C003C00u),
                                  acc, false);
  else
    return add_bf16x2(pair, acc);
}

// The value in the low / high 16 bits of a word.
template <int H16>
__device__ __forceinline__ float lo16(uint32_t x) {
  if constexpr (H16 == 2) return (float)__builtin_bit_cast(_Float16, (uint16_t)(x & 0xFFFFu));
  else return __uint_as_float(x << 16);
}
template <int H16>
__device__ __forceinline__ float hi16(uint32_t x) {
  if constexpr (H16 == 2) return (float)__builtin_bit_cast(_Float16, (uint16_t)(x >> 16));
  else return __uint_as_float(x & 0xFFFF0000u);
}

// The same at run time, for kernels that serve both kinds (merges).
__device__ __forceinline__ uint32_t pack16_rt(float lo, float hi, int h16) {
  return h16 == 2 ? pack16<2>(lo, hi) : pack16<1>(lo, hi);
}

// Raw buffer resources: loads past `bytes` (or at a negative offset, seen as
// a huge unsigned one) return zero and stores there are dropped, so ragged
// tiles need no branches.  Word 3 = 0x00020000: 32-bit data format, the
// setting for raw (unstructured) buffers on CDNA.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// s_waitcnt operand (gfx9 encoding) that waits for every vector memory load,
// LDS-direct buffer loads included, and leaves the other counters alone:
// vmcnt = 0 (bits 3:0 and 15:14), expcnt = 7 (bits 6:4), lgkmcnt = 15 (bits 11:8)
constexpr int kWaitVm0 = 0x0F70;

// A workgroup barrier that orders LDS accesses only.  Unlike __syncthreads it
// does not wait for the global loads and stores in flight (the next block's
// prefetch, the plan entries of the next item, the output stores of the item
// before).  LDS-direct buffer loads count as global loads: a barrier that
// publishes their data is preceded by an explicit wait (kWaitVm0).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

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
__device__ __forceinline__ void buf_store2(uint16_t v, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b16(v, r, byte_off, 0, 0);
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

// Transposing LDS read of 16-bit data (ds_read_b64_tr_b16).  In each group of
// 16 lanes, lane s gives the address of 4 consecutive elements; lane i of the
// group receives, in slot j, element i % 4 of lane 4j + i / 4.  So if lane s
// points at row s / 4, columns 4(s % 4) .. +4 of a 4 x 16 tile, lane i gets
// column i of the tile's 4 rows: a 16 x 4 transpose per group.
__device__ __forceinline__ u32x2_t lds_read_tr16(const void* p) {
  typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)p));
}

// 16-bit MFMA operand holding, in lane l, 8 values of column c0 + l % 32 of a
// row-major LDS tile (rows `pitch` elements apart): rows 16 kc + {4hh .. 4hh+3,
// 8+4hh .. 8+4hh+3} (hh = l / 32) -- the k-slots a score tile's registers give
// a 16-row chunk kc.  Two transposing reads of 4 rows each: in each group of
// 16 lanes, lane s points at row s / 4 of the four, columns 4 (s % 4) .. +4 of
// the group's 16.  The pitch must keep rows 8-byte aligned.
__device__ __forceinline__ u32x4_t tr_frag(const uint16_t* tile, int pitch, int kc, int c0) {
  const int lane = threadIdx.x & 63;
  const uint16_t* p = tile + (16 * kc + 4 * (lane >> 5) + ((lane >> 2) & 3)) * pitch + c0 + 16 * ((lane >> 4) & 1) +
                      4 * (lane & 3);
  const u32x2_t lo = lds_read_tr16(p), hi = lds_read_tr16(p + 8 * pitch);
  return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
}

// Tiles staged straight from memory into LDS (buffer loads with an LDS
// destination write each wave's 64 x 16 bytes contiguously) keep their rows
// unpadded: row r of D 16-bit elements holds its 16-byte piece p in slot
// p ^ swz_key(r).  The LDS has 64 four-byte banks, so a 128-byte row (D = 64)
// covers half of them (odd rows the other half) and a 256-byte row (D = 128)
// all of them.  The key keeps both read patterns free of bank conflicts:
//  - 16-byte row reads (16 lanes at a time: rows r0 .. r0+15, one piece):
//    the key is a bijection over the rows that share a bank half;
//  - transposing 8-byte reads (32 lanes at a time: rows r0 .. r0+3, r0 a
//    multiple of 4, pieces 4m .. 4m+3): rows of one bank half land in
//    different aligned groups of four slots.
template <int D>
__device__ __forceinline__ int swz_key(int r) {
  static_assert(D == 64 || D == 128, "swizzled tiles have 8 or 16 pieces per row");
  if constexpr (D == 64) return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  else return ((r & 3) << 2) | ((r >> 2) & 3);
}
// Element offset of (row r, column col), col a multiple of 4.
template <int D>
__device__ __forceinline__ int swz(int r, int col) {
  return r * D + (((col >> 3) ^ swz_key<D>(r)) << 3) + (col & 7);
}
// tr_frag of such a tile (rows 16 kc + ..., columns c0 + l % 32).
template <int D>
__device__ __forceinline__ u32x4_t tr_frag_swz(const uint16_t* tile, int kc, int c0) {
  const int lane = threadIdx.x & 63;
  const int row = 16 * kc + 4 * (lane >> 5) + ((lane >> 2) & 3);
  const int col = c0 + 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
  const u32x2_t lo = lds_read_tr16(tile + swz<D>(row, col)), hi = lds_read_tr16(tile + swz<D>(row + 8, col));
  return (u32x4_t){lo[0], lo[1], hi[0], hi[1]};
}

// One lane's 16 (or 4) bytes from global memory straight into LDS (a buffer
// load with an LDS destination; the lanes of the wave that run it write
// consecutive pieces from `lds`).  Counts as a vector memory load.
__device__ __forceinline__ void lds_load_direct16(const void* src, void* lds) {
  const rsrc_t r = make_rsrc(src, 16);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, 0, 0, 0, 0);
}
__device__ __forceinline__ void lds_load_direct4(const void* src, void* lds) {
  const rsrc_t r = make_rsrc(src, 4);
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, 0, 0, 0, 0);
}
// The same from a resource over a whole array (kernel-argument base, so the
// resource sits in scalar registers) at byte offset off.
__device__ __forceinline__ void lds_load_direct16_at(rsrc_t r, int off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, off, 0, 0, 0);
}
__device__ __forceinline__ void lds_load_direct4_at(rsrc_t r, int off, void* lds) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 4, off, 0, 0, 0);
}

// s_waitcnt operand that waits until at most n vector memory operations of
// the wave are outstanding (n < 64), other counters untouched.
constexpr int wait_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }

// Partial results of split tiles are written by one workgroup and merged by
// another, possibly on another XCD (each XCD has its own L2).  They are
// written and read with device-coherent accesses (cache policy sc1, as for
// agent-scope atomics: past the per-CU cache, coherent across the L2s), so
// handing them over needs no writeback or invalidation of whole caches.
constexpr int kDevCoherent = 16;  // buffer cache-policy bit sc1
__device__ __forceinline__ void buf_store16_dev(u32x4_t v, rsrc_t r, int byte_off) {
  __builtin_amdgcn_raw_buffer_store_b128(v, r, byte_off, 0, kDevCoherent);
}
__device__ __forceinline__ f32x4_t buf_load16_dev(rsrc_t r, int byte_off) {
  const u32x4_t u = __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, kDevCoherent);
  return (f32x4_t){__uint_as_float(u[0]), __uint_as_float(u[1]), __uint_as_float(u[2]), __uint_as_float(u[3])};
}
__device__ __forceinline__ u32x4_t as_u32x4(f32x4_t v) {
  return (u32x4_t){__float_as_uint(v[0]), __float_as_uint(v[1]), __float_as_uint(v[2]), __float_as_uint(v[3])};
}
__device__ __forceinline__ void st_dev(float* p, float x) {
  __hip_atomic_store(p, x, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_dev(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Called by a whole workgroup when a chunk of a split tile has stored its
// partial results (device-coherent); `left` counts the tile's chunks still
// running (the planner sets it to the chunk count).  True, in every thread,
// for the chunk that finishes last, which then merges the tile's chunks in
// chunk order, so the result does not depend on which chunk that
// is.  Every thread waits for its stores to complete before the count goes
// down, so the last chunk, which reads (device-coherent) after it, sees them
// all.  Nothing waits on another workgroup.
__device__ __forceinline__ bool split_done_last(int* left, int* s_flag) {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    *s_flag = __hip_atomic_fetch_add(left, -1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 1;
  __syncthreads();
  return *s_flag != 0;
}

// ---------------------------------------------------------------------------
// Work assignment.  A planner kernel writes, per pass, the list of work units
// sorted by cost (heaviest first) and zeroes the list's cursor (hdr[0]).  The
// pass's persistent workgroups start with item w = blockIdx.x; every later
// item is taken from the cursor: a workgroup takes its ticket at the start of
// the second-to-last step of its current item and loads the ticket's plan
// entries during the last, so the workgroups that finish first take the next
// (heaviest remaining) items and neither round trip delays a step.  Results
// never depend on which workgroup ran an item.
// ---------------------------------------------------------------------------

// A work item and its unit's plan entries.  Thread 0 loads the entries of
// the next item while the current item computes and publishes them in LDS
// (double-buffered by item parity) before the current item's output stores,
// so an item starts without a dependent chain of global loads.
// The entries of a work item as the kernels keep them in LDS (ints, 16-byte
// aligned groups): [0] the item, [4..7] its unit {sequence, tile, first step,
// end step}, [8..11] the sequence's rows {tiled start, end, other start, end},
// [12] partial slot, [13] split index.
constexpr int kInfItem = 0, kInfUnit = 4, kInfRows = 8, kInfSlot = 12, kInfSplit = 13;
constexpr int kItemInts = 16;
struct ItemInfo {
  int v[kItemInts];
};
template <typename PlanT>
__device__ __forceinline__ ItemInfo item_load(const PlanT& pl, int item, int per_unit, int total_items) {
  ItemInfo r;
  r.v[kInfItem] = item;
  if (item < total_items) {
    const int unit = item / per_unit;
    const int4 un = pl.units[unit], bd = pl.bounds[unit];
    r.v[kInfUnit + 0] = un.x; r.v[kInfUnit + 1] = un.y; r.v[kInfUnit + 2] = un.z; r.v[kInfUnit + 3] = un.w;
    r.v[kInfRows + 0] = bd.x; r.v[kInfRows + 1] = bd.y; r.v[kInfRows + 2] = bd.z; r.v[kInfRows + 3] = bd.w;
    r.v[kInfSlot] = pl.slots[unit];
    r.v[kInfSplit] = pl.sidx[unit];
  }
  return r;
}
__device__ __forceinline__ void item_store(int* dst, const ItemInfo& r) {
#pragma unroll
  for (int i = 0; i < kItemInts; ++i) dst[i] = r.v[i];
}

// The next item of a workgroup, taken by thread 0: at(n, steps) is called
// before step n of the current item's `steps`; it takes the ticket at
// n >= steps - 2 and at n >= steps - 1 loads the item's plan entries
// straight into the LDS entries `dst` (buffer loads with an LDS destination,
// so no registers hold them across the steps).  finish(steps), after the
// steps, waits for those loads; the item's closing barrier publishes them.
// Items are numbered gridDim.x + ticket.
template <typename PlanT>
struct NextItem {
  const PlanT& pl;
  int per_unit, total_items;
  int* dst;
  int ticket = 0;
  bool asked = false, have = false;
  __device__ __forceinline__ void at(int n, int steps) {
    if (threadIdx.x != 0) return;
    if (!asked && n >= steps - 2) {
      ticket = __hip_atomic_fetch_add(&pl.hdr[0], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      asked = true;
    }
    if (asked && !have && n >= steps - 1) {
      const int item = (int)gridDim.x + ticket;
      dst[kInfItem] = item;
      if (item < total_items) {
        const int unit = item / per_unit, units = total_items / per_unit;
        lds_load_direct16_at(make_rsrc(pl.units, (int64_t)units * 16), unit * 16, dst + kInfUnit);
        lds_load_direct16_at(make_rsrc(pl.bounds, (int64_t)units * 16), unit * 16, dst + kInfRows);
        lds_load_direct4_at(make_rsrc(pl.slots, (int64_t)units * 4), unit * 4, dst + kInfSlot);
        lds_load_direct4_at(make_rsrc(pl.sidx, (int64_t)units * 4), unit * 4, dst + kInfSplit);
      }
      have = true;
    }
  }
  __device__ __forceinline__ void finish(int steps) {
    at(steps, steps);
    if ((threadIdx.x >> 6) == 0) __builtin_amdgcn_s_waitcnt(kWaitVm0);  // thread 0's wave
  }
};

}  // namespace va
