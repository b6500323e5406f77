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

// ---------------------------------------------------------------------------
// Work queue.  A planner kernel writes, per pass, a list of work units sorted
// by cost (heaviest first) and zeroes hdr[0]; the pass's persistent
// workgroups then take items in list order, so the heavy units start first
// and the light ones fill in behind them.  Workgroup w starts with item w;
// later items are gridDim.x + a ticket from one device-scope atomic, taken
// by thread 0 one item ahead (a workgroup takes a ticket only while it holds
// a valid item, and tickets grow, so every valid item is run exactly once).
// The atomic's address goes through a register the compiler must treat as
// per-lane: a uniform address would be rewritten into a one-lane atomic plus
// an immediate broadcast, i.e. a wait for the atomic's full round trip (which
// also drains every store still in flight) at the point of the call.  This
// way the wait happens where the ticket is first used.
// ---------------------------------------------------------------------------
__device__ __forceinline__ int queue_take(int* hdr) {  // the ticket; its item is gridDim.x + ticket
  int z;
  asm volatile("v_mov_b32 %0, 0" : "=v"(z));
  return __hip_atomic_fetch_add(hdr + z, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A work item and its unit's plan entries.  Thread 0 loads the entries of
// the next item while the current item computes and publishes them in LDS
// (double-buffered by item parity) before the current item's output stores,
// so an item starts without a dependent chain of global loads.
struct ItemInfo {
  int v[10];  // item, sequence, tile, first step, end step, tiled start/end, other start/end, slot
};
template <typename PlanT>
__device__ __forceinline__ ItemInfo item_load(const PlanT& pl, int item, int per_unit, int total_items) {
  ItemInfo r;
  r.v[0] = item;
  if (item < total_items) {
    const int unit = item / per_unit;
    const int4 un = pl.units[unit], bd = pl.bounds[unit];
    r.v[1] = un.x; r.v[2] = un.y; r.v[3] = un.z; r.v[4] = un.w;
    r.v[5] = bd.x; r.v[6] = bd.y; r.v[7] = bd.z; r.v[8] = bd.w;
    r.v[9] = pl.slots[unit];
  }
  return r;
}
__device__ __forceinline__ void item_store(int* dst, const ItemInfo& r) {
#pragma unroll
  for (int i = 0; i < 10; ++i) dst[i] = r.v[i];
}

}  // namespace va
