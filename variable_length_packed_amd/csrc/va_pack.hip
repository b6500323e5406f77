// Packing metadata from a padding mask, and the gather (unpad) / scatter
// (pad) between the padded [batch, seqlen, ...] layout and the packed
// [total, ...] stream the attention kernels read.  All integer and byte
// work: results are exact.  Contract in include/va_pack.h.
#include "va_common.h"
#include "va_kernels.h"

namespace va {

namespace {

constexpr int PT = 256;  // threads per workgroup (4 waves)

// Sum of x over the workgroup (every thread gets it).
__device__ inline int block_sum(int x, int* red) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o, 64);
  const int wid = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wid] = x;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < PT / 64; ++w) t += red[w];
  return t;
}

// (1) row lengths: cu[b + 1] = number of nonzero mask bytes of row b; cu[0] = 0.
__global__ __launch_bounds__(PT) void pack_count_kernel(const uint8_t* __restrict__ mask, int batch,
                                                         int seqlen, int32_t* __restrict__ cu) {
  __shared__ int red[PT / 64];
  if (blockIdx.x == 0 && threadIdx.x == 0) cu[0] = 0;
  for (int b = blockIdx.x; b < batch; b += gridDim.x) {
    const uint8_t* row = mask + (size_t)b * seqlen;
    int n = 0;
    for (int s = threadIdx.x; s < seqlen; s += PT) n += row[s] != 0;
    n = block_sum(n, red);
    if (threadIdx.x == 0) cu[b + 1] = n;
  }
}

// (2) one workgroup: cu[1..batch] from lengths to running sums (in place, in
// chunks of PT with a carry), and the largest length.
__global__ __launch_bounds__(PT) void pack_scan_kernel(int batch, int32_t* __restrict__ cu,
                                                        int32_t* __restrict__ max_len) {
  __shared__ int wsum[PT / 64];
  __shared__ int wmax[PT / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  int carry = 0, mx = 0;
  for (int c0 = 0; c0 < batch; c0 += PT) {
    const int i = c0 + threadIdx.x;
    const int x = i < batch ? cu[i + 1] : 0;
    mx = max(mx, x);
    int incl = x;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(incl, o, 64);
      if (lane >= o) incl += y;
    }
    if (lane == 63) wsum[wid] = incl;
    __syncthreads();
    int before = 0, total = 0;
#pragma unroll
    for (int w = 0; w < PT / 64; ++w) {
      if (w < wid) before += wsum[w];
      total += wsum[w];
    }
    if (i < batch) cu[i + 1] = carry + before + incl;
    carry += total;
    __syncthreads();
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) mx = max(mx, __shfl_xor(mx, o, 64));
  if (lane == 0) wmax[wid] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    int m = 0;
#pragma unroll
    for (int w = 0; w < PT / 64; ++w) m = max(m, wmax[w]);
    *max_len = m;
  }
}

// (3) per row: the rank of every real token inside its row (ballot + lane
// count, wave totals through LDS, a running base per chunk of PT positions)
// gives its packed index cu[b] + rank.
__global__ __launch_bounds__(PT) void pack_index_kernel(const uint8_t* __restrict__ mask, int batch,
                                                         int seqlen, const int32_t* __restrict__ cu,
                                                         int32_t* __restrict__ indices,
                                                         int32_t* __restrict__ position_ids,
                                                         int32_t* __restrict__ inverse) {
  __shared__ int wcnt[PT / 64];
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  for (int b = blockIdx.x; b < batch; b += gridDim.x) {
    const uint8_t* row = mask + (size_t)b * seqlen;
    const int start = cu[b];
    int base = 0;
    for (int c0 = 0; c0 < seqlen; c0 += PT) {
      const int s = c0 + threadIdx.x;
      const bool keep = s < seqlen && row[s] != 0;
      const uint64_t bal = __builtin_amdgcn_ballot_w64(keep);
      const int in_wave = __builtin_amdgcn_mbcnt_hi((uint32_t)(bal >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)bal, 0));
      if (lane == 0) wcnt[wid] = __builtin_popcountll(bal);
      __syncthreads();
      int before = 0, total = 0;
#pragma unroll
      for (int w = 0; w < PT / 64; ++w) {
        if (w < wid) before += wcnt[w];
        total += wcnt[w];
      }
      if (s < seqlen) {
        const size_t p = (size_t)b * seqlen + s;
        if (keep) {
          const int rank = base + before + in_wave;
          const int t = start + rank;
          indices[t] = (int32_t)p;
          position_ids[t] = rank;
          inverse[p] = t;
        } else {
          inverse[p] = -1;
        }
      }
      base += total;
      __syncthreads();
    }
  }
}

template <int W>
struct Chunk;
template <> struct Chunk<16> { using T = u32x4_t; };
template <> struct Chunk<8> { using T = u32x2_t; };
template <> struct Chunk<4> { using T = uint32_t; };
template <> struct Chunk<2> { using T = uint16_t; };
template <> struct Chunk<1> { using T = uint8_t; };

// Gather: packed row t (< min(total, packed_rows)) of every tensor from padded
// row indices[t] (clamped into the padded buffer).  One wave per row; the
// index is read once for all tensors.
template <int W>
__global__ __launch_bounds__(PT) void unpad_kernel(PackArgs a, const int32_t* __restrict__ indices,
                                                   const int32_t* __restrict__ cu) {
  using C = typename Chunk<W>::T;
  const int lane = threadIdx.x & 63;
  const int64_t rows = a.padded_rows;
  int64_t total = cu[a.batch];
  total = total < 0 ? 0 : total;
  total = total > a.packed_rows ? a.packed_rows : total;
  total = total > rows ? rows : total;  // indices holds padded_rows entries
  const int64_t waves = (int64_t)gridDim.x * (PT / 64);
  for (int64_t t = (int64_t)blockIdx.x * (PT / 64) + (threadIdx.x >> 6); t < total; t += waves) {
    int64_t src = indices[t];
    src = src < 0 ? 0 : (src >= rows ? rows - 1 : src);
#pragma unroll
    for (int i = 0; i < kPackMaxTensors; ++i) {
      if (i >= a.n) break;
      const int64_t n = a.row_bytes[i] / W;
      const C* s = (const C*)((const uint8_t*)a.padded[i] + src * a.row_bytes[i]);
      C* d = (C*)((uint8_t*)a.packed[i] + t * a.row_bytes[i]);
      for (int64_t c = lane; c < n; c += 64) d[c] = s[c];
    }
  }
}

// Scatter: every padded row p gets packed row inverse[p], or zeros where
// inverse[p] is negative or not a row of the packed buffer.
template <int W>
__global__ __launch_bounds__(PT) void pad_kernel(PackArgs a, const int32_t* __restrict__ inverse) {
  using C = typename Chunk<W>::T;
  const int lane = threadIdx.x & 63;
  const int64_t waves = (int64_t)gridDim.x * (PT / 64);
  for (int64_t p = (int64_t)blockIdx.x * (PT / 64) + (threadIdx.x >> 6); p < a.padded_rows; p += waves) {
    const int64_t src = inverse[p];
    const bool real = src >= 0 && src < a.packed_rows;
#pragma unroll
    for (int i = 0; i < kPackMaxTensors; ++i) {
      if (i >= a.n) break;
      const int64_t n = a.row_bytes[i] / W;
      C* d = (C*)((uint8_t*)a.padded[i] + p * a.row_bytes[i]);
      if (real) {
        const C* s = (const C*)((const uint8_t*)a.packed[i] + src * a.row_bytes[i]);
        for (int64_t c = lane; c < n; c += 64) d[c] = s[c];
      } else {
        for (int64_t c = lane; c < n; c += 64) d[c] = C{};
      }
    }
  }
}

int grid_for(int64_t rows) {
  const int64_t g = (rows + PT / 64 - 1) / (PT / 64);
  return (int)(g < 1 ? 1 : (g > 65536 ? 65536 : g));
}

}  // namespace

hipError_t launch_pack_metadata(const uint8_t* mask, int batch, int seqlen, int32_t* cu, int32_t* max_len,
                                int32_t* indices, int32_t* position_ids, int32_t* inverse, hipStream_t st) {
  const int g = batch < 65536 ? batch : 65536;
  timing_before(st, "pack_count");
  hipLaunchKernelGGL(pack_count_kernel, dim3(g), dim3(PT), 0, st, mask, batch, seqlen, cu);
  timing_after(st);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  timing_before(st, "pack_scan");
  hipLaunchKernelGGL(pack_scan_kernel, dim3(1), dim3(PT), 0, st, batch, cu, max_len);
  timing_after(st);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  timing_before(st, "pack_index");
  hipLaunchKernelGGL(pack_index_kernel, dim3(g), dim3(PT), 0, st, mask, batch, seqlen, cu, indices,
                     position_ids, inverse);
  timing_after(st);
  return hipGetLastError();
}

hipError_t launch_unpad(const PackArgs& a, int width, const int32_t* indices, const int32_t* cu, hipStream_t st) {
  const int g = grid_for(a.padded_rows < a.packed_rows ? a.padded_rows : a.packed_rows);
  timing_before(st, "unpad");
  switch (width) {
    case 16: hipLaunchKernelGGL(unpad_kernel<16>, dim3(g), dim3(PT), 0, st, a, indices, cu); break;
    case 8: hipLaunchKernelGGL(unpad_kernel<8>, dim3(g), dim3(PT), 0, st, a, indices, cu); break;
    case 4: hipLaunchKernelGGL(unpad_kernel<4>, dim3(g), dim3(PT), 0, st, a, indices, cu); break;
    case 2: hipLaunchKernelGGL(unpad_kernel<2>, dim3(g), dim3(PT), 0, st, a, indices, cu); break;
    default: hipLaunchKernelGGL(unpad_kernel<1>, dim3(g), dim3(PT), 0, st, a, indices, cu); break;
  }
  timing_after(st);
  return hipGetLastError();
}

hipError_t launch_pad(const PackArgs& a, int width, const int32_t* inverse, hipStream_t st) {
  const int g = grid_for(a.padded_rows);
  timing_before(st, "pad");
  switch (width) {
    case 16: hipLaunchKernelGGL(pad_kernel<16>, dim3(g), dim3(PT), 0, st, a, inverse); break;
    case 8: hipLaunchKernelGGL(pad_kernel<8>, dim3(g), dim3(PT), 0, st, a, inverse); break;
    case 4: hipLaunchKernelGGL(pad_kernel<4>, dim3(g), dim3(PT), 0, st, a, inverse); break;
    case 2: hipLaunchKernelGGL(pad_kernel<2>, dim3(g), dim3(PT), 0, st, a, inverse); break;
    default: hipLaunchKernelGGL(pad_kernel<1>, dim3(g), dim3(PT), 0, st, a, inverse); break;
  }
  timing_after(st);
  return hipGetLastError();
}

}  // namespace va
