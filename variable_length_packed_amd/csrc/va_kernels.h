// Kernel argument blocks and launchers (host <-> device interface inside the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "va_varlen.h"

namespace va {

// The packed forward (va_varlen_fwd) with the bytes split tiles' partial
// results may take from the workspace as an argument, and the workspace it
// then needs (0 for arguments it would reject).  With bwd_workspace, the
// planner launch also builds the backward's two work plans in it
// (va_varlen_fwd_bwdplan).
va_status varlen_fwd(const void* q, const void* k, const void* v, const int32_t* cu_seqlens_q,
                     const int32_t* cu_seqlens_k, int32_t max_seqlen_q, int32_t max_seqlen_k,
                     float softmax_scale, int causal, const void* bias, const int64_t* bias_stride, void* out,
                     float* lse, const int64_t* qkv_row_stride, void* workspace, size_t workspace_bytes,
                     size_t part_budget, int32_t batch, int32_t total_q, int32_t total_k, int32_t num_heads_q,
                     int32_t num_heads_kv, int32_t head_dim, va_dtype dtype, va_stream stream,
                     void* bwd_workspace = nullptr, size_t bwd_workspace_bytes = 0);
size_t varlen_fwd_need(int32_t batch, int32_t total_q, int32_t total_k, int32_t max_seqlen_q,
                       int32_t max_seqlen_k, int32_t num_heads_q, int32_t num_heads_kv, int32_t head_dim,
                       va_dtype dtype, size_t part_budget);
// Sets the calling thread's va_last_error() text.
void set_error(const char* msg);

// ---------------------------------------------------------------------------
// Work plans.  A pass tiles one side of every sequence (query rows for the
// forward and dQ, key rows for dK/dV) and walks the other side in steps (key
// blocks, or query blocks).  A tile with more steps than `chunk` is split
// into nch = ceil(steps / chunk) units of near-equal step ranges; each unit
// of a split tile writes float32 partial results to its own slot, and the
// unit that finishes last combines the nch slots in chunk order.  The split rule depends only
// on the tile's own sequence, so a sequence's results never depend on the
// rest of the batch.  Units are listed by step count, largest first.
// ---------------------------------------------------------------------------
struct Plan {
  int* hdr;        // [0] work cursor (written 0), [1] units, [2] split tiles
  int4* units;     // [unit_cap] {sequence, tile, first step, end step}
  int4* bounds;    // [unit_cap] the sequence's rows: {tiled start, end, other start, end}
  int* slots;      // [unit_cap] partial slot of a chunk of a split tile, or -1
  int* sidx;       // [unit_cap] index of that split tile in `splits`, or -1
  int4* splits;    // [split_cap] {sequence, tile, first slot, chunks}
  int* left;       // [split_cap][heads] chunks of the split tile still to finish, per item
                   // head (set by the planner)
};

struct PlanArgs {
  Plan plan;
  const int32_t* cu_t;  // cu_seqlens of the tiled side
  const int32_t* cu_o;  // cu_seqlens of the stepped side
  int32_t total_t, total_o, batch;
  int32_t tile;    // rows per tile
  int32_t step;    // rows of the other side per step
  int32_t kside;   // 0: query tiles, end-aligned, steps over keys [0, kv_hi)
                   // 1: key tiles, start-aligned, steps over queries [qs, Lq)
  int32_t causal;
  int32_t chunk;   // most steps per unit
  int32_t unit_cap, slot_cap, split_cap;
  int32_t heads;   // work items (heads) per unit, each counting its chunks in `left`
};

struct PlanSet {
  PlanArgs p[3];
  int32_t nplans;  // plan_dsum_kernel: its first nplans workgroups build p[0 .. nplans)
};

hipError_t launch_plan(const PlanSet& s, int nplans, hipStream_t st);

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const void* bias;  // nullptr = no bias
  int64_t bs0, bs1, bs2, bs3;
  void* out;
  float* lse;
  int64_t q_rs, k_rs, v_rs;  // token strides of q, k, v (elements); out is dense
  Plan plan;
  float* part_o;    // [slot][hq][BM][d]  normalised partial outputs of split tiles
  float* part_lse;  // [slot][hq][BM]     their base-2 log-sum-exp
  int32_t batch, total_q, total_k, hq, hkv, n_rep, d;
  int32_t split_cap;
  float scale_log2;
  int32_t causal;
  int32_t bf16;      // element kind: 0 float32, 1 bfloat16, 2 float16
  int32_t bias_vec;  // keys contiguous (bs3 = 1), 4-key groups aligned: vector bias loads
  int32_t bias_tile;  // 16-bit bias, contiguous keys, 16-byte aligned rows: tiles staged in LDS
};

struct BwdArgs {
  const void* dout;
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const float* lse;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const void* bias;
  int64_t bs0, bs1, bs2, bs3;
  void* dq;
  void* dk;
  void* dv;
  int64_t q_rs, k_rs, v_rs;  // token strides of q, k, v (elements); dout, out and grads dense
  float* dsum;     // workspace [hq, total_q]: rowsum(dO * O)
  Plan plan_k;     // dK/dV pass: key tiles
  Plan plan_q;     // dQ pass: query tiles
  float* part_kv;  // [slot][hkv][2][BNK][d]  dK (unscaled) and dV partial sums
  float* part_q;   // [slot][hq][BMQ][d]      dQ (unscaled) partial sums
  // bias gradient (dbias_mode 0: none; 1: per pair, dS stored at element
  // b*ds0 + h*ds1 + r*ds2 + c*ds3; 2: per key (ds2 = 0), dS summed over rows,
  // and over the heads too when ds1 = 0 (one KV head))
  float* dbias;
  int64_t ds0, ds1, ds2, ds3;
  int32_t dbias_mode;
  float* part_db;  // [slot][hkv][n_rep][BNK]  per-key sums of split key tiles
  int32_t batch, total_q, total_k, hq, hkv, n_rep, d;
  int32_t split_cap_k, split_cap_q;
  float scale;
  float scale_log2;
  int32_t causal;
  int32_t bf16;       // element kind: 0 float32, 1 bfloat16, 2 float16
  int32_t grad_bf16;  // gradients in float32 (0) or in the input's 16-bit kind (its code)
  int32_t bias_vec;  // keys contiguous (bs3 = 1), 4-key groups aligned: vector bias loads
  int32_t bias_tile;  // a bias with contiguous keys and 16-byte aligned rows (per pair or per key):
                      // staged through LDS a tile at a time by the dK/dV pass
};

// Optional per-kernel event timing (see va_timing_start); no-ops when off.
void timing_before(hipStream_t st, const char* name);
void timing_after(hipStream_t st);

// Persistent grids: min(max_items, resident workgroups per device).
int resident_grid(const void* kernel, int threads, int64_t max_items);

// Tile and step sizes of each pass (the planner and the kernels must agree).
int fwd_block_m();
int fwd_block_n(bool bf16, int d);
hipError_t launch_fwd(const FwdArgs& a, int64_t max_items, hipStream_t st);

int bwd_block_q();                   // query rows per dQ tile
int bwd_block_k();                   // key rows per dK/dV tile
int bwd_dq_block_n(bool bf16, int d);  // keys per dQ step
int bwd_dkdv_block_q();              // queries per dK/dV step
// Launches the fused planner + D preprocess (plans ps.p[0] = dK/dV, ps.p[1] = dQ), then the passes.
hipError_t launch_bwd(const BwdArgs& a, const PlanSet& ps, int64_t max_q_items, int64_t max_k_items,
                      hipStream_t st);

// ---------------------------------------------------------------------------
// Decode steps against a paged KV cache.  A work item (one wave) is one
// (sequence, KV head, row block, key chunk): 32 rows = (new token, query
// head of the KV head's group) pairs, keys [chunk * c, chunk * (c + 1)).
// A planner kernel lists the (sequence, row block, chunk) triples that have
// work; items are (list entry, KV head), KV heads fastest.  A row block with
// more than one chunk writes float32 partials to slot entry * hkv + g,
// [slot][rows][d] and [slot][rows], and the merge kernel combines its chunks
// in order.
// ---------------------------------------------------------------------------
struct KvChunk {
  int32_t b, rb, c;      // sequence, 32-row block, key chunk
  int32_t q0, q1;        // the sequence's query rows
  int32_t lk, k0;        // its key count and first key row (ragged mode)
  int32_t chunk;         // keys per chunk of this sequence
};
struct KvArgs {
  const void* q;             // [total_q, hq, d], token stride q_rs
  const void* k_cache;       // paged: [num_pages, page_size, hkv, d]; ragged: [total_k, hkv, d]
  const void* v_cache;
  const int32_t* cu_q;       // [batch + 1]
  const int32_t* seqlens_k;  // paged: [batch]
  const int32_t* block_table;  // paged: [batch][bt_stride]
  const int32_t* cu_k;       // ragged (no table): [batch + 1] rows of k_cache / v_cache
  int64_t q_rs, k_rs, v_rs;  // token strides (elements); out is dense
  int32_t total_k;           // ragged: rows of k_cache / v_cache
  void* out;                 // [total_q, hq, d]
  float* lse;                // [hq, total_q]
  float* part_o;
  float* part_lse;
  int32_t* plan;             // [0] entries in `chunks`, [1] in `merges` (written by the planner)
  KvChunk* chunks;           // [cap]
  int32_t* merges;           // [cap_merge] list entry of chunk 0 of each row block with several chunks
  int32_t batch, total_q, hq, hkv, n_rep, d;
  int32_t bt_stride, page_shift, num_pages;
  int32_t max_k;             // paged: keys of a sequence are capped here (max_seqlen_k and the table's reach)
  int32_t rows;              // partial rows per slot
  int32_t chunk, nchunk;     // keys per chunk (a multiple of the step); most chunks of a row block
  int32_t cap;               // most list entries (and partial slots per KV head)
  int32_t cap_merge;         // most row blocks with several chunks (cap / 2)
  float scale_log2;
  int32_t causal;
  int32_t h16;               // 0 float32, 1 bfloat16, 2 float16
  // additive bias (the packed forward's short-query path only; nullptr otherwise):
  // element (b, h, r, c) at b*bs0 + h*bs1 + r*bs2 + c*bs3, in the input dtype
  const void* bias;
  int64_t bs0, bs1, bs2, bs3;
  int32_t bias_vec;          // bs3 == 1 and every 4-key group aligned: 4 keys per load
};
int kv_block_n(int d);  // keys per step of the decode kernel
hipError_t launch_kvcache(const KvArgs& a, hipStream_t st);

// ---------------------------------------------------------------------------
// Packing: metadata from a padding mask, unpad (gather) and pad (scatter).
// ---------------------------------------------------------------------------
constexpr int kPackMaxTensors = 4;
struct PackArgs {
  void* padded[kPackMaxTensors];  // [padded_rows][row_bytes] each
  void* packed[kPackMaxTensors];  // [packed_rows][row_bytes] each
  int64_t row_bytes[kPackMaxTensors];
  int32_t n;                      // tensors in use
  int32_t batch;
  int64_t padded_rows;            // batch * seqlen
  int64_t packed_rows;            // rows the packed buffers hold
};
hipError_t launch_pack_metadata(const uint8_t* mask, int batch, int seqlen, int32_t* cu, int32_t* max_len,
                                int32_t* indices, int32_t* position_ids, int32_t* inverse, hipStream_t st);
// width: bytes per copy (16, 8, 4, 2 or 1), dividing every row size and base address
hipError_t launch_unpad(const PackArgs& a, int width, const int32_t* indices, const int32_t* cu, hipStream_t st);
hipError_t launch_pad(const PackArgs& a, int width, const int32_t* inverse, hipStream_t st);

}  // namespace va
