// Index branch of MSA, decode: token scores Q_idx . K_idx^T against the single
// shared index-key head, max-pooled per KV block ("Block Max Pool"), following
// "MiniMax wird dünn", section 1, Schritt 1.
//
// One pass over every cached index key of every sequence: the keys are
// streamed from HBM exactly once, one KV block per single-wave workgroup (or,
// for batches whose full grid is mostly empty, a compact grid of workgroups
// walking the real blocks), through LDS (index_block_scores); all Hkv*n_i index-query rows of a
// sequence (32 at 8 groups x 4 heads) are the M side of a
// v_mfma_f32_16x16x32_bf16 so the 64-term dots run on the matrix cores and
// the kernel stays bound by HBM.
#include <algorithm>

#include "index_block.h"
#include "msa_device.h"
#include "msa_launch.h"
#include "timeline_marks.h"

namespace msa {

// ---------------------------------------------------------------- decode
// One wave per workgroup and one block per wave (index_block_scores); small
// single-wave workgroups let ten blocks per CU be in flight.  With an append
// (ap.k_new != nullptr) one extra workgroup per sequence writes the current
// token's key, value and index key into its own block's page, which the
// index branch never reads.
template <int B>
__device__ __forceinline__ void append_current_token(const DecodeAppend& ap, int s, int L,
                                                     int num_kv_heads, int idx_k_heads) {
  const int lane = threadIdx.x;
  const int own = (L - 1) / B, slot = (L - 1) % B;
  const size_t page = (size_t)ap.cache.block_table[(size_t)s * ap.cache.max_blocks + own];
  const size_t kv0 = (size_t)s * num_kv_heads * 128;
  for (int x = lane; x < num_kv_heads * 16; x += kWave) {  // K and V rows, 16-byte chunks
    const int g = x >> 4, c = x & 15;
    const size_t dst = ((page * num_kv_heads + g) * B + slot) * 128 + c * 8;
    *reinterpret_cast<u32x4*>(ap.cache.k + dst) =
        *reinterpret_cast<const u32x4*>(ap.k_new + kv0 + g * 128 + c * 8);
    *reinterpret_cast<u32x4*>(ap.cache.v + dst) =
        *reinterpret_cast<const u32x4*>(ap.v_new + kv0 + g * 128 + c * 8);
  }
  for (int x = lane; x < idx_k_heads * 8; x += kWave) {  // index-key rows, 16-byte chunks
    const int h = x >> 3, c = x & 7;
    *reinterpret_cast<u32x4*>(ap.cache.idx_k + ((page * idx_k_heads + h) * B + slot) * 64 + c * 8) =
        *reinterpret_cast<const u32x4*>(ap.idx_new + ((size_t)s * idx_k_heads + h) * 64 + c * 8);
  }
}

// PG: per-group index keys; workgroup (x, s, g) scores group g's n_i rows
// against its own key head of the block (grid z = Hkv).
template <int B, int NI, int MT, bool PG>
__global__ __launch_bounds__(64) void index_score_decode_kernel(
    const uint16_t* __restrict__ idx_k, const int32_t* __restrict__ block_table,
    int32_t max_blocks, const uint16_t* __restrict__ idx_q, const int32_t* __restrict__ seq_lens,
    int32_t num_kv_heads, int32_t idx_k_heads, float* __restrict__ pooled,
    uint32_t* __restrict__ counters, DecodeAppend ap) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[B * 128];
  const int s = blockIdx.y, gz = blockIdx.z;
  const int lane = threadIdx.x;
  if (counters != nullptr && blockIdx.x == 0 && gz == 0 && lane < num_kv_heads)
    counters[s * num_kv_heads + lane] = 0u;
  // with an append, workgroup 0 (dispatched first, so its latency hides
  // behind the scoring) writes the current token and block b is scored by
  // workgroup b + 1
  int b = blockIdx.x;
  if (ap.k_new != nullptr) {
    if (b == 0) {
      if (gz == 0) append_current_token<B>(ap, s, seq_lens[s], num_kv_heads, idx_k_heads);
      return;
    }
    --b;
  }
  // the page id is read together with the length (one round trip): every
  // launched b is below (max_seq_len - 1) / B < max_blocks, so the entry
  // exists; the exit test reads both, which keeps the two loads side by side
  // (a negative page id, outside the contract, is never dereferenced)
  const int32_t page = block_table[(size_t)s * max_blocks + b];
  const int L = seq_lens[s];
  const int own = (L - 1) / B;
  if (b >= own || page < 0) return;
  float* out = pooled + (size_t)s * num_kv_heads * max_blocks + b;
  if constexpr (PG) {
    index_block_scores<B, NI, 1>(idx_k, page * idx_k_heads + gz,
                                 idx_q + ((size_t)s * num_kv_heads + gz) * NI * 64, 1, stage,
                                 [&](int, float v) { out[(size_t)gz * max_blocks] = v; });
  } else {
    index_block_scores<B, NI, MT>(idx_k, page, idx_q + (size_t)s * num_kv_heads * NI * 64,
                                  num_kv_heads, stage,
                                  [&](int g, float v) { out[(size_t)g * max_blocks] = v; });
  }
  MSA_MARK_LATEST(MSA_MARK_INDEX_END);
}

// Batches whose full (block, sequence) grid is mostly empty (lengths far
// below the longest): a compact grid of resident single-wave workgroups walks
// the real items only.  Item order: per sequence, its append item (with an
// append) and then its blocks 0 .. own-1; each workgroup finds the sequence of
// an item from an in-wave scan of the lengths (batch <= 64) and prefetches the
// page id of its next item while it scores the current one.
template <int B, int NI, int MT>
__global__ __launch_bounds__(64) void index_score_decode_compact_kernel(
    const uint16_t* __restrict__ idx_k, const int32_t* __restrict__ block_table,
    int32_t max_blocks, const uint16_t* __restrict__ idx_q, const int32_t* __restrict__ seq_lens,
    int32_t batch, int32_t num_kv_heads, int32_t idx_k_heads, float* __restrict__ pooled,
    uint32_t* __restrict__ counters, DecodeAppend ap) {
  __shared__ __attribute__((aligned(16))) uint8_t stage[B * 128];
  const int lane = threadIdx.x;
  if (counters != nullptr && blockIdx.x == 0)
    for (int x = lane; x < batch * num_kv_heads; x += kWave) counters[x] = 0u;
  const int n_app = ap.k_new != nullptr ? 1 : 0;
  const int L = lane < batch ? seq_lens[lane] : 1;
  const int items = lane < batch ? (L - 1) / B + n_app : 0;
  int incl = items;  // inclusive scan over the sequences
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const int t = __shfl_up(incl, d, kWave);
    if (lane >= d) incl += t;
  }
  const int excl = incl - items;
  const int total = __builtin_amdgcn_readlane(incl, kWave - 1);
  // (sequence, item index within it) of item w: the last sequence whose
  // first item is at or before w
  auto locate = [&](int w, int& s, int& i) {
    const uint64_t m = __ballot(lane < batch && excl <= w);
    s = 63 - __builtin_clzll(m);
    i = w - __builtin_amdgcn_readlane(excl, s);
  };
  auto page_of = [&](int s, int i) {
    return i >= n_app ? block_table[(size_t)s * max_blocks + (i - n_app)] : 0;
  };
  int w = blockIdx.x;
  if (w >= total) return;
  int s, i;
  locate(w, s, i);
  int32_t page = page_of(s, i);
  for (;;) {
    const int wn = w + (int)gridDim.x;
    int sn = 0, in = 0;
    int32_t page_n = 0;
    if (wn < total) {  // next item's page id, in flight while this item runs
      locate(wn, sn, in);
      page_n = page_of(sn, in);
    }
    if (i < n_app) {
      append_current_token<B>(ap, s, __builtin_amdgcn_readlane(L, s), num_kv_heads, idx_k_heads);
    } else if (page >= 0) {
      const int b = i - n_app;
      float* out = pooled + (size_t)s * num_kv_heads * max_blocks + b;
      index_block_scores<B, NI, MT>(idx_k, __builtin_amdgcn_readfirstlane(page),
                                    idx_q + (size_t)s * num_kv_heads * NI * 64, num_kv_heads,
                                    stage, [&](int g, float v) { out[(size_t)g * max_blocks] = v; });
    }
    if (wn >= total) break;
    w = wn;
    s = sn;
    i = in;
    page = page_n;
  }
  MSA_MARK_LATEST(MSA_MARK_INDEX_END);
}

template <int B, int NI>
static hipError_t launch_decode_ni(int mt, bool pg, dim3 grid, hipStream_t st,
                                   const uint16_t* idx_k, const int32_t* bt, int32_t mb,
                                   const uint16_t* idx_q, const int32_t* sl, int32_t hkv,
                                   int32_t hk, float* pooled, uint32_t* ctr,
                                   const DecodeAppend& ap) {
#define MSA_IDX_ARGS idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap
  if (pg) {
    hipLaunchKernelGGL((index_score_decode_kernel<B, NI, 1, true>), grid, dim3(64), 0, st, MSA_IDX_ARGS);
    return hipGetLastError();
  }
  switch (mt) {
    case 1: hipLaunchKernelGGL((index_score_decode_kernel<B, NI, 1, false>), grid, dim3(64), 0, st, MSA_IDX_ARGS); break;
    case 2: hipLaunchKernelGGL((index_score_decode_kernel<B, NI, 2, false>), grid, dim3(64), 0, st, MSA_IDX_ARGS); break;
    case 3: hipLaunchKernelGGL((index_score_decode_kernel<B, NI, 3, false>), grid, dim3(64), 0, st, MSA_IDX_ARGS); break;
    default: hipLaunchKernelGGL((index_score_decode_kernel<B, NI, 4, false>), grid, dim3(64), 0, st, MSA_IDX_ARGS); break;
  }
#undef MSA_IDX_ARGS
  return hipGetLastError();
}

template <int B, int NI>
static hipError_t launch_compact_ni(int mt, int wgs, hipStream_t st, const uint16_t* idx_k,
                                   const int32_t* bt, int32_t mb, const uint16_t* idx_q,
                                   const int32_t* sl, int32_t batch, int32_t hkv, int32_t hk,
                                   float* pooled, uint32_t* ctr, const DecodeAppend& ap) {
#define MSA_IDX_ARGS idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap
  switch (mt) {
    case 1: hipLaunchKernelGGL((index_score_decode_compact_kernel<B, NI, 1>), dim3(wgs), dim3(64), 0, st, MSA_IDX_ARGS); break;
    case 2: hipLaunchKernelGGL((index_score_decode_compact_kernel<B, NI, 2>), dim3(wgs), dim3(64), 0, st, MSA_IDX_ARGS); break;
    case 3: hipLaunchKernelGGL((index_score_decode_compact_kernel<B, NI, 3>), dim3(wgs), dim3(64), 0, st, MSA_IDX_ARGS); break;
    default: hipLaunchKernelGGL((index_score_decode_compact_kernel<B, NI, 4>), dim3(wgs), dim3(64), 0, st, MSA_IDX_ARGS); break;
  }
#undef MSA_IDX_ARGS
  return hipGetLastError();
}

template <int B>
static hipError_t launch_compact_b(int ni, int mt, int wgs, hipStream_t st, const uint16_t* idx_k,
                                   const int32_t* bt, int32_t mb, const uint16_t* idx_q,
                                   const int32_t* sl, int32_t batch, int32_t hkv, int32_t hk,
                                   float* pooled, uint32_t* ctr, const DecodeAppend& ap) {
  switch (ni) {
    case 1: return launch_compact_ni<B, 1>(mt, wgs, st, idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap);
    case 2: return launch_compact_ni<B, 2>(mt, wgs, st, idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap);
    case 4: return launch_compact_ni<B, 4>(mt, wgs, st, idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap);
    case 8: return launch_compact_ni<B, 8>(mt, wgs, st, idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap);
    default: return launch_compact_ni<B, 16>(mt, wgs, st, idx_k, bt, mb, idx_q, sl, batch, hkv, hk, pooled, ctr, ap);
  }
}

template <int B>
static hipError_t launch_decode_b(int ni, int mt, bool pg, dim3 grid, hipStream_t st,
                                  const uint16_t* idx_k, const int32_t* bt, int32_t mb,
                                  const uint16_t* idx_q, const int32_t* sl, int32_t hkv, int32_t hk,
                                  float* pooled, uint32_t* ctr, const DecodeAppend& ap) {
  switch (ni) {
    case 1: return launch_decode_ni<B, 1>(mt, pg, grid, st, idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap);
    case 2: return launch_decode_ni<B, 2>(mt, pg, grid, st, idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap);
    case 4: return launch_decode_ni<B, 4>(mt, pg, grid, st, idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap);
    case 8: return launch_decode_ni<B, 8>(mt, pg, grid, st, idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap);
    default: return launch_decode_ni<B, 16>(mt, pg, grid, st, idx_k, bt, mb, idx_q, sl, hkv, hk, pooled, ctr, ap);
  }
}

// Full grids above this many workgroups take the compact kernel (batches of
// 2..64 sequences); 160 KiB of LDS per CU bounds the resident workgroups.
constexpr size_t kCompactMinGrid = 10240;
constexpr int kLdsPerCu = 160 * 1024;
// Workgroups per resident slot: the dispatcher refills slots as workgroups
// finish, so a few per slot even out the per-item latency (1, 2, 4, 8 per
// slot on the 32-sequence paged batch: 133, 124.5, 123, 125.5 us per step).
constexpr int kCompactPerSlot = 4;

hipError_t launch_index_score_decode(const Dims& d, const Cache& c, const uint16_t* idx_q,
                                     const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                     float* pooled, uint32_t* counters, hipStream_t stream,
                                     const DecodeAppend* append) {
  const int B = d.block_size;
  const int max_own = (max_seq_len - 1) / B;
  // blocks 0 .. max_own-1 are scored; with an append, one more workgroup
  // per sequence writes the current token
  const int gx = append != nullptr ? max_own + 1 : (max_own > 0 ? max_own : 1);
  DecodeAppend ap{};
  if (append != nullptr) ap = *append;
  const int mt = (d.num_kv_heads * d.num_idx_heads + 15) / 16;
  const bool pg = d.idx_k_heads > 1;
  // Large batches of up to 64 sequences (where lengths can differ widely):
  // the compact grid, kCompactPerSlot workgroups per slot the LDS keeps
  // resident.
  const size_t full = (size_t)gx * batch;
  if (!pg && batch > 1 && batch <= 64 && full > kCompactMinGrid) {
    const int wgs = (int)std::min<size_t>(full, (size_t)kCompactPerSlot * 256 * (kLdsPerCu / (B * 128)));
    if (B == 64)
      return launch_compact_b<64>(d.num_idx_heads, mt, wgs, stream, c.idx_k, c.block_table,
                                  c.max_blocks, idx_q, seq_lens, batch, d.num_kv_heads,
                                  d.idx_k_heads, pooled, counters, ap);
    return launch_compact_b<128>(d.num_idx_heads, mt, wgs, stream, c.idx_k, c.block_table,
                                 c.max_blocks, idx_q, seq_lens, batch, d.num_kv_heads,
                                 d.idx_k_heads, pooled, counters, ap);
  }
  dim3 grid(gx, batch, pg ? d.num_kv_heads : 1);
  if (B == 64)
    return launch_decode_b<64>(d.num_idx_heads, mt, pg, grid, stream, c.idx_k, c.block_table,
                               c.max_blocks, idx_q, seq_lens, d.num_kv_heads, d.idx_k_heads,
                               pooled, counters, ap);
  return launch_decode_b<128>(d.num_idx_heads, mt, pg, grid, stream, c.idx_k, c.block_table,
                              c.max_blocks, idx_q, seq_lens, d.num_kv_heads, d.idx_k_heads, pooled,
                              counters, ap);
}

#ifdef MSA_TIMELINE
MSA_TIMELINE_ACCESSORS(index)
#endif

}  // namespace msa
