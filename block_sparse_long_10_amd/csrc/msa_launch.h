// Internal launch interface between the host dispatch (msa_api.cpp) and the
// HIP kernels.  Every launcher enqueues on `stream` and returns the
// hipGetLastError() of its launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

struct Dims {
  int32_t num_q_heads, num_kv_heads, head_dim, num_idx_heads, idx_dim, block_size, top_k;
  float softmax_scale;
  int32_t sink_blocks, local_blocks;  // forced blocks of the selection
  int32_t idx_k_heads;                // 1 (shared index-key head) or Hkv (one per group)
};

struct Cache {
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* idx_k;
  const int32_t* block_table;
  int32_t num_pages, max_blocks;
};

// Writable view of the same cache (cache append).
struct CacheW {
  uint16_t* k;
  uint16_t* v;
  uint16_t* idx_k;
  const int32_t* block_table;
  int32_t num_pages, max_blocks;
};

// The current token of each sequence (position seq_lens[s]-1) written into
// its page: k_new, v_new [batch][Hkv][D], idx_new [batch][d_i].
struct DecodeAppend {
  CacheW cache;
  const uint16_t* k_new;
  const uint16_t* v_new;
  const uint16_t* idx_new;
};

// Step 1, decode: pooled[s][g][b] for b < own(s).  When counters is not
// null, counters [batch][Hkv] are cleared for the attention launch.  When
// append is not null, the launch also writes each sequence's current token
// into its own block (which the index branch never reads).
hipError_t launch_index_score_decode(const Dims& d, const Cache& c, const uint16_t* idx_q,
                                     const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                                     float* pooled, uint32_t* counters, hipStream_t stream,
                                     const DecodeAppend* append = nullptr);

// Cache append: n_new tokens per sequence at positions start_pos[s] ..
// start_pos[s]+n_new-1; k_new, v_new [batch][n_new][Hkv][D],
// idx_new [batch][n_new][d_i].
hipError_t launch_cache_append(const Dims& d, const CacheW& c, const uint16_t* k_new,
                               const uint16_t* v_new, const uint16_t* idx_new,
                               const int32_t* start_pos, int32_t batch, int32_t n_new,
                               hipStream_t stream);

// TopK, Step 2 over the kept blocks (one partial per block) and the merge of
// the partials, decode.  counters must be zero on entry.
hipError_t launch_decode_attn(const Dims& d, const Cache& c, const uint16_t* q,
                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              const float* pooled, float* part_o, float* part_ml,
                              uint32_t* counters, int32_t* sel, float* out, hipStream_t stream);

// Prefill chunks of one or several sequences.  Tiles are numbered sequence
// after sequence; tile u of the call is local tile t of sequence s, whose
// chunk rows start at row q_start[s] of q / idx_q / out.  With
// tile_seq == nullptr there is one sequence (s = 0, t = u, q rows from 0)
// whose lengths are prior_len and chunk_len.
struct ChunkMap {
  const int32_t* tile_seq;    // [num_tiles] sequence of each tile (device)
  const int32_t* tile_start;  // [batch + 1] first tile of each sequence
  const int32_t* q_start;     // [batch + 1] first chunk row of each sequence
  const int32_t* prior_lens;  // [batch]
  const int32_t* chunk_lens;  // [batch]
  int32_t prior_len, chunk_len;
  int32_t max_blocks;         // block-table row stride
};

// Builds tile_seq, tile_start and q_start of a batch of chunks (one
// workgroup) from the device lengths.
hipError_t launch_chunk_map(const int32_t* prior_lens, const int32_t* chunk_lens, int32_t batch,
                            int32_t block_size, int32_t num_tiles, int32_t* tile_seq,
                            int32_t* tile_start, int32_t* q_start, hipStream_t stream);

// Measurement kernels (peak_probes.hip).
hipError_t launch_read_stream(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream);
hipError_t launch_mfma_loop(int32_t iters, int32_t workgroups, float* sink, hipStream_t stream);
hipError_t launch_latency_chain(const int32_t* next, int32_t n, int32_t steps, int32_t start,
                                int32_t* sink, hipStream_t stream);

// Step 1, prefill: pooled[u][g][b] for b < own(u) = prior/B + t; max_own is
// the largest own block of the call.
hipError_t launch_index_score_prefill(const Dims& d, const Cache& c, const uint16_t* idx_q,
                                      const ChunkMap& m, int32_t num_tiles, int32_t max_own,
                                      float* pooled, hipStream_t stream);

// TopK, prefill: sel[u][g][k].
hipError_t launch_block_topk_prefill(const Dims& d, const ChunkMap& m, int32_t num_tiles,
                                     int32_t max_blocks, const float* pooled, int32_t* sel,
                                     hipStream_t stream);

// Step 2, prefill, for a given selection.
hipError_t launch_sparse_attn_prefill(const Dims& d, const Cache& c, const uint16_t* q,
                                      const ChunkMap& m, int32_t num_tiles, const int32_t* sel,
                                      float* out, hipStream_t stream);

#ifdef MSA_TIMELINE
// Timeline build: copy out / clear the marks of the attention and index
// translation units (synchronous).
hipError_t timeline_read_attn(unsigned long long* out);
hipError_t timeline_clear_attn();
hipError_t timeline_read_index(unsigned long long* out);
hipError_t timeline_clear_index();
#endif

}  // namespace msa
