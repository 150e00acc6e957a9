// Host side of libmsa.so: argument validation, workspace layout and the
// launch sequence of each entry point declared in include/msa.h.
//
// Validation is pure host code and runs before any HIP call, so a rejected
// call touches no device state.  Nothing here allocates, copies or
// synchronises.  No C++ exception can leave an entry point: the error text
// lives in a fixed thread-local buffer (no allocation), and every entry point
// also catches whatever a callee might throw.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>

#include "msa.h"
#include "msa_launch.h"
#include "msa_probes.h"
#include "msa_timeline.h"
#include "msa_api_internal.h"

namespace {

thread_local char g_last_error[512];

msa_status fail(msa_status st, const char* msg) {
  std::snprintf(g_last_error, sizeof g_last_error, "%s", msg);
  return st;
}

size_t align_up(size_t x) { return (x + 255) & ~size_t(255); }

bool is_pow2_idx_heads(int n) { return n == 1 || n == 2 || n == 4 || n == 8 || n == 16; }

msa_status check_params(const msa_params* p) {
  if (p == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "params is NULL");
  if (p->num_q_heads < 1 || p->num_kv_heads < 1 || p->head_dim < 1 || p->num_idx_heads < 1 ||
      p->idx_dim < 1 || p->block_size < 1 || p->top_k < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "head counts, dims, block_size and top_k must be >= 1");
  if (p->num_q_heads % p->num_kv_heads != 0)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_q_heads must be a multiple of num_kv_heads");
  if (!std::isfinite(p->softmax_scale))
    return fail(MSA_ERR_INVALID_ARGUMENT, "softmax_scale must be finite");
  if (p->sink_blocks < 0 || p->local_blocks < 0 ||
      (int64_t)p->sink_blocks + p->local_blocks > (int64_t)p->top_k - 1)
    return fail(MSA_ERR_INVALID_ARGUMENT,
                "sink_blocks and local_blocks must be >= 0 with sink + local <= top_k - 1");
  if (p->head_dim != 128) return fail(MSA_ERR_UNSUPPORTED, "head_dim must be 128");
  if (p->idx_dim != 64) return fail(MSA_ERR_UNSUPPORTED, "idx_dim must be 64");
  if (p->block_size != 64 && p->block_size != 128)
    return fail(MSA_ERR_UNSUPPORTED, "block_size must be 64 or 128");
  if (p->top_k > 64) return fail(MSA_ERR_UNSUPPORTED, "top_k must be <= 64");
  if (!is_pow2_idx_heads(p->num_idx_heads))
    return fail(MSA_ERR_UNSUPPORTED, "num_idx_heads must be 1, 2, 4, 8 or 16");
  if (p->num_kv_heads * p->num_idx_heads > 64)
    return fail(MSA_ERR_UNSUPPORTED, "num_kv_heads * num_idx_heads must be <= 64");
  if (p->num_q_heads / p->num_kv_heads > 16)
    return fail(MSA_ERR_UNSUPPORTED, "group size num_q_heads/num_kv_heads must be <= 16");
  if (p->num_idx_k_heads != 0 && p->num_idx_k_heads != 1 && p->num_idx_k_heads != p->num_kv_heads)
    return fail(MSA_ERR_UNSUPPORTED, "num_idx_k_heads must be 0, 1 or num_kv_heads");
  return MSA_OK;
}

msa_status check_kv(const msa_paged_kv* kv) {
  if (kv == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (kv->k == nullptr || kv->v == nullptr || kv->idx_k == nullptr || kv->block_table == nullptr)
    return fail(MSA_ERR_INVALID_ARGUMENT, "kv cache pointer is NULL");
  if (kv->num_pages < 1 || kv->max_blocks_per_seq < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages and max_blocks_per_seq must be >= 1");
  return MSA_OK;
}

msa_status check_kv_mut(const msa_paged_kv_mut* kv) {
  if (kv == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "kv is NULL");
  if (kv->k == nullptr || kv->v == nullptr || kv->idx_k == nullptr || kv->block_table == nullptr)
    return fail(MSA_ERR_INVALID_ARGUMENT, "kv cache pointer is NULL");
  if (kv->num_pages < 1 || kv->max_blocks_per_seq < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "num_pages and max_blocks_per_seq must be >= 1");
  return MSA_OK;
}

msa::CacheW cache_w_of(const msa_paged_kv_mut* kv) {
  return msa::CacheW{static_cast<uint16_t*>(kv->k), static_cast<uint16_t*>(kv->v),
                     static_cast<uint16_t*>(kv->idx_k), kv->block_table, kv->num_pages,
                     kv->max_blocks_per_seq};
}

msa_paged_kv read_view(const msa_paged_kv_mut* kv) {
  return msa_paged_kv{kv->k, kv->v, kv->idx_k, kv->block_table, kv->num_pages,
                      kv->max_blocks_per_seq};
}

msa::Dims dims_of(const msa_params* p) {
  return msa::Dims{p->num_q_heads, p->num_kv_heads, p->head_dim,   p->num_idx_heads,
                   p->idx_dim,     p->block_size,   p->top_k,      p->softmax_scale,
                   p->sink_blocks, p->local_blocks,
                   p->num_idx_k_heads > 1 ? p->num_idx_k_heads : 1};
}

msa::Cache cache_of(const msa_paged_kv* kv) {
  return msa::Cache{static_cast<const uint16_t*>(kv->k), static_cast<const uint16_t*>(kv->v),
                    static_cast<const uint16_t*>(kv->idx_k), kv->block_table, kv->num_pages,
                    kv->max_blocks_per_seq};
}

msa_status hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return MSA_OK;
  std::snprintf(g_last_error, sizeof g_last_error, "%s: %s", what, hipGetErrorString(e));
  return MSA_ERR_HIP;
}

// decode workspace layout
struct DecodeWs {
  size_t pooled, part_o, part_ml, counters, sel, total;
};
DecodeWs decode_layout(const msa_params* p, int32_t batch, int32_t max_blocks) {
  const size_t G = (size_t)(p->num_q_heads / p->num_kv_heads);
  const size_t sg = (size_t)batch * p->num_kv_heads;
  DecodeWs w{};
  size_t off = 0;
  w.pooled = off;
  off += align_up(sg * (size_t)max_blocks * sizeof(float));
  w.part_o = off;
  off += align_up(sg * p->top_k * G * p->head_dim * sizeof(float));
  w.part_ml = off;
  off += align_up(sg * p->top_k * G * 4 * sizeof(float));
  w.counters = off;
  off += align_up(sg * sizeof(uint32_t));
  w.sel = off;
  off += align_up(sg * p->top_k * sizeof(int32_t));
  w.total = off;
  return w;
}

int32_t num_tiles_of(int32_t prior_len, int32_t chunk_len, int32_t B) {
  return (int32_t)(((int64_t)prior_len + chunk_len + B - 1) / B - prior_len / B);
}

struct PrefillWs {
  size_t pooled, sel, total;
};
PrefillWs prefill_layout(const msa_params* p, int32_t prior_len, int32_t chunk_len,
                         int32_t max_blocks) {
  const size_t rows = (size_t)num_tiles_of(prior_len, chunk_len, p->block_size) * p->num_kv_heads;
  PrefillWs w{};
  w.pooled = 0;
  w.sel = align_up(rows * (size_t)max_blocks * sizeof(float));
  w.total = w.sel + align_up(rows * p->top_k * sizeof(int32_t));
  return w;
}

// One sequence as a chunk map (no device tables).
msa::ChunkMap single_map(int32_t prior_len, int32_t chunk_len, int32_t max_blocks) {
  return msa::ChunkMap{nullptr, nullptr, nullptr, nullptr, nullptr, prior_len, chunk_len,
                       max_blocks};
}

// Sizes of a batch of chunks, from the host copies of the lengths.
struct VarlenSizes {
  int64_t tiles, rows;
  int32_t max_own;
};
VarlenSizes varlen_sizes(const int32_t* prior, const int32_t* chunk, int32_t batch, int32_t B) {
  VarlenSizes v{0, 0, 0};
  for (int32_t s = 0; s < batch; ++s) {
    const int64_t p = prior[s], c = chunk[s];
    v.tiles += (p + c + B - 1) / B - p / B;
    v.rows += c;
    v.max_own = std::max(v.max_own, (int32_t)((p + c - 1) / B));
  }
  return v;
}

struct VarlenWs {
  size_t pooled, sel, tile_seq, tile_start, q_start, total;
};
VarlenWs varlen_layout(const msa_params* p, int64_t tiles, int32_t batch, int32_t max_blocks) {
  const size_t rows = (size_t)tiles * p->num_kv_heads;
  VarlenWs w{};
  size_t off = 0;
  w.pooled = off;
  off += align_up(rows * (size_t)max_blocks * sizeof(float));
  w.sel = off;
  off += align_up(rows * p->top_k * sizeof(int32_t));
  w.tile_seq = off;
  off += align_up((size_t)tiles * sizeof(int32_t));
  w.tile_start = off;
  off += align_up(((size_t)batch + 1) * sizeof(int32_t));
  w.q_start = off;
  off += align_up(((size_t)batch + 1) * sizeof(int32_t));
  w.total = off;
  return w;
}

msa_status check_varlen(const msa_params* p, int32_t max_blocks, const int32_t* prior_host,
                        const int32_t* chunk_host, int32_t batch) {
  if (prior_host == nullptr || chunk_host == nullptr)
    return fail(MSA_ERR_INVALID_ARGUMENT, "host length arrays must not be NULL");
  if (batch < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  for (int32_t s = 0; s < batch; ++s) {
    if (prior_host[s] < 0 || chunk_host[s] < 1)
      return fail(MSA_ERR_INVALID_ARGUMENT, "prior_lens must be >= 0 and chunk_lens >= 1");
    if ((int64_t)prior_host[s] + chunk_host[s] > (int64_t)max_blocks * p->block_size)
      return fail(MSA_ERR_INVALID_ARGUMENT,
                  "prior_len + chunk_len exceeds max_blocks_per_seq * block_size");
  }
  const VarlenSizes v = varlen_sizes(prior_host, chunk_host, batch, p->block_size);
  if (v.tiles > 0x7FFFFFFF || v.rows > 0x7FFFFFFF)
    return fail(MSA_ERR_UNSUPPORTED, "total tiles and chunk rows must fit in int32");
  if (p->block_size * p->num_idx_heads > 512)
    return fail(MSA_ERR_UNSUPPORTED, "prefill needs block_size * num_idx_heads <= 512");
  return MSA_OK;
}

msa_status check_prefill_sizes(const msa_params* p, const msa_paged_kv* kv, int32_t prior_len,
                               int32_t chunk_len) {
  if (prior_len < 0 || chunk_len < 1)
    return fail(MSA_ERR_INVALID_ARGUMENT, "prior_len must be >= 0 and chunk_len >= 1");
  if ((int64_t)prior_len + chunk_len > (int64_t)kv->max_blocks_per_seq * p->block_size)
    return fail(MSA_ERR_INVALID_ARGUMENT,
                "prior_len + chunk_len exceeds max_blocks_per_seq * block_size");
  if (p->block_size * p->num_idx_heads > 512)
    return fail(MSA_ERR_UNSUPPORTED, "prefill needs block_size * num_idx_heads <= 512");
  return MSA_OK;
}

}  // namespace

namespace msa {
msa_status set_error(msa_status st, const char* msg) { return fail(st, msg); }
}  // namespace msa

extern "C" {

const char* msa_last_error(void) { return g_last_error; }

const char* msa_version(void) { return "msa-mi355x 0.1.0 (gfx950)"; }

size_t msa_decode_workspace_bytes(const msa_params* params, int32_t batch,
                                  int32_t max_blocks_per_seq) {
  try {
    if (check_params(params) != MSA_OK || batch < 1 || max_blocks_per_seq < 1) return 0;
    return decode_layout(params, batch, max_blocks_per_seq).total;
  } catch (...) {
    return 0;
  }
}

msa_status msa_index_score_decode(const msa_params* params, const msa_paged_kv* kv,
                                  const void* idx_q, const int32_t* seq_lens, int32_t batch,
                                  int32_t max_seq_len, float* pooled, void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv(kv)) != MSA_OK) return st;
    if (idx_q == nullptr || seq_lens == nullptr || pooled == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "idx_q, seq_lens and pooled must not be NULL");
    if (batch < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
    if (max_seq_len < 1 || (int64_t)max_seq_len > (int64_t)kv->max_blocks_per_seq * params->block_size)
      return fail(MSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [1, max_blocks_per_seq*block_size]");
    return hip_status(msa::launch_index_score_decode(dims_of(params), cache_of(kv),
                                                     static_cast<const uint16_t*>(idx_q), seq_lens,
                                                     batch, max_seq_len, pooled, nullptr,
                                                     static_cast<hipStream_t>(stream)),
                      "index score launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

msa_status msa_cache_append(const msa_params* params, const msa_paged_kv_mut* kv,
                            const void* k_new, const void* v_new, const void* idx_k_new,
                            const int32_t* start_pos, int32_t batch, int32_t n_new, void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv_mut(kv)) != MSA_OK) return st;
    if (k_new == nullptr || v_new == nullptr || idx_k_new == nullptr || start_pos == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "k_new, v_new, idx_k_new and start_pos must not be NULL");
    if (batch < 1 || n_new < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "batch and n_new must be >= 1");
    if (batch > 65535) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535");
    if ((int64_t)n_new > (int64_t)kv->max_blocks_per_seq * params->block_size)
      return fail(MSA_ERR_INVALID_ARGUMENT, "n_new exceeds max_blocks_per_seq * block_size");
    return hip_status(msa::launch_cache_append(dims_of(params), cache_w_of(kv),
                                               static_cast<const uint16_t*>(k_new),
                                               static_cast<const uint16_t*>(v_new),
                                               static_cast<const uint16_t*>(idx_k_new), start_pos,
                                               batch, n_new, static_cast<hipStream_t>(stream)),
                      "cache append launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

using msa::decode_impl;

msa_status msa_decode(const msa_params* params, const msa_paged_kv* kv, const void* q,
                      const void* idx_q, const int32_t* seq_lens, int32_t batch,
                      int32_t max_seq_len, float* out, int32_t* sel, void* workspace,
                      size_t workspace_bytes, void* stream) {
  try {
    return decode_impl(params, kv, q, idx_q, seq_lens, batch, max_seq_len, out, sel, workspace,
                       workspace_bytes, stream, nullptr);
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

msa_status msa_decode_append(const msa_params* params, const msa_paged_kv_mut* kv,
                             const void* k_new, const void* v_new, const void* idx_k_new,
                             const void* q, const void* idx_q, const int32_t* seq_lens,
                             int32_t batch, int32_t max_seq_len, float* out, int32_t* sel,
                             void* workspace, size_t workspace_bytes, void* stream) {
  try {
    msa_status st = check_kv_mut(kv);
    if (st != MSA_OK) return st;
    if (k_new == nullptr || v_new == nullptr || idx_k_new == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "k_new, v_new and idx_k_new must not be NULL");
    const msa_paged_kv view = read_view(kv);
    const msa::DecodeAppend ap{cache_w_of(kv), static_cast<const uint16_t*>(k_new),
                               static_cast<const uint16_t*>(v_new),
                               static_cast<const uint16_t*>(idx_k_new)};
    return decode_impl(params, &view, q, idx_q, seq_lens, batch, max_seq_len, out, sel, workspace,
                       workspace_bytes, stream, &ap);
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

}  // extern "C"

// (shared with the allocation-free entry point, msa_decode_noalloc)
msa_status msa::decode_impl(const msa_params* params, const msa_paged_kv* kv, const void* q,
                            const void* idx_q, const int32_t* seq_lens, int32_t batch,
                            int32_t max_seq_len, float* out, int32_t* sel, void* workspace,
                            size_t workspace_bytes, void* stream,
                            const msa::DecodeAppend* append) {
  msa_status st = check_params(params);
  if (st != MSA_OK) return st;
  if ((st = check_kv(kv)) != MSA_OK) return st;
  if (q == nullptr || idx_q == nullptr || seq_lens == nullptr || out == nullptr)
    return fail(MSA_ERR_INVALID_ARGUMENT, "q, idx_q, seq_lens and out must not be NULL");
  if (batch < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "batch must be >= 1");
  if (batch > 65535) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535");
  if (max_seq_len < 1 || (int64_t)max_seq_len > (int64_t)kv->max_blocks_per_seq * params->block_size)
    return fail(MSA_ERR_INVALID_ARGUMENT, "max_seq_len must be in [1, max_blocks_per_seq*block_size]");
  const DecodeWs w = decode_layout(params, batch, kv->max_blocks_per_seq);
  if (workspace == nullptr || workspace_bytes < w.total)
    return fail(MSA_ERR_WORKSPACE, "workspace missing or smaller than msa_decode_workspace_bytes()");
  uint8_t* ws = static_cast<uint8_t*>(workspace);
  float* pooled = reinterpret_cast<float*>(ws + w.pooled);
  uint32_t* counters = reinterpret_cast<uint32_t*>(ws + w.counters);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const msa::Dims d = dims_of(params);
  const msa::Cache c = cache_of(kv);
  st = hip_status(msa::launch_index_score_decode(d, c, static_cast<const uint16_t*>(idx_q),
                                                 seq_lens, batch, max_seq_len, pooled, counters, s,
                                                 append),
                  "index score launch");
  if (st != MSA_OK) return st;
  return hip_status(
      msa::launch_decode_attn(d, c, static_cast<const uint16_t*>(q), seq_lens, batch, max_seq_len,
                              pooled,
                              reinterpret_cast<float*>(ws + w.part_o),
                              reinterpret_cast<float*>(ws + w.part_ml), counters,
                              sel != nullptr ? sel : reinterpret_cast<int32_t*>(ws + w.sel), out, s),
      "sparse attention launch");
}

extern "C" {

size_t msa_prefill_workspace_bytes(const msa_params* params, int32_t prior_len, int32_t chunk_len,
                                   int32_t max_blocks_per_seq) {
  try {
    if (check_params(params) != MSA_OK || prior_len < 0 || chunk_len < 1 || max_blocks_per_seq < 1)
      return 0;
    return prefill_layout(params, prior_len, chunk_len, max_blocks_per_seq).total;
  } catch (...) {
    return 0;
  }
}

msa_status msa_index_score_prefill(const msa_params* params, const msa_paged_kv* kv,
                                   const void* idx_q, int32_t prior_len, int32_t chunk_len,
                                   float* pooled, void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv(kv)) != MSA_OK) return st;
    if (idx_q == nullptr || pooled == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "idx_q and pooled must not be NULL");
    if ((st = check_prefill_sizes(params, kv, prior_len, chunk_len)) != MSA_OK) return st;
    const int32_t B = params->block_size;
    const int32_t tiles = num_tiles_of(prior_len, chunk_len, B);
    return hip_status(msa::launch_index_score_prefill(
                          dims_of(params), cache_of(kv), static_cast<const uint16_t*>(idx_q),
                          single_map(prior_len, chunk_len, kv->max_blocks_per_seq), tiles,
                          prior_len / B + tiles - 1, pooled, static_cast<hipStream_t>(stream)),
                      "prefill index score launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

msa_status msa_block_topk_prefill(const msa_params* params, int32_t prior_len, int32_t chunk_len,
                                  int32_t max_blocks_per_seq, const float* pooled, int32_t* sel,
                                  void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if (pooled == nullptr || sel == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "pooled and sel must not be NULL");
    if (prior_len < 0 || chunk_len < 1 || max_blocks_per_seq < 1 ||
        (int64_t)prior_len + chunk_len > (int64_t)max_blocks_per_seq * params->block_size)
      return fail(MSA_ERR_INVALID_ARGUMENT, "inconsistent prior_len, chunk_len, max_blocks_per_seq");
    return hip_status(msa::launch_block_topk_prefill(
                          dims_of(params), single_map(prior_len, chunk_len, max_blocks_per_seq),
                          num_tiles_of(prior_len, chunk_len, params->block_size),
                          max_blocks_per_seq, pooled, sel, static_cast<hipStream_t>(stream)),
                      "prefill topk launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

msa_status msa_sparse_attn_prefill(const msa_params* params, const msa_paged_kv* kv, const void* q,
                                   int32_t prior_len, int32_t chunk_len, const int32_t* sel,
                                   float* out, void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv(kv)) != MSA_OK) return st;
    if (q == nullptr || sel == nullptr || out == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "q, sel and out must not be NULL");
    if ((st = check_prefill_sizes(params, kv, prior_len, chunk_len)) != MSA_OK) return st;
    return hip_status(msa::launch_sparse_attn_prefill(
                          dims_of(params), cache_of(kv), static_cast<const uint16_t*>(q),
                          single_map(prior_len, chunk_len, kv->max_blocks_per_seq),
                          num_tiles_of(prior_len, chunk_len, params->block_size), sel, out,
                          static_cast<hipStream_t>(stream)),
                      "prefill sparse attention launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

msa_status msa_prefill_chunk(const msa_params* params, const msa_paged_kv* kv, const void* q,
                             const void* idx_q, int32_t prior_len, int32_t chunk_len, float* out,
                             int32_t* sel, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv(kv)) != MSA_OK) return st;
    if (q == nullptr || idx_q == nullptr || out == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "q, idx_q and out must not be NULL");
    if ((st = check_prefill_sizes(params, kv, prior_len, chunk_len)) != MSA_OK) return st;
    const PrefillWs w = prefill_layout(params, prior_len, chunk_len, kv->max_blocks_per_seq);
    if (workspace == nullptr || workspace_bytes < w.total)
      return fail(MSA_ERR_WORKSPACE, "workspace missing or smaller than msa_prefill_workspace_bytes()");
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* pooled = reinterpret_cast<float*>(ws + w.pooled);
    int32_t* sel_buf = sel != nullptr ? sel : reinterpret_cast<int32_t*>(ws + w.sel);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const msa::Dims d = dims_of(params);
    const msa::Cache c = cache_of(kv);
    const msa::ChunkMap m = single_map(prior_len, chunk_len, kv->max_blocks_per_seq);
    const int32_t tiles = num_tiles_of(prior_len, chunk_len, params->block_size);
    const int32_t max_own = prior_len / params->block_size + tiles - 1;
    st = hip_status(msa::launch_index_score_prefill(d, c, static_cast<const uint16_t*>(idx_q), m,
                                                    tiles, max_own, pooled, s),
                    "prefill index score launch");
    if (st != MSA_OK) return st;
    st = hip_status(msa::launch_block_topk_prefill(d, m, tiles, kv->max_blocks_per_seq, pooled,
                                                   sel_buf, s),
                    "prefill topk launch");
    if (st != MSA_OK) return st;
    return hip_status(msa::launch_sparse_attn_prefill(d, c, static_cast<const uint16_t*>(q), m,
                                                      tiles, sel_buf, out, s),
                      "prefill sparse attention launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

size_t msa_prefill_varlen_workspace_bytes(const msa_params* params, const int32_t* prior_lens_host,
                                          const int32_t* chunk_lens_host, int32_t batch,
                                          int32_t max_blocks_per_seq) {
  try {
    if (check_params(params) != MSA_OK || max_blocks_per_seq < 1 ||
        check_varlen(params, max_blocks_per_seq, prior_lens_host, chunk_lens_host, batch) != MSA_OK)
      return 0;
    const VarlenSizes v = varlen_sizes(prior_lens_host, chunk_lens_host, batch, params->block_size);
    return varlen_layout(params, v.tiles, batch, max_blocks_per_seq).total;
  } catch (...) {
    return 0;
  }
}

msa_status msa_prefill_varlen(const msa_params* params, const msa_paged_kv* kv, const void* q,
                              const void* idx_q, const int32_t* prior_lens,
                              const int32_t* chunk_lens, const int32_t* prior_lens_host,
                              const int32_t* chunk_lens_host, int32_t batch, float* out,
                              int32_t* sel, void* workspace, size_t workspace_bytes,
                              void* stream) {
  try {
    msa_status st = check_params(params);
    if (st != MSA_OK) return st;
    if ((st = check_kv(kv)) != MSA_OK) return st;
    if (q == nullptr || idx_q == nullptr || out == nullptr || prior_lens == nullptr ||
        chunk_lens == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT,
                  "q, idx_q, out, prior_lens and chunk_lens must not be NULL");
    if (batch > 65535) return fail(MSA_ERR_UNSUPPORTED, "batch must be <= 65535");
    if ((st = check_varlen(params, kv->max_blocks_per_seq, prior_lens_host, chunk_lens_host,
                           batch)) != MSA_OK)
      return st;
    const VarlenSizes v = varlen_sizes(prior_lens_host, chunk_lens_host, batch, params->block_size);
    const VarlenWs w = varlen_layout(params, v.tiles, batch, kv->max_blocks_per_seq);
    if (workspace == nullptr || workspace_bytes < w.total)
      return fail(MSA_ERR_WORKSPACE,
                  "workspace missing or smaller than msa_prefill_varlen_workspace_bytes()");
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* pooled = reinterpret_cast<float*>(ws + w.pooled);
    int32_t* sel_buf = sel != nullptr ? sel : reinterpret_cast<int32_t*>(ws + w.sel);
    int32_t* tile_seq = reinterpret_cast<int32_t*>(ws + w.tile_seq);
    int32_t* tile_start = reinterpret_cast<int32_t*>(ws + w.tile_start);
    int32_t* q_start = reinterpret_cast<int32_t*>(ws + w.q_start);
    hipStream_t s = static_cast<hipStream_t>(stream);
    const msa::Dims d = dims_of(params);
    const msa::Cache c = cache_of(kv);
    const int32_t tiles = (int32_t)v.tiles;
    st = hip_status(msa::launch_chunk_map(prior_lens, chunk_lens, batch, params->block_size, tiles,
                                          tile_seq, tile_start, q_start, s),
                    "prefill chunk map launch");
    if (st != MSA_OK) return st;
    const msa::ChunkMap m{tile_seq, tile_start, q_start, prior_lens, chunk_lens, 0, 0,
                          kv->max_blocks_per_seq};
    st = hip_status(msa::launch_index_score_prefill(d, c, static_cast<const uint16_t*>(idx_q), m,
                                                    tiles, v.max_own, pooled, s),
                    "prefill index score launch");
    if (st != MSA_OK) return st;
    st = hip_status(msa::launch_block_topk_prefill(d, m, tiles, kv->max_blocks_per_seq, pooled,
                                                   sel_buf, s),
                    "prefill topk launch");
    if (st != MSA_OK) return st;
    return hip_status(msa::launch_sparse_attn_prefill(d, c, static_cast<const uint16_t*>(q), m,
                                                      tiles, sel_buf, out, s),
                      "prefill sparse attention launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

}  // extern "C"

// ------------------------------------------------------------ measurement
extern "C" msa_status msa_probe_read_stream(const void* src, size_t bytes, int32_t workgroups,
                                            uint32_t* sink, void* stream) {
  try {
    if (src == nullptr || sink == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "src and sink must not be NULL");
    if (bytes < 16 || bytes % 16 != 0)
      return fail(MSA_ERR_INVALID_ARGUMENT, "bytes must be a positive multiple of 16");
    if (workgroups < 1 || workgroups > (1 << 20))
      return fail(MSA_ERR_INVALID_ARGUMENT, "workgroups must be in [1, 2^20]");
    return hip_status(msa::launch_read_stream(src, bytes, workgroups, sink,
                                              static_cast<hipStream_t>(stream)),
                      "read stream launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

extern "C" msa_status msa_probe_mfma_bf16(int32_t iters, int32_t workgroups, float* sink,
                                          void* stream) {
  try {
    if (sink == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "sink must not be NULL");
    if (iters < 1 || iters > (1 << 24))
      return fail(MSA_ERR_INVALID_ARGUMENT, "iters must be in [1, 2^24]");
    if (workgroups < 1 || workgroups > 65536)
      return fail(MSA_ERR_INVALID_ARGUMENT, "workgroups must be in [1, 65536]");
    return hip_status(msa::launch_mfma_loop(iters, workgroups, sink, static_cast<hipStream_t>(stream)),
                      "mfma loop launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

extern "C" msa_status msa_probe_latency_chain(const int32_t* next, int32_t n, int32_t steps,
                                              int32_t start, int32_t* sink, void* stream) {
  try {
    if (next == nullptr || sink == nullptr)
      return fail(MSA_ERR_INVALID_ARGUMENT, "next and sink must not be NULL");
    if (n < 1) return fail(MSA_ERR_INVALID_ARGUMENT, "n must be >= 1");
    if (start < 0 || start >= n) return fail(MSA_ERR_INVALID_ARGUMENT, "start must be in [0, n)");
    if (steps < 0 || steps > (1 << 24))
      return fail(MSA_ERR_INVALID_ARGUMENT, "steps must be in [0, 2^24]");
    return hip_status(msa::launch_latency_chain(next, n, steps, start, sink,
                                                static_cast<hipStream_t>(stream)),
                      "latency chain launch");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

#ifdef MSA_TIMELINE
// Timeline build only: the marks of msa_timeline.h.
extern "C" msa_status msa_timeline_clear(void) {
  try {
    const hipError_t e = msa::timeline_clear_attn();
    if (e != hipSuccess) return hip_status(e, "timeline clear");
    return hip_status(msa::timeline_clear_index(), "timeline clear");
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}

extern "C" msa_status msa_timeline_read(uint64_t* marks, int32_t n) {
  try {
    if (marks == nullptr) return fail(MSA_ERR_INVALID_ARGUMENT, "marks must not be NULL");
    if (n < MSA_NUM_MARKS) return fail(MSA_ERR_INVALID_ARGUMENT, "n must be >= MSA_NUM_MARKS");
    unsigned long long attn[MSA_NUM_MARKS], index[MSA_NUM_MARKS];
    hipError_t e = hipDeviceSynchronize();
    if (e == hipSuccess) e = msa::timeline_read_attn(attn);
    if (e == hipSuccess) e = msa::timeline_read_index(index);
    if (e != hipSuccess) return hip_status(e, "timeline read");
    for (int i = 0; i < MSA_NUM_MARKS; ++i) marks[i] = attn[i];
    marks[MSA_MARK_INDEX_END] = index[MSA_MARK_INDEX_END];
    return MSA_OK;
  } catch (...) {
    return fail(MSA_ERR_HIP, "unexpected internal error");
  }
}
#endif
