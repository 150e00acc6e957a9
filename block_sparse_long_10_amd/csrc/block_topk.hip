// TopK of the prefill index branch: one 256-thread workgroup per (tile, group)
// selects the tile's kept blocks from its pooled scores ("MiniMax wird dünn",
// section 1, Schritt 1, TopK; the diagonal block of the tile is forced, and
// so are the optional sink and local-window blocks).
#include "block_topk.h"
#include "chunk_map.h"
#include "msa_launch.h"

namespace msa {

template <int B>
__global__ __launch_bounds__(256) void block_topk_prefill_kernel(
    const float* __restrict__ pooled, ChunkMap map, int32_t num_kv_heads, int32_t max_blocks,
    int32_t top_k, int32_t n_sink, int32_t n_local, int32_t* __restrict__ sel) {
  __shared__ TopkShared sh;
  __shared__ int sel_s[kMaxTopK], tmp_s[kMaxTopK];
  const int tile = blockIdx.x, g = blockIdx.y;
  const TileLoc loc = locate_tile(map, tile);
  const size_t row = (size_t)tile * num_kv_heads + g;
  block_topk_forced<true>(pooled + row * max_blocks, loc.prior / B + loc.tile, top_k, n_sink, n_local,
                    sel_s, tmp_s, sh);
  for (int i = threadIdx.x; i < top_k; i += blockDim.x) sel[row * top_k + i] = sel_s[i];
}

hipError_t launch_block_topk_prefill(const Dims& d, const ChunkMap& map, int32_t num_tiles,
                                     int32_t max_blocks, const float* pooled, int32_t* sel,
                                     hipStream_t stream) {
  if (d.block_size == 64)
    hipLaunchKernelGGL(block_topk_prefill_kernel<64>, dim3(num_tiles, d.num_kv_heads), dim3(256),
                       0, stream, pooled, map, d.num_kv_heads, max_blocks, d.top_k, d.sink_blocks,
                       d.local_blocks, sel);
  else
    hipLaunchKernelGGL(block_topk_prefill_kernel<128>, dim3(num_tiles, d.num_kv_heads), dim3(256),
                       0, stream, pooled, map, d.num_kv_heads, max_blocks, d.top_k, d.sink_blocks,
                       d.local_blocks, sel);
  return hipGetLastError();
}

// ------------------------------------------------------------- chunk map
// One 1024-thread workgroup: thread i takes a contiguous run of sequences,
// the per-thread tile and row totals are scanned in LDS, and every thread then
// writes the offsets and the tile -> sequence entries of its run.
__global__ __launch_bounds__(1024) void chunk_map_kernel(const int32_t* __restrict__ prior_lens,
                                                         const int32_t* __restrict__ chunk_lens,
                                                         int32_t batch, int32_t B,
                                                         int32_t num_tiles,
                                                         int32_t* __restrict__ tile_seq,
                                                         int32_t* __restrict__ tile_start,
                                                         int32_t* __restrict__ q_start) {
  __shared__ int64_t sc_t[1024], sc_q[1024];
  const int tid = threadIdx.x;
  const int per = (batch + 1023) / 1024;
  const int s0 = min(batch, tid * per), s1 = min(batch, s0 + per);
  int64_t nt = 0, nq = 0;
  for (int s = s0; s < s1; ++s) {
    const int64_t p = prior_lens[s], c = chunk_lens[s];
    nt += (p + c + B - 1) / B - p / B;
    nq += c;
  }
  sc_t[tid] = nt;
  sc_q[tid] = nq;
  __syncthreads();
  for (int off = 1; off < 1024; off <<= 1) {  // inclusive Hillis-Steele scan
    const int64_t at = tid >= off ? sc_t[tid - off] : 0, aq = tid >= off ? sc_q[tid - off] : 0;
    __syncthreads();
    sc_t[tid] += at;
    sc_q[tid] += aq;
    __syncthreads();
  }
  int64_t t0 = sc_t[tid] - nt, q0 = sc_q[tid] - nq;
  for (int s = s0; s < s1; ++s) {
    const int64_t p = prior_lens[s], c = chunk_lens[s];
    const int64_t n = (p + c + B - 1) / B - p / B;
    tile_start[s] = (int32_t)t0;
    q_start[s] = (int32_t)q0;
    for (int64_t u = t0; u < t0 + n && u < num_tiles; ++u) tile_seq[u] = s;
    t0 += n;
    q0 += c;
  }
  if (tid == 1023) {
    tile_start[batch] = (int32_t)sc_t[1023];
    q_start[batch] = (int32_t)sc_q[1023];
  }
}

hipError_t launch_chunk_map(const int32_t* prior_lens, const int32_t* chunk_lens, int32_t batch,
                            int32_t block_size, int32_t num_tiles, int32_t* tile_seq,
                            int32_t* tile_start, int32_t* q_start, hipStream_t stream) {
  hipLaunchKernelGGL(chunk_map_kernel, dim3(1), dim3(1024), 0, stream, prior_lens, chunk_lens,
                     batch, block_size, num_tiles, tile_seq, tile_start, q_start);
  return hipGetLastError();
}

}  // namespace msa
