// TopK of the prefill index branch: one 256-thread workgroup per (tile, group)
// selects the tile's kept blocks from its pooled scores ("MiniMax wird dünn",
// section 1, Schritt 1, TopK; the diagonal block of the tile is forced, and
// so are the optional sink and local-window blocks).
#include "block_topk.h"
#include "msa_launch.h"

namespace msa {

__global__ __launch_bounds__(256) void block_topk_prefill_kernel(
    const float* __restrict__ pooled, int32_t first_block, int32_t num_kv_heads, int32_t max_blocks,
    int32_t top_k, int32_t n_sink, int32_t n_local, int32_t* __restrict__ sel) {
  __shared__ TopkShared sh;
  __shared__ int sel_s[kMaxTopK], tmp_s[kMaxTopK];
  const int tile = blockIdx.x, g = blockIdx.y;
  const size_t row = (size_t)tile * num_kv_heads + g;
  block_topk_forced(pooled + row * max_blocks, first_block + tile, top_k, n_sink, n_local, sel_s,
                    tmp_s, sh);
  for (int i = threadIdx.x; i < top_k; i += blockDim.x) sel[row * top_k + i] = sel_s[i];
}

hipError_t launch_block_topk_prefill(const Dims& d, int32_t prior_len, int32_t chunk_len,
                                     int32_t max_blocks, const float* pooled, int32_t* sel,
                                     hipStream_t stream) {
  const int B = d.block_size;
  const int first = prior_len / B;
  const int num_tiles = (prior_len + chunk_len + B - 1) / B - first;
  hipLaunchKernelGGL(block_topk_prefill_kernel, dim3(num_tiles, d.num_kv_heads), dim3(256), 0,
                     stream, pooled, first, d.num_kv_heads, max_blocks, d.top_k, d.sink_blocks,
                     d.local_blocks, sel);
  return hipGetLastError();
}

}  // namespace msa
