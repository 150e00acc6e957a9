// Cache append: the keys, values and index keys of new tokens are written
// into their pages before the index branch scores them.  "MiniMax wird dünn",
// section 1, Schritt 1 produces one index key per token (K_idx has a single
// head) and section 2 keeps the real, uncompressed K/V; the page layout is
// the one the other kernels read:
//   k     [page][Hkv][B][D]   token-major
//   v     [page][Hkv][B][D]   token-major
//   idx_k [page][Hk][B][d_i]  (Hk = 1, the shared head, or Hkv per group)
//
// One 256-thread workgroup per (sequence, touched block, group) writes the
// new tokens that fall into one page: K, V and index-key rows are 16-byte
// copies, consecutive lanes on consecutive chunks of a row.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

template <int B>
__global__ __launch_bounds__(256) void cache_append_kernel(
    uint16_t* __restrict__ kc, uint16_t* __restrict__ vc, uint16_t* __restrict__ ic,
    const int32_t* __restrict__ block_table, int32_t max_blocks, int32_t num_kv_heads,
    int32_t idx_k_heads,
    const uint16_t* __restrict__ k_new, const uint16_t* __restrict__ v_new,
    const uint16_t* __restrict__ idx_new, const int32_t* __restrict__ start_pos, int32_t n_new) {
  const int j = blockIdx.x, g = blockIdx.y, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int start = start_pos[s];
  const int b = start / B + j;
  const int t_lo = max(start, b * B), t_hi = min(start + n_new, (b + 1) * B);
  if (t_lo >= t_hi) return;  // uniform
  const int n = t_hi - t_lo, slot0 = t_lo - b * B, i0 = t_lo - start;
  const size_t page = (size_t)block_table[(size_t)s * max_blocks + b];
  const size_t tok0 = (size_t)s * n_new + i0;  // first new token of this workgroup

  // K and V rows of group g: 16 chunks of 16 bytes per token each
  for (int x = tid; x < n * 16; x += 256) {
    const int i = x >> 4, c = x & 15;
    const size_t src = ((tok0 + i) * num_kv_heads + g) * 128 + c * 8;
    const size_t dst = ((page * num_kv_heads + g) * B + slot0 + i) * 128 + c * 8;
    const u32x4 kval = *reinterpret_cast<const u32x4*>(k_new + src);
    const u32x4 vval = *reinterpret_cast<const u32x4*>(v_new + src);
    *reinterpret_cast<u32x4*>(kc + dst) = kval;
    *reinterpret_cast<u32x4*>(vc + dst) = vval;
  }
  // index-key rows: the shared head is written once, by group 0; per-group
  // heads by their group
  if (idx_k_heads > 1 || g == 0) {
    const int h = idx_k_heads > 1 ? g : 0;
    for (int x = tid; x < n * 8; x += 256) {
      const int i = x >> 3, c = x & 7;
      const u32x4 val =
          *reinterpret_cast<const u32x4*>(idx_new + ((tok0 + i) * idx_k_heads + h) * 64 + c * 8);
      *reinterpret_cast<u32x4*>(ic + ((page * idx_k_heads + h) * B + slot0 + i) * 64 + c * 8) = val;
    }
  }
}

hipError_t launch_cache_append(const Dims& d, const CacheW& c, const uint16_t* k_new,
                               const uint16_t* v_new, const uint16_t* idx_new,
                               const int32_t* start_pos, int32_t batch, int32_t n_new,
                               hipStream_t stream) {
  const int B = d.block_size;
  // n_new tokens starting anywhere touch at most ceil(n_new/B) + 1 blocks
  const dim3 grid((n_new + B - 1) / B + 1, d.num_kv_heads, batch);
  if (B == 64)
    hipLaunchKernelGGL(cache_append_kernel<64>, grid, dim3(256), 0, stream, c.k, c.v, c.idx_k,
                       c.block_table, c.max_blocks, d.num_kv_heads, d.idx_k_heads, k_new, v_new,
                       idx_new, start_pos, n_new);
  else
    hipLaunchKernelGGL(cache_append_kernel<128>, grid, dim3(256), 0, stream, c.k, c.v, c.idx_k,
                       c.block_table, c.max_blocks, d.num_kv_heads, d.idx_k_heads, k_new, v_new,
                       idx_new, start_pos, n_new);
  return hipGetLastError();
}

}  // namespace msa
