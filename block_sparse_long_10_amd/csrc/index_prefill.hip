// Index branch of MSA, chunked prefill: per (tile, group) the tile's
// queries x index heads (up to 512 rows) are held in registers as the A side
// of v_mfma_f32_16x16x32_bf16 and every eligible key block is staged through
// LDS (XOR-swizzled 16-byte chunks, double-buffered) as the B side; the 16x16
// score tiles fold with v_max3 into one running max per lane and are reduced
// across the workgroup once per block ("MiniMax wird dünn", section 1,
// Schritt 1: Q_idx . K_idx^T, Block Max Pool; the prefill index branch still
// scans the whole context, section 3).
#include "chunk_map.h"
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// --------------------------------------------------------------- prefill
// Longest key-block range of one workgroup.
constexpr int kPrefillMaxBlocksPerSplit = 256;

// Workgroup: 4 waves x 128 row slots (8 M tiles of 16) = 512 rows of one
// (tile, group); rows are (query, index head) pairs, padding rows repeat row 0.
// Keys: blocks [b_lo, b_hi) of the tile's eligible range, one block per step,
// double-buffered in LDS (two buffers, alternated by unrolling the loop by
// two).  Each wave streams a quarter of the next block with 1 KB
// direct-to-LDS loads (lane l of a load fills token 8q + l/8, chunk slot l%8
// with source chunk (l%8) ^ (l/8): the XOR-swizzled image the MFMA B operand
// reads without bank conflicts).  Per block, each wave folds its 16x16 score
// tiles with v_max3 into four values per lane and reduces them over the wave;
// one thread combines the four wave maxima.  (The 16x16x32 shape needs 106
// VGPRs, against 163 for 32x32x16 tiles, so four workgroups fit a CU instead
// of three; the kernel is power-bound, and the smaller shape also moves fewer
// accumulator registers per flop.)
template <int B>
__global__ __launch_bounds__(256, 4) void index_score_prefill_kernel(
    const uint16_t* __restrict__ idx_k, const int32_t* __restrict__ block_table,
    const uint16_t* __restrict__ idx_q, ChunkMap map, int32_t num_kv_heads,
    int32_t num_idx_heads, int32_t idx_k_heads, int32_t max_blocks, int32_t blocks_per_split,
    float* __restrict__ pooled) {
  constexpr int BLOCK_BYTES = B * 128;             // B tokens x 64 bf16
  constexpr int WLOADS = BLOCK_BYTES / 1024 / 4;   // 1 KB loads per wave per block
  // the two key buffers are separate objects, each addressed at compile time:
  // reads of one then provably miss the direct loads into the other, and need
  // not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf0[BLOCK_BYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kbuf1[BLOCK_BYTES];
  __shared__ float wmax0[4], wmax1[4];
  // physical pages of the workgroup's key blocks, read once up front so that
  // no block-table load sits in front of each block's key loads
  __shared__ int32_t pages[kPrefillMaxBlocksPerSplit];

  const int tile = blockIdx.x, g = blockIdx.y, split = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const TileLoc loc = locate_tile(map, tile);
  const int own = loc.prior / B + loc.tile;
  const int b_lo = split * blocks_per_split;
  const int b_hi = min(b_lo + blocks_per_split, own);
  if (b_lo >= b_hi) return;
  const int q0 = loc.q0 + max(0, own * B - loc.prior);  // rows of q / idx_q
  const int q1 = loc.q0 + min(loc.chunk, (own + 1) * B - loc.prior);
  const int nrows = (q1 - q0) * num_idx_heads;

  // A operand: row slot = wave*128 + mt*16 + (lane & 15); K = 64 in 2 steps of 32.
  bf16x8 a[8][2];
  const int q4 = lane >> 4;
#pragma unroll
  for (int mt = 0; mt < 8; ++mt) {
    int r = wave * 128 + mt * 16 + (lane & 15);
    if (r >= nrows) r = 0;
    const int qi = q0 + r / num_idx_heads, h = r % num_idx_heads;
    const uint16_t* p =
        idx_q + (((size_t)qi * num_kv_heads + g) * num_idx_heads + h) * 64 + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a[mt][ks] = load_bf16x8(p + ks * 32);
  }

  const int32_t* bt = block_table + (size_t)loc.seq * map.max_blocks;
  for (int i = tid; i < b_hi - b_lo; i += 256) pages[i] = bt[b_lo + i];
  __syncthreads();
  const uint32_t src_off = (uint32_t)((lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4));
  const int wave_u = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int b, uint8_t* dst) {
    // the block's index keys: the shared head, or group g's own head
    const int page = __builtin_amdgcn_readfirstlane(pages[b - b_lo]);
    const uint8_t* src = reinterpret_cast<const uint8_t*>(idx_k) +
                         ((size_t)page * idx_k_heads + (idx_k_heads > 1 ? g : 0)) * BLOCK_BYTES;
#pragma unroll
    for (int i = 0; i < WLOADS; ++i) {
      const int q = wave_u * WLOADS + i;
      load_lds16(src + (size_t)q * 1024 + src_off, dst + q * 1024);
    }
  };

  // Scores of block b (staged in cur) folded into its pooled maximum, with
  // block b + 1 streaming into nxt meanwhile.
  auto step = [&](int b, const uint8_t* cur, uint8_t* nxt, float* wm) {
    // nxt was last read in the previous step, which ended with a barrier
    if (b + 1 < b_hi) issue(b + 1, nxt);
    f32x4 run = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
    for (int np = 0; np < B / 32; ++np) {
      bf16x8 bf[2][2];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int t = (2 * np + u) * 16 + (lane & 15);
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) {
          const int c = ks * 4 + q4;
          bf[u][ks] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(cur + t * 128 + ((c ^ (t & 7)) << 4)));
        }
      }
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        if (wave * 128 + mt * 16 >= nrows) continue;  // uniform
        f32x4 acc0 = mfma16(a[mt][0], bf[0][0], f32x4{0.f, 0.f, 0.f, 0.f});
        f32x4 acc1 = mfma16(a[mt][0], bf[1][0], f32x4{0.f, 0.f, 0.f, 0.f});
        acc0 = mfma16(a[mt][1], bf[0][1], acc0);
        acc1 = mfma16(a[mt][1], bf[1][1], acc1);
#pragma unroll
        for (int v = 0; v < 4; ++v) run[v] = fmaxf(fmaxf(run[v], acc0[v]), acc1[v]);
      }
    }
    const float m = wave_max(max4(run));
    if (lane == 0) wm[wave] = m;
    wait_vmem();  // this wave's quarter of block b + 1 has landed
    __syncthreads();
    if (tid == 0) {
      const float r = fmaxf(fmaxf(wm[0], wm[1]), fmaxf(wm[2], wm[3]));
      pooled[((size_t)tile * num_kv_heads + g) * max_blocks + b] = r;
    }
  };

  issue(b_lo, kbuf0);
  wait_vmem();
  __syncthreads();
  for (int b = b_lo; b < b_hi; b += 2) {
    step(b, kbuf0, kbuf1, wmax0);
    if (b + 1 >= b_hi) break;
    step(b + 1, kbuf1, kbuf0, wmax1);
  }}

hipError_t launch_index_score_prefill(const Dims& d, const Cache& c, const uint16_t* idx_q,
                                      const ChunkMap& map, int32_t num_tiles, int32_t max_own,
                                      float* pooled, hipStream_t stream) {
  const int B = d.block_size;
  // split the key range so that the grid holds many workgroups per CU
  const int units = num_tiles * d.num_kv_heads;
  int splits = (4096 + units - 1) / units;
  if (splits > max_own) splits = max_own > 0 ? max_own : 1;
  int per = max_own > 0 ? (max_own + splits - 1) / splits : 1;
  // cap the key range of one workgroup: with tiles of very different context
  // lengths (batched prefill) long ranges would leave a few workgroups
  // running long after the rest
  if (per > kPrefillMaxBlocksPerSplit) {
    per = kPrefillMaxBlocksPerSplit;
    splits = (max_own + per - 1) / per;
  }
  dim3 grid(num_tiles, d.num_kv_heads, splits);
  if (B == 64)
    hipLaunchKernelGGL(index_score_prefill_kernel<64>, grid, dim3(256), 0, stream, c.idx_k,
                       c.block_table, idx_q, map, d.num_kv_heads,
                       d.num_idx_heads, d.idx_k_heads, c.max_blocks, per, pooled);
  else
    hipLaunchKernelGGL(index_score_prefill_kernel<128>, grid, dim3(256), 0, stream, c.idx_k,
                       c.block_table, idx_q, map, d.num_kv_heads,
                       d.num_idx_heads, d.idx_k_heads, c.max_blocks, per, pooled);
  return hipGetLastError();
}

}  // namespace msa
