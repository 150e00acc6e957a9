// Sparse branch of MSA: exact softmax attention of every query head of a GQA
// group over the real keys/values of the group's kept blocks only
// ("MiniMax wird dünn", section 1, Schritt 2; all heads of a group share one
// selection, Q1-Q3 -> I_1, Q4-Q6 -> I_2).
//
// Both kernels compute S^T = K Q^T (keys on the MFMA M side, query rows on the
// N side) so that a query row's softmax statistics live in one lane pair, and
// O^T = V^T P^T.  K and V pages are token-major ([B][D] per page and head); V
// is staged in LDS and V^T, whose MFMA operand holds 8 consecutive tokens of
// one dimension, is formed by LDS transpose reads (ds_read_b64_tr_b16).
// In decode, probabilities enter the bf16 PV contraction as hi + lo bf16
// parts (P - hi - lo < 2^-16 P), so the only rounding left is fp32
// accumulation; prefill uses half precision (below).
//
// Decode: one launch after the index scores (two for large batches).  One
// workgroup per (sequence, group, kept-block slot) derives the group's
// selection (or reads it from a preceding TopK launch), attends to its block
// (4 waves x 32 tokens, v_mfma_f32_16x16x32_bf16, heads padded to 16) and
// publishes a partial (max, sum, unnormalised output); the last slot
// workgroup of each (sequence, group) to finish merges the partials by
// log-sum-exp.  No workgroup ever waits for another.
//
// Prefill: one workgroup per (tile, group, 256 query rows); rows are
// (query, head) pairs of the group.  Kept blocks are staged whole through LDS
// (K and V token-major, XOR-swizzled 16-byte chunks) and
// consumed 32 keys at a time with v_mfma_f32_32x32x16_bf16 and an online
// softmax; the causal mask applies inside the tile's diagonal block only.
// The PV product runs in IEEE half when the staged V block allows it: V is
// converted in LDS (exact for magnitudes in [2^-14, 65504]; the block is
// taken when its largest magnitude lies in [2^-8, 2^15]) and P is rounded to
// nearest-even half (11 significant bits), the row sums adding the rounded
// values; on the 1M prefill attention shape the worst row error of half P is
// 4.8e-4 in the oracle, against 3.6e-3 for bf16 P.  One MFMA per product
// instead of the hi + lo pair.  Outside the diagonal block the 32-key steps
// are software-pipelined: the scores of step s + 1 go to the matrix cores
// before the probabilities of step s are formed.  A workgroup that meets a
// block outside the half range stops, marks its first output row (a NaN in
// its first element) and a second launch of the same kernel, with the bf16
// hi + lo form throughout, redoes exactly the marked workgroups (the others
// exit after one load).
#include <algorithm>
#include <type_traits>

#include "block_topk.h"
#include "chunk_map.h"
#include "decode_attend.h"
#include "msa_device.h"
#include "msa_launch.h"
#include "timeline_marks.h"

namespace msa {

// ---------------------------------------------------------------- decode
// TopK of every (sequence, group): one workgroup each (large batches); REGS
// as in decode_attn_kernel.
template <int B, int REGS = 32>
__global__ __launch_bounds__(256) void decode_topk_kernel(const float* __restrict__ pooled,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int32_t num_kv_heads, int32_t max_blocks,
                                                          int32_t top_k, int32_t n_sink,
                                                          int32_t n_local, int32_t* __restrict__ sel) {
  __shared__ TopkShared sh;
  __shared__ int sel_s[kMaxTopK], tmp_s[kMaxTopK];
  const int g = blockIdx.x, s = blockIdx.y;
  const size_t sg = (size_t)s * num_kv_heads + g;
  block_topk_forced<false, true, REGS>(pooled + sg * max_blocks, (seq_lens[s] - 1) / B, top_k, n_sink, n_local, sel_s,
                    tmp_s, sh);
  for (int i = threadIdx.x; i < top_k; i += 256) sel[sg * top_k + i] = sel_s[i];
}

// Attention of the G heads of group g over one kept block (slot) of
// sequence s: 4 waves x 32 tokens, partial (max, sum, unnormalised output)
// per head combined across the waves in LDS; the last of the top_k slot
// workgroups of (s, g) merges the partials by log-sum-exp.  With FUSED_TOPK
// every slot workgroup first derives the selection from the pooled scores
// (the same blocks in the same slots in all of them, not necessarily
// ascending), and slot 0 stores it in ascending order once its own part is
// done; otherwise it reads sel.  REGS: the selection's scores per thread in
// registers (4 when no row is longer than 1024 blocks).
template <int B, bool FUSED_TOPK, int REGS = 32>
__global__ __launch_bounds__(256) void decode_attn_kernel(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, int32_t max_blocks, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ seq_lens, const float* __restrict__ pooled,
    int32_t* __restrict__ sel, int32_t num_kv_heads, int32_t group, int32_t top_k,
    int32_t n_sink, int32_t n_local, float scale_log2, float* __restrict__ part_o,
    float* __restrict__ part_ml, uint32_t* __restrict__ counters, float* __restrict__ out) {
  __shared__ TopkShared tsh;
  __shared__ int sel_s[kMaxTopK], tmp_s[kMaxTopK];
  __shared__ AttendShared ash;
  __shared__ int is_last;
  // dynamic LDS: the staged V rows of the block attention, then the per-wave
  // outputs (sized by the group), then the merge's scratch (each phase starts
  // after a barrier that follows the last read of the previous one)
  extern __shared__ __attribute__((aligned(16))) float dyn_lds[];
  MergeShared& msh = *reinterpret_cast<MergeShared*>(dyn_lds);

  // Workgroups are dispatched round-robin over the XCDs, each with its own
  // L2.  Taking the group from the low digits of the (slot, group) index puts
  // a group's slot workgroups on the same XCD(s), where they share one L2 copy
  // of the group's pooled scores (grid: top_k x num_kv_heads x batch).
  const int lin = blockIdx.x + blockIdx.y * gridDim.x;
  const int g = lin % num_kv_heads, slot = lin / num_kv_heads, s = blockIdx.z;
  const int tid = threadIdx.x;
  MSA_MARK(MSA_MARK_START);
  const int Hq = num_kv_heads * group;
  const int L = seq_lens[s];
  const size_t sg = (size_t)s * num_kv_heads + g;
  int blk;
  if constexpr (FUSED_TOPK) {
    block_topk_forced<false, false, REGS>(pooled + sg * max_blocks, (L - 1) / B, top_k, n_sink,
                                          n_local, sel_s, tmp_s, tsh);
    blk = sel_s[slot];
  } else {
    blk = sel[sg * top_k + slot];
  }
  MSA_MARK(MSA_MARK_BLOCK_KNOWN);

  // partials of (s, g): o [top_k][group][128] and (m, l, -, -) [top_k][group]
  const uint32_t o_bytes = (uint32_t)top_k * group * 128 * 4, ml_bytes = (uint32_t)top_k * group * 16;
  const __amdgpu_buffer_rsrc_t ro = buffer_of(part_o + sg * top_k * group * 128, o_bytes);
  const __amdgpu_buffer_rsrc_t rml = buffer_of(part_ml + sg * top_k * group * 4, ml_bytes);
  const int32_t page = blk >= 0 ? block_table[(size_t)s * max_blocks + blk] : 0;
  attend_block<B>(kc, vc, page, blk, L, q + ((size_t)s * Hq + (size_t)g * group) * 128,
                  num_kv_heads, g, group, scale_log2, slot, ro, rml, ash, dyn_lds,
                  reinterpret_cast<uint8_t*>(dyn_lds));

  MSA_MARK(MSA_MARK_STORED);
  // hand-off: stores complete, then count this slot in; the last slot
  // workgroup reads the partials with agent-scope loads issued after its
  // increment returned
  wait_vmem();
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&counters[sg], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(top_k - 1);
  __syncthreads();
  MSA_MARK(MSA_MARK_COUNTED_IN);
  // the selection output, ascending and -1 padded (wave 0 of slot 0, after
  // its partial is counted in: off the merge's path)
  auto store_selection = [&]() __attribute__((always_inline)) {
    if (tid >= kWave) return;
    const int b = tid < top_k ? sel_s[tid] : -1;
    uint32_t v = b >= 0 ? ~(uint32_t)b : 0u;
    wave_sort_desc<64>(v);
    if (tid < top_k) sel[sg * top_k + tid] = v != 0u ? (int)~v : -1;
  };
  if (!is_last) {
    if (FUSED_TOPK && slot == 0) store_selection();
    return;
  }
  merge_partials(ro, rml, top_k, group, out + ((size_t)s * Hq + (size_t)g * group) * 128, msh);
  MSA_MARK_IF(s == 0 && g == 0, MSA_MARK_MERGED);
  if (FUSED_TOPK && slot == 0) store_selection();
}

// Slot workgroups beyond which TopK runs in its own launch instead of being
// repeated in every slot workgroup.
constexpr int kFusedTopkMaxWorkgroups = 1024;

hipError_t launch_decode_attn(const Dims& d, const Cache& c, const uint16_t* q,
                              const int32_t* seq_lens, int32_t batch, int32_t max_seq_len,
                              const float* pooled, float* part_o, float* part_ml,
                              uint32_t* counters, int32_t* sel, float* out, hipStream_t stream) {
  const int G = d.num_q_heads / d.num_kv_heads;
  const float sl2 = d.softmax_scale * kLog2e;
  const dim3 grid_sg(d.num_kv_heads, batch);
  const dim3 grid_attn(d.top_k, d.num_kv_heads, batch);
  const bool fused = (size_t)d.top_k * d.num_kv_heads * batch <= kFusedTopkMaxWorkgroups;
  // rows of at most 1024 (4096) blocks: the selection with 4 (16) scores
  // per thread
  const int max_own = (max_seq_len - 1) / d.block_size;
  const bool short_rows = max_own <= kTopkThreads * 4;
  const bool mid_rows = max_own <= kTopkThreads * 16;
  // the dynamic LDS (staged V, block outputs, then merge scratch)
  const size_t dyn = std::max(std::max(attend_wo_bytes(G), sizeof(MergeShared)), kAttendVStageBytes);
#define MSA_ATTN_ARGS c.k, c.v, c.block_table, c.max_blocks, q, seq_lens, pooled, sel, \
    d.num_kv_heads, G, d.top_k, d.sink_blocks, d.local_blocks, sl2, part_o, part_ml, counters, out
  if (d.block_size == 64) {
    if (fused && short_rows) {
      hipLaunchKernelGGL((decode_attn_kernel<64, true, 4>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else if (fused) {
      hipLaunchKernelGGL((decode_attn_kernel<64, true>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else {
      if (mid_rows)
        hipLaunchKernelGGL((decode_topk_kernel<64, 16>), grid_sg, dim3(256), 0, stream, pooled,
                           seq_lens, d.num_kv_heads, c.max_blocks, d.top_k, d.sink_blocks,
                           d.local_blocks, sel);
      else
        hipLaunchKernelGGL(decode_topk_kernel<64>, grid_sg, dim3(256), 0, stream, pooled, seq_lens,
                           d.num_kv_heads, c.max_blocks, d.top_k, d.sink_blocks, d.local_blocks, sel);
      hipLaunchKernelGGL((decode_attn_kernel<64, false>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    }
  } else {
    if (fused && short_rows) {
      hipLaunchKernelGGL((decode_attn_kernel<128, true, 4>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else if (fused) {
      hipLaunchKernelGGL((decode_attn_kernel<128, true>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else {
      if (mid_rows)
        hipLaunchKernelGGL((decode_topk_kernel<128, 16>), grid_sg, dim3(256), 0, stream, pooled,
                           seq_lens, d.num_kv_heads, c.max_blocks, d.top_k, d.sink_blocks,
                           d.local_blocks, sel);
      else
        hipLaunchKernelGGL(decode_topk_kernel<128>, grid_sg, dim3(256), 0, stream, pooled, seq_lens,
                           d.num_kv_heads, c.max_blocks, d.top_k, d.sink_blocks, d.local_blocks, sel);
      hipLaunchKernelGGL((decode_attn_kernel<128, false>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    }
  }
#undef MSA_ATTN_ARGS
  return hipGetLastError();
}

// --------------------------------------------------------------- prefill
// One workgroup: 8 waves x 32 rows = 256 (query, head) rows of one (tile,
// group).  Every kept block is staged whole (K token-major, V^T
// dimension-major) in a two-slot LDS ring by direct global->LDS loads: block
// j+1 streams in while block j is computed.  Workgroups are numbered so that
// the row groups of one (tile, group) run at the same time on the same XCD and
// share its L2 for the block data.
constexpr int kPrefillWaves = 8;
constexpr int kPrefillRows = kPrefillWaves * 32;
constexpr float kRescaleSlack = 8.f;  // log2 units the running max may lag by

// Chunk swizzle of a 256-byte key row: the 16 lanes that read one 16-byte
// chunk column (keys kmap(0..15) of a 32-key sub-tile) hit 16 different
// chunk positions.
__device__ __forceinline__ int kswz(int key) {
  return (key & 3) | ((key >> 1) & 4) | ((key & 4) << 1);
}
// Row m of a 32-key S^T tile holds key kmap(m): then value v of lane half h
// is key 16*(v/8) + 8*h + v%8, i.e. each lane's 16 scores are two runs of 8
// consecutive keys, exactly the P^T operand layout of the PV product.
__device__ __forceinline__ int kmap(int m) {
  return 16 * (m >> 4) + 8 * ((m >> 2) & 1) + 4 * ((m >> 3) & 1) + (m & 3);
}
// A value and its counterpart 32 lanes away (the other half of the same row):
// v_permlane32_swap exchanges the upper half of one register with the lower
// half of another, so with both holding v the two results are v and its
// counterpart, in some order.  (Written as asm: the builtin's two results are
// merged into one when both inputs are the same value.)
__device__ __forceinline__ void half_swap(float v, float& a, float& b) {
  a = v;
  b = v;
  asm volatile("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
}
__device__ __forceinline__ float half_swap_max(float v) {
  float a, b;
  half_swap(v, a, b);
  return __builtin_fmaxf(a, b);
}
__device__ __forceinline__ float half_swap_sum(float v) {
  float a, b;
  half_swap(v, a, b);
  return a + b;
}
// bf16 pair from the upper halves of two floats (truncation).
__device__ __forceinline__ uint32_t upper_pair(float a, float b) {
  return (__builtin_bit_cast(uint32_t, b) & 0xFFFF0000u) | (__builtin_bit_cast(uint32_t, a) >> 16);
}
__device__ __forceinline__ float truncated_rest(float a) {
  return a - __builtin_bit_cast(float, __builtin_bit_cast(uint32_t, a) & 0xFFFF0000u);
}


template <int B, bool HALF>
__global__ __launch_bounds__(512) void prefill_attn_kernel(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ sel, ChunkMap map, int32_t num_kv_heads, int32_t group,
    int32_t top_k, int32_t num_units, int32_t zr, float scale_log2, float* __restrict__ out) {
  constexpr int KBYTES = B * 256;          // K block: B rows of 256 bytes
  constexpr int VBYTES = B * 256;          // V block: B rows of 256 bytes
  constexpr int KI = KBYTES / 1024 / kPrefillWaves;  // 1 KB wave loads per block, K
  constexpr int VI = VBYTES / 1024 / kPrefillWaves;  // and V
  // the two ring slots are separate objects, each addressed at compile time:
  // reads of one slot then provably miss the direct loads into the other,
  // and need not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t kslot0[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot1[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot0[VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot1[VBYTES];
  // (the small arrays first in LDS, at addresses an instruction offset reaches)
  __shared__ __attribute__((aligned(2048))) struct {
    int32_t pages[64], blocks[64];
    uint32_t vmax_w[kPrefillWaves];
  } sm;
  int32_t* const pages = sm.pages;
  int32_t* const blocks = sm.blocks;
  uint32_t* const vmax_w = sm.vmax_w;

  // workgroup -> (unit, row group); unit = tile * Hkv + g
  const int wg = blockIdx.x;
  const int unit = (wg / (8 * zr)) * 8 + (wg & 7);
  const int z = (wg >> 3) % zr;
  if (unit >= num_units) return;
  const int tile = unit / num_kv_heads, g = unit % num_kv_heads;
  const int tid = threadIdx.x, lane = tid & (kWave - 1);
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);  // (uniform: scalar)
  const TileLoc loc = locate_tile(map, tile);
  const int prior_len = loc.prior;
  const int own = prior_len / B + loc.tile;
  const int q0 = max(0, own * B - prior_len);  // chunk-local query range of the tile
  const int q1 = min(loc.chunk, (own + 1) * B - prior_len);
  const int nq = q1 - q0;
  const int nrows = nq * group;
  const int row0 = z * kPrefillRows;
  if (row0 >= nrows) return;
  const int Hq = num_kv_heads * group;
  // the first element of the workgroup's first output row: the mark of a
  // workgroup the half-precision launch left to the bf16 one
  float* const mark =
      out + ((size_t)(loc.q0 + q0 + row0 % nq) * Hq + (size_t)g * group + row0 / nq) * 128;
  if constexpr (!HALF) {
    if (!__builtin_isnan(*mark)) return;  // (uniform) done by the half-precision launch
  }

  const int32_t* srow = sel + (size_t)unit * top_k;
  int blk_t = -1;
  if (tid < top_k) {
    blk_t = srow[tid];
    pages[tid] = blk_t >= 0 ? block_table[(size_t)loc.seq * map.max_blocks + blk_t] : 0;
    blocks[tid] = blk_t;
  }
  const int nsel = __syncthreads_count(tid < top_k && blk_t >= 0);

  // this lane's row (N side of S^T): (query, head) = (q0 + r % nq, r / nq)
  const int half = lane >> 5;
  int r = row0 + wave * 32 + (lane & 31);
  const bool row_ok = r < nrows;
  if (!row_ok) r = 0;
  const int qi = q0 + r % nq, hh = r / nq;
  const int pos = prior_len + qi;
  bf16x8 qf[8];
  {
    const uint16_t* qp =
        q + ((size_t)(loc.q0 + qi) * Hq + (size_t)g * group + hh) * 128 + half * 8;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) qf[ks] = load_bf16x8(qp + ks * 16);
  }
  // the wave's query positions, for the causal diagonal block (wave-uniform:
  // held in scalar registers)
  const int pos_min = __builtin_amdgcn_readfirstlane(wave_min_i(pos));
  const int pos_max = __builtin_amdgcn_readfirstlane(wave_max_i(pos));
  // tokens of the diagonal block past the sequence's end (the last tile's):
  // their V rows are zeroed in LDS after staging, since unwritten cache slots
  // may hold any bits and a zero probability times NaN is NaN
  const int seq_end = prior_len + loc.chunk;
  const int diag_valid = min(B, seq_end - own * B);

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc);
  // Block j's K and V^T into a ring slot: a wave-uniform page base plus
  // 32-bit lane offsets, recomputed per block from an opaque copy of the lane
  // index so that no per-lane address stays live across the block loop.
  auto issue = [&](int j, uint8_t* kdst, uint8_t* vdst) __attribute__((always_inline)) {
    const size_t ph = (size_t)__builtin_amdgcn_readfirstlane(pages[j]) * num_kv_heads + g;
    const uint8_t* kg = kbase + ph * KBYTES;
    const uint8_t* vg = vbase + ph * VBYTES;
    int ln = lane;
    asm volatile("" : "+v"(ln));
#pragma unroll
    for (int i = 0; i < KI; ++i) {
      const int ins = wave * KI + i;
      const int key = ins * 4 + (ln >> 4);
      const int c = (ln & 15) ^ kswz(key);
      load_lds16(kg + (uint32_t)(key * 256 + c * 16), kdst + ins * 1024);
    }
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      const int ins = wave * VI + i;
      const int key = ins * 4 + (ln >> 4);
      const int c = (ln & 15) ^ (4 * (key & 3));
      load_lds16(vg + (uint32_t)(key * 256 + c * 16), vdst + ins * 1024);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;  // m_run: row max in log2 units (lagging)
  constexpr int NS = B / 32;           // 32-key steps per block
  const int m = lane & 31;

  // Row maximum of a score tile in log2 units (both lane halves of a row).
  auto tile_max = [&](const f32x16& acc) __attribute__((always_inline)) {
    float mx = acc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = __builtin_fmaxf(mx, acc[v]);
    return half_swap_max(mx) * scale_log2;
  };
  // Raise the running max only when a row's max exceeds it by more than the
  // slack; the output and the sum are rescaled then (exact: both always
  // refer to the same running max).
  auto raise_max = [&](float mx) __attribute__((always_inline)) {
    if (__ballot(mx > m_run + kRescaleSlack) != 0) {
      const float m_new = fmaxf(m_run, mx);
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      l_run *= alpha;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int v = 0; v < 16; ++v) o[mt][v] *= alpha;
      m_run = m_new;
    }
  };
  // P = exp2(S scale - m) of a score tile, added to the row sum and split into
  // bfloat16 hi + lo, hi the truncation of P: P - hi - lo < 2^-16 P.
  auto probabilities = [&](const f32x16& acc, bf16x8* phi, bf16x8* plo) __attribute__((always_inline)) {
    float p[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      p[v] = __builtin_amdgcn_exp2f(fmaf(acc[v], scale_log2, -m_run));
      l_run += p[v];
    }
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      const float* pp = p + 8 * s2;
      phi[s2] = __builtin_bit_cast(
          bf16x8, u32x4{upper_pair(pp[0], pp[1]), upper_pair(pp[2], pp[3]),
                        upper_pair(pp[4], pp[5]), upper_pair(pp[6], pp[7])});
      plo[s2] = __builtin_bit_cast(
          bf16x8, u32x4{upper_pair(truncated_rest(pp[0]), truncated_rest(pp[1])),
                        upper_pair(truncated_rest(pp[2]), truncated_rest(pp[3])),
                        upper_pair(truncated_rest(pp[4]), truncated_rest(pp[5])),
                        upper_pair(truncated_rest(pp[6]), truncated_rest(pp[7]))});
    }
  };
  // O^T += V^T P^T over 32 keys (two K steps of 16), hi and lo parts.
  auto accumulate_pv = [&](const bf16x8 (&vf)[2][4], const bf16x8* phi, const bf16x8* plo) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        o[mt] = mfma32(vf[s2][mt], phi[s2], o[mt]);
        o[mt] = mfma32(vf[s2][mt], plo[s2], o[mt]);
      }
  };
  // The same in half precision: P rounded to nearest-even half, one product;
  // the row sum adds the rounded values (v_dot2 with ones), so that numerator
  // and denominator weigh each key alike.
  auto probabilities_h = [&](const f32x16& acc, f16x8* ph) __attribute__((always_inline)) {
    const half2 ones = {(_Float16)1.f, (_Float16)1.f};
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2) {
      half2 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __builtin_amdgcn_exp2f(fmaf(acc[8 * s2 + 2 * e], scale_log2, -m_run));
        const float b = __builtin_amdgcn_exp2f(fmaf(acc[8 * s2 + 2 * e + 1], scale_log2, -m_run));
        h[e] = half2{(_Float16)a, (_Float16)b};
        l_run = __builtin_amdgcn_fdot2(h[e], ones, l_run, false);
      }
      ph[s2] = f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    }
  };
  auto accumulate_pv_h = [&](const f16x8 (&vf)[2][4], const f16x8* ph) __attribute__((always_inline)) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) o[mt] = mfma32_f16(vf[s2][mt], ph[s2], o[mt]);
  };

  // LDS byte addresses of this lane's operand rows.  K: chunk ks of key
  // 32 s + kmap(m) sits at s*8192 + (k_lane ^ 32 ks).  V (16-byte chunk c of
  // key row r stored at chunk c ^ 4(r%4)): the V^T operand of dimensions
  // 32 mt .. 32 mt + 31 and keys 32 s + 16 s2 + 8 half .. +7 is two transpose
  // reads, in which lane u = lane%16 of 16-lane group h4 = lane/16 addresses key
  // row 32 s + 16 s2 + 8 (h4/2) + u/4 (+4 for the second read), dimensions
  // 32 mt + 16 (h4%2) + 4 (u%4) .. +3: at (v_lane + (32 s + 16 s2) 256) ^ 64 mt.
  // (The swizzles XOR only address bits 4..7 and rows are 256 bytes, so the
  // XOR and the row/step offsets commute.)
  const uint32_t k_lane = (uint32_t)(kmap(m) * 256 + ((half ^ kswz(kmap(m))) << 4));
  const int u16 = lane & 15, h4 = lane >> 4;
  const uint32_t v_lane = (uint32_t)((8 * (h4 >> 1) + (u16 >> 2)) * 256 + 64 * (u16 >> 2) +
                                     32 * (h4 & 1) + 8 * (u16 & 3));

  // attention of the wave's rows over kept block j, staged in ks_ and vs_
  // (V in half precision when VHALF; two copies of the step loop, so that each
  // keeps its own registers)
  auto attend = [&](int j, const uint8_t* ks_, const uint8_t* vs_, auto vhalf_tag) __attribute__((always_inline)) {
    constexpr bool VHALF = decltype(vhalf_tag)::value;
    // (per-step addresses start from opaque copies of the lane offsets, so
    // that the compiler does not hold every step's addresses across the loop)
    auto load_k = [&](int s, bf16x8* kf) __attribute__((always_inline)) {
      uint32_t a = k_lane;
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kf[ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(ks_ + (a ^ (uint32_t)(ks << 5)) + s * 8192));
    };
    auto load_v = [&](int s, bf16x8 (&vf)[2][4]) __attribute__((always_inline)) {
      uint32_t a = v_lane;
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t a2 = a + (uint32_t)((32 * s + 16 * s2) * 256);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const uint32_t am = a2 ^ (uint32_t)(64 * mt);
          vf[s2][mt] = join_tr(lds_read_tr16(vs_ + am), lds_read_tr16(vs_ + am + 4 * 256));
        }
      }
    };
    // S^T = K Q^T of 32 keys x the wave's 32 rows
    auto scores = [&](const bf16x8* kf) __attribute__((always_inline)) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) acc = mfma32(kf[ks], qf[ks], acc);
      return acc;
    };
    // on the diagonal block the causal mask applies, and 32-key steps past
    // the wave's last query are skipped
    const bool diag = __builtin_amdgcn_readfirstlane(blocks[j]) == own;
    const int key0 = own * B;
    bf16x8 kf[8];
    load_k(0, kf);
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      if (diag && key0 + 32 * s > pos_max) break;  // wave sees none of these keys
      f32x16 acc = scores(kf);
      if (s + 1 < NS) load_k(s + 1, kf);
      bf16x8 vf[2][4];
      load_v(s, vf);
      if (diag && key0 + 32 * s + 31 > pos_min) {
        // value v holds key key0 + 32 s + 16 (v / 8) + 8 half + v % 8
        int lim = pos - key0 - 32 * s - 8 * half;
        asm volatile("" : "+v"(lim));  // (nothing of this hoisted out of the block loop)
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if (16 * (v >> 3) + (v & 7) > lim) acc[v] = -INFINITY;
      }
      raise_max(tile_max(acc));
      if constexpr (VHALF) {
        f16x8 vh[2][4], ph[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
          for (int mt = 0; mt < 4; ++mt) vh[s2][mt] = __builtin_bit_cast(f16x8, vf[s2][mt]);
        probabilities_h(acc, ph);
        accumulate_pv_h(vh, ph);
      } else {
        bf16x8 phi[2], plo[2];
        probabilities(acc, phi, plo);
        accumulate_pv(vf, phi, plo);
      }
    }
  };

  // Attention of the wave's rows over a staged non-diagonal block in half
  // precision, software-pipelined: the scores of step s + 1 are issued before
  // the probabilities of step s are formed, so that the matrix cores work on
  // them while the vector unit computes exponentials.  Lane addresses are
  // formed once per block (LDS byte addresses, opaque to the compiler, with
  // every step's displacement an instruction offset).
  auto attend_pipe = [&](const uint8_t* ks_, const uint8_t* vs_, auto&& after_prologue) __attribute__((always_inline)) {
    // (from opaque copies of the lane offsets, so that nothing is hoisted
    // out of the block loop to stay live across it)
    uint32_t kl = k_lane, vl = v_lane;
    asm volatile("" : "+v"(kl), "+v"(vl));
    auto load_k = [&](int s, bf16x8* kf) __attribute__((always_inline)) {
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kf[ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(ks_ + (kl ^ (uint32_t)(ks << 5)) + s * 8192));
    };
    // V^T operands of keys 32 s + 16 s2 .. +15 (all four dimension tiles)
    auto load_v = [&](int s, int s2, f16x8* vf) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const uint8_t* a = vs_ + (vl ^ (uint32_t)(64 * mt)) + (32 * s + 16 * s2) * 256;
        vf[mt] = __builtin_bit_cast(f16x8, join_tr(lds_read_tr16(a), lds_read_tr16(a + 1024)));
      }
    };
    auto scores = [&](const bf16x8* kf) __attribute__((always_inline)) {
      f32x16 acc = {};
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) acc = mfma32(kf[ks], qf[ks], acc);
      return acc;
    };
    // half-precision P of keys 32 s + 16 s2 .. +15 (values 8 s2 .. 8 s2 + 7
    // of the score tile), added to the row sum as rounded
    auto probs = [&](const f32x16& acc, int s2) __attribute__((always_inline)) {
      const half2 ones = {(_Float16)1.f, (_Float16)1.f};
      half2 h[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = __builtin_amdgcn_exp2f(fmaf(acc[8 * s2 + 2 * e], scale_log2, -m_run));
        const float b = __builtin_amdgcn_exp2f(fmaf(acc[8 * s2 + 2 * e + 1], scale_log2, -m_run));
        h[e] = half2{(_Float16)a, (_Float16)b};
        l_run = __builtin_amdgcn_fdot2(h[e], ones, l_run, false);
      }
      return f16x8{h[0][0], h[0][1], h[1][0], h[1][1], h[2][0], h[2][1], h[3][0], h[3][1]};
    };
    auto pv = [&](const f16x8* vf, f16x8 ph) __attribute__((always_inline)) {
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) o[mt] = mfma32_f16(vf[mt], ph, o[mt]);
    };
    bf16x8 kf[8];
    load_k(0, kf);
    f32x16 acc = scores(kf);
    load_k(1, kf);
    after_prologue();  // (the next block's loads, issued behind the first scores)
    raise_max(tile_max(acc));
    // Each step below is one scheduling region (the rescale branch closes
    // it), laid out in three phases fenced from each other, each spreading
    // one kind of work between the matrix products of another:
    //   1. scores of step s + 1 (8 products) | P of keys 0..15 of step s,
    //      V^T operands of those keys
    //   2. PV of keys 0..15 (4 products) | P of keys 16..31, their V^T
    //      operands
    //   3. PV of keys 16..31 (4 products) | K operands of step s + 2, row
    //      maxima of step s + 1
    // (K operands are loaded only once the scores of step s are dead, which
    // keeps the register peak under the 256 of two waves per SIMD.)
#pragma unroll
    for (int s = 0; s < NS; ++s) {
      f16x8 vf0[4], vf1[4];
      f32x16 accn;
      // phase 1
      load_v(s, 0, vf0);
      if (s + 1 < NS) accn = scores(kf);
      const f16x8 ph0 = probs(acc, 0);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // matrix product
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // LDS read
        __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // vector ALU
      }
      __builtin_amdgcn_sched_barrier(0);
      // phase 2
      load_v(s, 1, vf1);
      pv(vf0, ph0);
      const f16x8 ph1 = probs(acc, 1);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 1);
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        __builtin_amdgcn_sched_group_barrier(0x002, 6, 1);
      }
      __builtin_amdgcn_sched_barrier(0);
      // phase 3
      if (s + 2 < NS) load_k(s + 2, kf);
      pv(vf1, ph1);
      if (s + 1 < NS) {
        const float mx = tile_max(accn);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 2);
          __builtin_amdgcn_sched_group_barrier(0x100, 2, 2);
          __builtin_amdgcn_sched_group_barrier(0x002, 4, 2);
        }
        __builtin_amdgcn_sched_barrier(0);
        acc = accn;
        raise_max(mx);
      }
    }
  };

  // Half-precision V for block j staged in vs_, converted by the wave that
  // loaded each piece (a wave's direct loads have landed once its own vector
  // memory count is zero, so no barrier is needed first): rows past the
  // sequence's end (the last tile's diagonal block) are zeroed, then the
  // block's largest |v| (bf16 magnitude bits, ordered as integers) decides for
  // the whole workgroup after the one barrier, which also publishes the
  // converted block.  When it lies in [2^-8, 2^15] every value converts to
  // half exactly or (below 2^-14) to within 2^-25; otherwise the workgroup
  // leaves the tile to the bf16 launch, which stages its own copy.
  auto convert_own = [&](int j, uint8_t* vs_) __attribute__((always_inline)) {
    int ln = lane;  // (opaque: nothing lane-indexed is held across the block loop)
    asm volatile("" : "+v"(ln));
    if (diag_valid < B && __builtin_amdgcn_readfirstlane(blocks[j]) == own) {  // rare
#pragma unroll
      for (int i = 0; i < VI; ++i) {
        const int ins = wave * VI + i;
        if (ins * 4 + (ln >> 4) >= diag_valid)
          *reinterpret_cast<u32x4*>(vs_ + ins * 1024 + ln * 16) = u32x4{0u, 0u, 0u, 0u};
      }
    }
    u32x4 r[VI];
#pragma unroll
    for (int i = 0; i < VI; ++i)
      r[i] = *reinterpret_cast<const u32x4*>(vs_ + (wave * VI + i) * 1024 + ln * 16);
    u16x2 mx2 = {0, 0};  // largest magnitude bits of each half-word
#pragma unroll
    for (int i = 0; i < VI; ++i) {
      u32x4 h;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        mx2 = __builtin_elementwise_max(mx2, __builtin_bit_cast(u16x2, r[i][e] & 0x7FFF7FFFu));
        const half2 v = {(_Float16)__builtin_bit_cast(float, r[i][e] << 16),
                         (_Float16)__builtin_bit_cast(float, r[i][e] & 0xFFFF0000u)};
        h[e] = __builtin_bit_cast(uint32_t, v);
      }
      *reinterpret_cast<u32x4*>(vs_ + (wave * VI + i) * 1024 + ln * 16) = h;
    }
    const uint32_t mx = wave_umax(umax_(mx2[0], mx2[1]));
    if (lane == 0) vmax_w[wave] = mx;
    __syncthreads();
    uint32_t bm = vmax_w[0];
#pragma unroll
    for (int w = 1; w < kPrefillWaves; ++w) bm = umax_(bm, vmax_w[w]);
    return bm >= 0x3B80u && bm <= 0x4700u;  // |v| in [2^-8, 2^15]
  };

  // V rows of the staged diagonal block past the sequence's end are zeroed
  // (only the last tile's diagonal block has any; uniform).
  auto zero_tail = [&](int j, uint8_t* vs_) __attribute__((always_inline)) {
    if (diag_valid < B && __builtin_amdgcn_readfirstlane(blocks[j]) == own) {
      for (int x = tid + 16 * diag_valid; x < B * 16; x += 512)
        *reinterpret_cast<u32x4*>(vs_ + x * 16) = u32x4{0u, 0u, 0u, 0u};
      __syncthreads();
    }
  };

  // Two blocks per trip, one per slot: block j + 1 streams into the other
  // slot while block j is computed; the barrier before each block (in the
  // half-precision form, the one inside convert_own) also closes every
  // wave's reads of the slot the next load overwrites, whose loads are
  // issued after it.
  // The half-precision launch stops at a block outside the half range: the
  // direct loads in flight land first, then the mark (uniform).
  auto give_up = [&]() __attribute__((always_inline)) {
    wait_vmem();
    if (tid == 0) *mark = __builtin_nanf("");
  };
  if (nsel > 0) issue(0, kslot0, vslot0);
  if constexpr (HALF) {
    // the diagonal block (causal mask, steps past the wave's last query
    // skipped) takes the plain step loop
    auto attend_h = [&](int j, const uint8_t* ks_, const uint8_t* vs_, auto&& nxt) __attribute__((always_inline)) {
      if (__builtin_amdgcn_readfirstlane(blocks[j]) == own) {
        nxt();
        attend(j, ks_, vs_, std::true_type{});
      } else {
        attend_pipe(ks_, vs_, nxt);
      }
    };
    for (int j = 0; j < nsel; j += 2) {
      wait_vmem();
      if (!convert_own(j, vslot0)) return give_up();
      attend_h(j, kslot0, vslot0, [&]() { if (j + 1 < nsel) issue(j + 1, kslot1, vslot1); });
      if (j + 1 >= nsel) break;
      wait_vmem();
      if (!convert_own(j + 1, vslot1)) return give_up();
      attend_h(j + 1, kslot1, vslot1, [&]() { if (j + 2 < nsel) issue(j + 2, kslot0, vslot0); });
    }
  } else {
    for (int j = 0; j < nsel; j += 2) {
      wait_vmem();
      __syncthreads();
      zero_tail(j, vslot0);
      if (j + 1 < nsel) issue(j + 1, kslot1, vslot1);
      attend(j, kslot0, vslot0, std::false_type{});
      if (j + 1 >= nsel) break;
      wait_vmem();
      __syncthreads();
      zero_tail(j + 1, vslot1);
      if (j + 2 < nsel) issue(j + 2, kslot0, vslot0);
      attend(j + 1, kslot1, vslot1, std::false_type{});
    }
  }
  const float l_row = half_swap_sum(l_run);
  if (!row_ok) return;
  const float inv = 1.f / l_row;
  float* op = out + ((size_t)(loc.q0 + qi) * Hq + (size_t)g * group + hh) * 128;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int v4 = 0; v4 < 4; ++v4) {
      const int d0 = mt * 32 + 8 * v4 + 4 * half;
      *reinterpret_cast<f32x4*>(op + d0) =
          f32x4{o[mt][4 * v4] * inv, o[mt][4 * v4 + 1] * inv, o[mt][4 * v4 + 2] * inv,
                o[mt][4 * v4 + 3] * inv};
    }
}

hipError_t launch_sparse_attn_prefill(const Dims& d, const Cache& c, const uint16_t* q,
                                      const ChunkMap& map, int32_t num_tiles, const int32_t* sel,
                                      float* out, hipStream_t stream) {
  const int B = d.block_size;
  const int G = d.num_q_heads / d.num_kv_heads;
  const int units = num_tiles * d.num_kv_heads;
  const int zr = (B * G + kPrefillRows - 1) / kPrefillRows;
  const int nwg = (units + 7) / 8 * 8 * zr;
  const float sl2 = d.softmax_scale * kLog2e;
  // half-precision PV first; then the bf16 form for the workgroups it marked
#define MSA_PREFILL_ATTN(BB, H)                                                                 \
  hipLaunchKernelGGL((prefill_attn_kernel<BB, H>), dim3(nwg), dim3(512), 0, stream, c.k, c.v,  \
                     c.block_table, q, sel, map, d.num_kv_heads, G, d.top_k, units, zr, sl2, out)
  if (B == 64) {
    MSA_PREFILL_ATTN(64, true);
    MSA_PREFILL_ATTN(64, false);
  } else {
    MSA_PREFILL_ATTN(128, true);
    MSA_PREFILL_ATTN(128, false);
  }
#undef MSA_PREFILL_ATTN
  return hipGetLastError();
}

#ifdef MSA_TIMELINE
MSA_TIMELINE_ACCESSORS(attn)
#endif

}  // namespace msa
