// Sparse branch of MSA: exact softmax attention of every query head of a GQA
// group over the real keys/values of the group's kept blocks only
// ("MiniMax wird dünn", section 1, Schritt 2; all heads of a group share one
// selection, Q1-Q3 -> I_1, Q4-Q6 -> I_2).
//
// Both kernels compute S^T = K Q^T (keys on the MFMA M side, query rows on the
// N side) so that a query row's softmax statistics live in one lane pair, and
// O^T = V^T P^T with V^T read straight from the page layout [D][B] (8
// consecutive tokens of one dimension = one 16-byte operand).  Probabilities
// enter the bf16 PV contraction as hi + lo bf16 parts (P - hi - lo < 2^-16 P),
// so the only rounding left is fp32 accumulation.
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
// (K token-major, V^T dimension-major, XOR-swizzled 16-byte chunks) and
// consumed 32 keys at a time with v_mfma_f32_32x32x16_bf16 and an online
// softmax; the causal mask applies inside the tile's diagonal block only.
#include <algorithm>

#include "block_topk.h"
#include "chunk_map.h"
#include "decode_attend.h"
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

// ---------------------------------------------------------------- decode
// TopK of every (sequence, group): one workgroup each (large batches).
template <int B>
__global__ __launch_bounds__(256) void decode_topk_kernel(const float* __restrict__ pooled,
                                                          const int32_t* __restrict__ seq_lens,
                                                          int32_t num_kv_heads, int32_t max_blocks,
                                                          int32_t top_k, int32_t n_sink,
                                                          int32_t n_local, int32_t* __restrict__ sel) {
  __shared__ TopkShared sh;
  __shared__ int sel_s[kMaxTopK], tmp_s[kMaxTopK];
  const int g = blockIdx.x, s = blockIdx.y;
  const size_t sg = (size_t)s * num_kv_heads + g;
  block_topk_forced<false>(pooled + sg * max_blocks, (seq_lens[s] - 1) / B, top_k, n_sink, n_local, sel_s,
                    tmp_s, sh);
  for (int i = threadIdx.x; i < top_k; i += 256) sel[sg * top_k + i] = sel_s[i];
}

// Attention of the G heads of group g over one kept block (slot) of
// sequence s: 4 waves x 32 tokens, partial (max, sum, unnormalised output)
// per head combined across the waves in LDS; the last of the top_k slot
// workgroups of (s, g) merges the partials by log-sum-exp.  With FUSED_TOPK
// every slot workgroup first derives the selection from the pooled scores
// (identical in all slots) and slot 0 stores it; otherwise it reads sel.
template <int B, bool FUSED_TOPK>
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
  // dynamic LDS: the per-wave outputs of the block attention (sized by the
  // group), then the merge's scratch (the merge runs after a barrier that
  // follows the last read of the outputs)
  extern __shared__ __attribute__((aligned(16))) float dyn_lds[];
  MergeShared& msh = *reinterpret_cast<MergeShared*>(dyn_lds);

  // Workgroups are dispatched round-robin over the XCDs, each with its own
  // L2.  Taking the group from the low digits of the (slot, group) index puts
  // a group's slot workgroups on the same XCD(s), where they share one L2 copy
  // of the group's pooled scores (grid: top_k x num_kv_heads x batch).
  const int lin = blockIdx.x + blockIdx.y * gridDim.x;
  const int g = lin % num_kv_heads, slot = lin / num_kv_heads, s = blockIdx.z;
  const int tid = threadIdx.x;
  const int Hq = num_kv_heads * group;
  const int L = seq_lens[s];
  const size_t sg = (size_t)s * num_kv_heads + g;
  int blk;
  if constexpr (FUSED_TOPK) {
    block_topk_forced<false>(pooled + sg * max_blocks, (L - 1) / B, top_k, n_sink, n_local, sel_s, tmp_s,
                      tsh);
    if (slot == 0)
      for (int i = tid; i < top_k; i += 256) sel[sg * top_k + i] = sel_s[i];
    blk = sel_s[slot];
  } else {
    blk = sel[sg * top_k + slot];
  }

  // partials of (s, g): o [top_k][group][128] and (m, l, -, -) [top_k][group]
  const uint32_t o_bytes = (uint32_t)top_k * group * 128 * 4, ml_bytes = (uint32_t)top_k * group * 16;
  const __amdgpu_buffer_rsrc_t ro = buffer_of(part_o + sg * top_k * group * 128, o_bytes);
  const __amdgpu_buffer_rsrc_t rml = buffer_of(part_ml + sg * top_k * group * 4, ml_bytes);
  const int32_t page = blk >= 0 ? block_table[(size_t)s * max_blocks + blk] : 0;
  attend_block<B>(kc, vc, page, blk, L, q + ((size_t)s * Hq + (size_t)g * group) * 128,
                  num_kv_heads, g, group, scale_log2, slot, ro, rml, ash, dyn_lds);

  // hand-off: stores complete, then count this slot in; the last slot
  // workgroup reads the partials with agent-scope loads issued after its
  // increment returned
  wait_vmem();
  __syncthreads();
  if (tid == 0)
    is_last = __hip_atomic_fetch_add(&counters[sg], 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT) == (unsigned)(top_k - 1);
  __syncthreads();
  if (!is_last) return;
  merge_partials(ro, rml, top_k, group, out + ((size_t)s * Hq + (size_t)g * group) * 128, msh);
}

// Slot workgroups beyond which TopK runs in its own launch instead of being
// repeated in every slot workgroup.
constexpr int kFusedTopkMaxWorkgroups = 1024;

hipError_t launch_decode_attn(const Dims& d, const Cache& c, const uint16_t* q,
                              const int32_t* seq_lens, int32_t batch, const float* pooled,
                              float* part_o, float* part_ml, uint32_t* counters, int32_t* sel,
                              float* out, hipStream_t stream) {
  const int G = d.num_q_heads / d.num_kv_heads;
  const float sl2 = d.softmax_scale * kLog2e;
  const dim3 grid_sg(d.num_kv_heads, batch);
  const dim3 grid_attn(d.top_k, d.num_kv_heads, batch);
  const bool fused = (size_t)d.top_k * d.num_kv_heads * batch <= kFusedTopkMaxWorkgroups;
  // the dynamic LDS (block outputs, then merge scratch) is sized by the group:
  // at group 8 it is half the size of group 16's, so more workgroups fit a CU
  const size_t dyn = std::max(attend_wo_bytes(G), sizeof(MergeShared));
#define MSA_ATTN_ARGS c.k, c.v, c.block_table, c.max_blocks, q, seq_lens, pooled, sel, \
    d.num_kv_heads, G, d.top_k, d.sink_blocks, d.local_blocks, sl2, part_o, part_ml, counters, out
  if (d.block_size == 64) {
    if (fused) {
      hipLaunchKernelGGL((decode_attn_kernel<64, true>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else {
      hipLaunchKernelGGL(decode_topk_kernel<64>, grid_sg, dim3(256), 0, stream, pooled, seq_lens,
                         d.num_kv_heads, c.max_blocks, d.top_k, d.sink_blocks, d.local_blocks, sel);
      hipLaunchKernelGGL((decode_attn_kernel<64, false>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    }
  } else {
    if (fused) {
      hipLaunchKernelGGL((decode_attn_kernel<128, true>), grid_attn, dim3(256), dyn, stream, MSA_ATTN_ARGS);
    } else {
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

// A wave-uniform float moved to a scalar register.
__device__ __forceinline__ float uniform_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_readfirstlane(__builtin_bit_cast(int, v)));
}

template <int B>
__global__ __launch_bounds__(512) void prefill_attn_kernel(
    const uint16_t* __restrict__ kc, const uint16_t* __restrict__ vc,
    const int32_t* __restrict__ block_table, const uint16_t* __restrict__ q,
    const int32_t* __restrict__ sel, ChunkMap map, int32_t num_kv_heads, int32_t group,
    int32_t top_k, int32_t num_units, int32_t zr, float scale_log2, float* __restrict__ out) {
  constexpr int KBYTES = B * 256;          // K block: B rows of 256 bytes
  constexpr int VROW = 2 * B;              // V^T row: B keys
  constexpr int VCH = B / 8;               // 16-byte chunks per V^T row
  constexpr int VBYTES = 128 * VROW;
  constexpr int KI = KBYTES / 1024 / kPrefillWaves;  // 1 KB wave loads per block, K
  constexpr int VI = VBYTES / 1024 / kPrefillWaves;  // and V^T
  constexpr int VRPI = 1024 / VROW;                  // V^T rows per wave load
  // the two ring slots are separate objects, each addressed at compile time:
  // reads of one slot then provably miss the direct loads into the other,
  // and need not wait for them
  __shared__ __attribute__((aligned(1024))) uint8_t kslot0[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t kslot1[KBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot0[VBYTES];
  __shared__ __attribute__((aligned(1024))) uint8_t vslot1[VBYTES];
  __shared__ int32_t pages[64], blocks[64];

  // workgroup -> (unit, row group); unit = tile * Hkv + g
  const int wg = blockIdx.x;
  const int unit = (wg / (8 * zr)) * 8 + (wg & 7);
  const int z = (wg >> 3) % zr;
  if (unit >= num_units) return;
  const int tile = unit / num_kv_heads, g = unit % num_kv_heads;
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
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
  const float pos_min = uniform_f32(wave_min((float)pos));
  const float pos_max = uniform_f32(wave_max((float)pos));

  const uint8_t* kbase = reinterpret_cast<const uint8_t*>(kc);
  const uint8_t* vbase = reinterpret_cast<const uint8_t*>(vc);
  // Block j's K and V^T into a ring slot: a wave-uniform page base plus
  // 32-bit lane offsets, recomputed per block from an opaque copy of the lane
  // index so that no per-lane address stays live across the block loop.
  auto issue = [&](int j, uint8_t* kdst, uint8_t* vdst) {
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
      const int dd = ins * VRPI + ln / VCH;
      const int c = (ln % VCH) ^ (dd & (VCH - 1));
      load_lds16(vg + (uint32_t)(dd * VROW + c * 16), vdst + ins * 1024);
    }
  };

  f32x16 o[4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt) o[mt] = f32x16{};
  float m_run = -1e30f, l_run = 0.f;  // m_run: row max in log2 units (lagging)
  constexpr int NS = B / 32;           // 32-key steps per block
  const int m = lane & 31;

  // Row maximum of a score tile in log2 units (both lane halves of a row).
  auto tile_max = [&](const f32x16& acc) {
    float mx = acc[0];
#pragma unroll
    for (int v = 1; v < 16; ++v) mx = __builtin_fmaxf(mx, acc[v]);
    return half_swap_max(mx) * scale_log2;
  };
  // Raise the running max only when a row's max exceeds it by more than the
  // slack; the output and the sum are rescaled then (exact: both always
  // refer to the same running max).
  auto raise_max = [&](float mx) {
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
  auto probabilities = [&](const f32x16& acc, bf16x8* phi, bf16x8* plo) {
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
  auto accumulate_pv = [&](const bf16x8 (&vf)[2][4], const bf16x8* phi, const bf16x8* plo) {
#pragma unroll
    for (int s2 = 0; s2 < 2; ++s2)
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        o[mt] = mfma32(vf[s2][mt], phi[s2], o[mt]);
        o[mt] = mfma32(vf[s2][mt], plo[s2], o[mt]);
      }
  };

  // LDS byte addresses of this lane's operand rows.  K: chunk ks of key
  // 32 s + kmap(m) sits at s*8192 + (k_lane ^ 32 ks); V^T: keys 32 s + 16 s2 +
  // 8 half.. of dimension 32 mt + m sit at 32 mt VROW + (v_lane ^ 16 (4 s +
  // 2 s2)).  (The swizzles XOR only address bits 4..7, and rows are 256 or 128
  // bytes, so the XOR and the row/step/slot offsets commute.)
  const uint32_t k_lane = (uint32_t)(kmap(m) * 256 + ((half ^ kswz(kmap(m))) << 4));
  const uint32_t v_lane = (uint32_t)(m * VROW + (((m & (VCH - 1)) ^ half) << 4));

  // attention of the wave's rows over kept block j, staged in ks_ and vs_
  auto attend = [&](int j, const uint8_t* ks_, const uint8_t* vs_) {
    // (per-step addresses start from opaque copies of the lane offsets, so
    // that the compiler does not hold every step's addresses across the loop)
    auto load_k = [&](int s, bf16x8* kf) {
      uint32_t a = k_lane;
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int ks = 0; ks < 8; ++ks)
        kf[ks] = __builtin_bit_cast(
            bf16x8, *reinterpret_cast<const u32x4*>(ks_ + (a ^ (uint32_t)(ks << 5)) + s * 8192));
    };
    auto load_v = [&](int s, bf16x8 (&vf)[2][4]) {
      uint32_t a = v_lane;
      asm volatile("" : "+v"(a));
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t a2 = a ^ (uint32_t)((s * 4 + 2 * s2) << 4);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
          vf[s2][mt] = __builtin_bit_cast(
              bf16x8, *reinterpret_cast<const u32x4*>(vs_ + a2 + mt * 32 * VROW));
      }
    };
    // S^T = K Q^T of 32 keys x the wave's 32 rows
    auto scores = [&](const bf16x8* kf) {
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
      if (diag && (float)(key0 + 32 * s) > pos_max) break;  // wave sees none of these keys
      f32x16 acc = scores(kf);
      if (s + 1 < NS) load_k(s + 1, kf);
      bf16x8 vf[2][4];
      load_v(s, vf);
      if (diag && (float)(key0 + 32 * s + 31) > pos_min) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
          const int kk = 32 * s + 16 * (v >> 3) + 8 * half + (v & 7);
          if (key0 + kk > pos) acc[v] = -INFINITY;
        }
      }
      raise_max(tile_max(acc));
      bf16x8 phi[2], plo[2];
      probabilities(acc, phi, plo);
      accumulate_pv(vf, phi, plo);
    }
  };

  // Two blocks per trip, one per slot: block j + 1 streams into the other
  // slot while block j is computed; the barrier before each block also
  // closes every wave's reads of the slot the next load overwrites.
  if (nsel > 0) issue(0, kslot0, vslot0);
  for (int j = 0; j < nsel; j += 2) {
    wait_vmem();
    __syncthreads();
    if (j + 1 < nsel) issue(j + 1, kslot1, vslot1);
    attend(j, kslot0, vslot0);
    if (j + 1 >= nsel) break;
    wait_vmem();
    __syncthreads();
    if (j + 2 < nsel) issue(j + 2, kslot0, vslot0);
    attend(j + 1, kslot1, vslot1);
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
  if (B == 64)
    hipLaunchKernelGGL(prefill_attn_kernel<64>, dim3(nwg), dim3(512), 0, stream, c.k, c.v,
                       c.block_table, q, sel, map, d.num_kv_heads, G, d.top_k, units, zr, sl2,
                       out);
  else
    hipLaunchKernelGGL(prefill_attn_kernel<128>, dim3(nwg), dim3(512), 0, stream, c.k, c.v,
                       c.block_table, q, sel, map, d.num_kv_heads, G, d.top_k, units, zr, sl2,
                       out);
  return hipGetLastError();
}

}  // namespace msa
