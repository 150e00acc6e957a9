// Device building blocks of the sparse branch of an MSA decode step:
//   attend_block        - softmax attention of a group's heads over one kept
//                         block, as a partial (max, sum, unnormalised output)
//                         (section 1, Schritt 2)
//   merge_partials      - log-sum-exp merge of a group's partials
#pragma once

#include "msa_device.h"
#include "timeline_marks.h"

namespace msa {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kMaxSlots = 64;  // top_k <= 64

// Cross-workgroup hand-off without a cache write-back: every value another
// workgroup reads is written with an agent-scope (sc1) store, which writes
// through to the point where the caches of all XCDs are coherent, and read
// with an agent-scope (sc1) load.  Buffer instructions carry the cache policy
// and move 16 bytes per lane (the (max, sum) pair of a head is padded to 16
// bytes; only the 16-byte buffer forms are used).
constexpr int kCachePolicySC1 = 16;
constexpr int kBufferDword3 = 0x00020000;  // raw 32-bit elements (gfx9 family)
// (The base address and size are made wave-uniform so that the descriptor
// lives in scalar registers: a descriptor in vector registers turns every
// buffer access into a loop over lanes.)
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buffer_of(const void* p, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(p);
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
  void* base = reinterpret_cast<void*>(((uint64_t)hi << 32) | lo);
  return __builtin_amdgcn_make_buffer_rsrc(base, (short)0, (int)__builtin_amdgcn_readfirstlane(bytes),
                                           kBufferDword3);
}
__device__ __forceinline__ void store_shared4(__amdgpu_buffer_rsrc_t r, uint32_t off, f32x4 v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, v), r, (int)off, 0, kCachePolicySC1);
}
__device__ __forceinline__ f32x4 load_shared4(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, kCachePolicySC1));
}

// ------------------------------------------------------- block attention
// Per-wave partials combined in LDS: (max, sum) here, the outputs in a
// region sized by the group, w_o[wave][head][kWoStride] (heads < group), which
// the caller may reuse once the partial is stored.
struct AttendShared {
  float w_m[4][16], w_l[4][16];
};
constexpr int kWoStride = 128 + 4;  // floats per (wave, head) row: conflict-free reads
__host__ __device__ constexpr size_t attend_wo_bytes(int group) {
  return (size_t)4 * group * kWoStride * sizeof(float);
}

// LDS bytes for staging V: 32 token rows of 256 bytes per wave.
constexpr size_t kAttendVStageBytes = 4 * 32 * 256;

// Swizzle of the staged V rows: 16-byte chunk c of row r is stored at chunk
// c ^ 2*vswz(r), so that the transpose reads of one instruction (rows
// r0 .. r0+3 and r0+8 .. r0+11, 32 bytes each) fall on distinct banks.
__device__ __forceinline__ int vswz(int r) { return (r & 3) | ((r >> 1) & 4); }

// Attention of the G heads of group g of sequence s over kept block blk
// (blk < 0: an empty slot) by a 256-thread workgroup: 4 waves x 32 tokens,
// S^T = K Q^T and O^T = V^T P^T on v_mfma_f32_16x16x32_bf16 (heads padded to
// 16), the per-wave partials combined in LDS.  K rows come straight from the
// token-major page as the A operand; the wave's 32 V rows are staged in LDS
// (vstage, kAttendVStageBytes) by direct loads, and V^T, the A operand of the
// PV product, is read from them with LDS transpose reads.  vstage may alias
// w_o.  V rows past the sequence's last token are zeroed in LDS: their
// probability is zero, and unwritten cache slots may hold any bits.  The
// result is stored as the partial of `slot`: o at ro[(slot*G + h)*128 ..] and
// (max, sum) at rml[(slot*G + h)*16] (16-byte records), both with agent-scope
// stores.  Probabilities enter the PV contraction as hi + lo bf16 parts
// (P - hi - lo < 2^-16 P).
template <int B>
__device__ __forceinline__ void attend_block(const uint16_t* __restrict__ kc,
                                             const uint16_t* __restrict__ vc, int32_t page,
                                             int blk, int L, const uint16_t* __restrict__ q_sg,
                                             int num_kv_heads, int g, int group, float scale_log2,
                                             int slot, __amdgpu_buffer_rsrc_t ro,
                                             __amdgpu_buffer_rsrc_t rml, AttendShared& sh,
                                             float* __restrict__ w_o, uint8_t* __restrict__ vstage) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  if (blk < 0) {  // empty slot: weight zero in the merge, output zeros
    for (int h = tid; h < group; h += 256)
      store_shared4(rml, (slot * group + h) * 16, f32x4{-INFINITY, 0.f, 0.f, 0.f});
    for (int x = tid; x < group * 32; x += 256)
      store_shared4(ro, ((slot * group + (x >> 5)) * 128 + 4 * (x & 31)) * 4,
                    f32x4{0.f, 0.f, 0.f, 0.f});
    return;
  }
  const int n_valid = min(B, L - blk * B);
  const int t0 = wave * 32;
  const int r16 = lane & 15, q4 = lane >> 4;
  float m_w = -INFINITY, l_w = 0.f;
  f32x4 o[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) o[i] = f32x4{0.f, 0.f, 0.f, 0.f};
  if (t0 < n_valid) {
    // all loads first: Q^T (B operand, head r16), K rows (A operand), V^T (A operand)
    // (no branches around the loads: a join would wait for them; padding
    // heads read head group-1 and are zeroed afterwards)
    bf16x8 qf[4], kf[2][4], vf[8];
    const uint16_t* qp = q_sg + (size_t)min(r16, group - 1) * 128 + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = load_bf16x8(qp + ks * 32);
    // S^T tiles: M row r of tile mt is token t0 + 8*(r>>2) + 4*mt + (r&3), so
    // that lane (r16, q4) ends up with tokens t0 + 8*q4 + 0..7 of head r16.
    const uint16_t* kp = kc + ((size_t)page * num_kv_heads + g) * (size_t)(B * 128);
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      const int tok = t0 + 8 * (r16 >> 2) + 4 * mt + (r16 & 3);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) kf[mt][ks] = load_bf16x8(kp + (size_t)tok * 128 + q4 * 8 + ks * 32);
    }
    // V rows t0 .. t0+31 into the wave's 8 KiB of LDS: load i fills rows
    // 4i .. 4i+3, lane l row 4i + l/16 at chunk position l%16
    uint8_t* vs = vstage + wave * 8192;
    {
      const uint8_t* vsrc = reinterpret_cast<const uint8_t*>(vc) +
                            (((size_t)page * num_kv_heads + g) * B + t0) * 256;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int row = 4 * i + (lane >> 4);
        const int c = (lane & 15) ^ (2 * vswz(row));
        load_lds16(vsrc + row * 256 + c * 16, vs + i * 1024);
      }
    }
    wait_vmem();  // K, Q and the staged V rows are in place (one wave: no barrier)
    MSA_MARK(MSA_MARK_KV_IN);
    if (t0 + 32 > n_valid) {  // rows past the last token: zero (uniform)
      for (int x = lane + 16 * (n_valid - t0); x < 32 * 16; x += kWave)
        *reinterpret_cast<u32x4*>(vs + x * 16) = u32x4{0u, 0u, 0u, 0u};
    }
    // (no LDS read may move above the stores)
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    // V^T operand of dims 16 mt .. 16 mt + 15, tokens 8 q4 .. 8 q4 + 7: lane
    // u = r16 of its 16-lane group addresses row 8 q4 + u/4 (+4), dims
    // 16 mt + 4 (u%4) .. +3, at swizzled chunk positions
    {
      const int row = 8 * q4 + (r16 >> 2);
      const uint32_t a0 = (uint32_t)(row * 256 + 32 * vswz(row) + 8 * (r16 & 3));
#pragma unroll
      for (int mt = 0; mt < 8; ++mt) {
        const uint32_t a = a0 ^ (uint32_t)(32 * mt);
        vf[mt] = join_tr(lds_read_tr16(vs + a), lds_read_tr16(vs + a + 4 * 256));
      }
    }

#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = r16 < group ? qf[ks] : zero_bf16x8();
    float z[8];
#pragma unroll
    for (int mt = 0; mt < 2; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) acc = mfma16(kf[mt][ks], qf[ks], acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int tok = t0 + 8 * q4 + 4 * mt + j;
        z[mt * 4 + j] = tok < n_valid ? acc[j] * scale_log2 : -INFINITY;
      }
    }
    float mx = z[0];
#pragma unroll
    for (int i = 1; i < 8; ++i) mx = fmaxf(mx, z[i]);
    mx = fmaxf(mx, xor_lane(mx, 16));
    mx = fmaxf(mx, xor_lane(mx, 32));
    MSA_MARK(MSA_MARK_SCORES);
    float p[8], sum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      p[i] = z[i] == -INFINITY ? 0.f : exp2f(z[i] - mx);
      sum += p[i];
    }
    sum += xor_lane(sum, 16);
    sum += xor_lane(sum, 32);
    m_w = mx;
    l_w = sum;
    MSA_MARK(MSA_MARK_SOFTMAX);
    // P^T as the B operand (keys 8*q4 + j of head r16), hi + lo bf16 parts
    uint32_t hi[8], lo[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) split_bf16(p[i], hi[i], lo[i]);
    const bf16x8 phi = __builtin_bit_cast(
        bf16x8, u32x4{pack2(hi[0], hi[1]), pack2(hi[2], hi[3]), pack2(hi[4], hi[5]), pack2(hi[6], hi[7])});
    const bf16x8 plo = __builtin_bit_cast(
        bf16x8, u32x4{pack2(lo[0], lo[1]), pack2(lo[2], lo[3]), pack2(lo[4], lo[5]), pack2(lo[6], lo[7])});
#pragma unroll
    for (int mt = 0; mt < 8; ++mt) {
      o[mt] = mfma16(vf[mt], phi, o[mt]);
      o[mt] = mfma16(vf[mt], plo, o[mt]);
    }
    MSA_MARK(MSA_MARK_PV);
  }
  // o[mt][j] = O^T[dim 16*mt + 4*q4 + j][head r16]
  if (lane < 16) {
    sh.w_m[wave][lane] = m_w;
    sh.w_l[wave][lane] = l_w;
  }
  __syncthreads();  // every wave's V reads are done before w_o (aliasing vstage) is written
  MSA_MARK(MSA_MARK_WAVES_DONE);
  if (r16 < group) {
    float* row = w_o + (wave * group + r16) * kWoStride;
#pragma unroll
    for (int mt = 0; mt < 8; ++mt)
#pragma unroll
      for (int j = 0; j < 4; ++j) row[16 * mt + 4 * q4 + j] = o[mt][j];
  }
  __syncthreads();
  MSA_MARK(MSA_MARK_COMBINED);
  // combine the waves: thread -> (head h, dims 4*d4 .. +3)
  for (int idx = tid; idx < group * 32; idx += 256) {
    const int h = idx >> 5, d4 = idx & 31;
    float M = sh.w_m[0][h];
#pragma unroll
    for (int w = 1; w < 4; ++w) M = fmaxf(M, sh.w_m[w][h]);
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    float l = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      if (sh.w_m[w][h] == -INFINITY) continue;
      const float e = exp2f(sh.w_m[w][h] - M);
      l += e * sh.w_l[w][h];
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] += e * w_o[(w * group + h) * kWoStride + 4 * d4 + j];
    }
    store_shared4(ro, ((slot * group + h) * 128 + 4 * d4) * 4, acc);
    if (d4 == 0) store_shared4(rml, (slot * group + h) * 16, f32x4{M, l, 0.f, 0.f});
  }
}

// Log-sum-exp merge of the top_k partials of one (sequence, group) into
// out_sg[h*128 ..] (256 threads).  Every thread first issues the loads of its
// (head h, dims 4*d4 .. +3) partial outputs, 16 slots at a time; meanwhile the
// weights e^(m_k - M) / sum_k e^(m_k - M) l_k of every (head, slot) are
// formed once in LDS (up to 16 slots: one lane per (head, slot), reduced
// within DPP rows), so the fold is one multiply-add per partial value.
// Empty slots carry m = -inf (weight 0) and zero outputs.
struct MergeShared {
  float m[16][kMaxSlots], l[16][kMaxSlots];
  float w[16][kMaxSlots];
};

// Weights of up to 16 slots: lane (h, k) of a DPP row of 16 (h = tid/16,
// k = tid%16) takes the (max, sum) record v of slot k, head h.
__device__ __forceinline__ void row_weights(f32x4 v, int top_k, int group, MergeShared& ms) {
  const int tid = threadIdx.x, hh = tid >> 4, k = tid & 15;
  const bool live = hh < group && k < top_k;
  const float m = live ? v[0] : -INFINITY;
  const float M = row16_max(m);
  const float e = live ? exp2f(m - M) : 0.f;  // 0 for an empty slot
  float den = e * v[1];
  den += row_ror<8>(den);
  den += row_ror<4>(den);
  den += row_ror<2>(den);
  den += row_ror<1>(den);
  if (live) ms.w[hh][k] = e / den;
}

__device__ __forceinline__ void merge_partials(__amdgpu_buffer_rsrc_t ro, __amdgpu_buffer_rsrc_t rml,
                                               int top_k, int group, float* __restrict__ out_sg,
                                               MergeShared& ms) {
  constexpr int kChunk = 16;
  const int tid = threadIdx.x;
  // item = (head h, dims 4*d4 .. +3): group*32 of them, one or two per thread
  const int items = group * 32;
  if (items <= 256 && top_k <= kChunk) {  // uniform
    // one item and one chunk per thread, in straight-line code: the weight
    // lane's (max, sum) record is loaded first and the item's partials after
    // it, so that the weights, which wait for the record only (loads complete
    // in order), are formed while the partials stream in.  Slots past top_k
    // and rows past the group read beyond the buffer range: zeros.
    const f32x4 v = load_shared4(rml, ((tid & 15) * group + (tid >> 4)) * 16);
    const int h = tid >> 5, d4 = tid & 31;
    f32x4 o[kChunk];
#pragma unroll
    for (int k = 0; k < kChunk; ++k)
      o[k] = load_shared4(ro, ((k * group + h) * 128 + 4 * d4) * 4);
    row_weights(v, top_k, group, ms);
    __syncthreads();
    if (tid >= items) return;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int k = 0; k < kChunk; ++k) {
      const float w = k < top_k ? ms.w[h][k] : 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, o[k][j], acc[j]);
    }
    *reinterpret_cast<f32x4*>(out_sg + (size_t)h * 128 + 4 * d4) = acc;
    return;
  }
  // general case (group 16, or more than 16 slots): the weights first, then
  // the partials in small chunks (so that only one chunk of registers is
  // ever live)
  if (top_k <= 16) {  // uniform
    row_weights(load_shared4(rml, ((tid & 15) * group + (tid >> 4)) * 16), top_k, group, ms);
  } else {
    for (int x = tid; x < group * top_k; x += 256) {
      const int hh = x / top_k, k = x - hh * top_k;
      const f32x4 v = load_shared4(rml, (k * group + hh) * 16);
      ms.m[hh][k] = v[0];
      ms.l[hh][k] = v[1];
    }
    __syncthreads();
    if (tid < group) {
      float M = -INFINITY;
      for (int k = 0; k < top_k; ++k) M = fmaxf(M, ms.m[tid][k]);
      float den = 0.f;
      for (int k = 0; k < top_k; ++k) {
        const float e = exp2f(ms.m[tid][k] - M);  // 0 for an empty slot
        ms.w[tid][k] = e;
        den += e * ms.l[tid][k];
      }
      const float inv = 1.f / den;
      for (int k = 0; k < top_k; ++k) ms.w[tid][k] *= inv;
    }
  }
  __syncthreads();
  constexpr int kLoopChunk = 4;
  for (int it = tid; it < items; it += 256) {
    const int h = it >> 5, d4 = it & 31;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int k0 = 0; k0 < top_k; k0 += kLoopChunk) {
      f32x4 ol[kLoopChunk];
#pragma unroll
      for (int k = 0; k < kLoopChunk; ++k)
        ol[k] = load_shared4(ro, (((k0 + k) * group + h) * 128 + 4 * d4) * 4);
#pragma unroll
      for (int k = 0; k < kLoopChunk; ++k) {
        const float w = k0 + k < top_k ? ms.w[h][k0 + k] : 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] = fmaf(w, ol[k][j], acc[j]);
      }
    }
    *reinterpret_cast<f32x4*>(out_sg + (size_t)h * 128 + 4 * d4) = acc;
  }
}

}  // namespace msa
