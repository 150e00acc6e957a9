// Index scores of one KV block for every group of a sequence (decode): the
// device building block of the index branch ("MiniMax wird dünn", section 1,
// Schritt 1: Q_idx . K_idx^T against the single shared index-key head, then
// the block max pool).
#pragma once

#include "msa_device.h"

namespace msa {

// ------------------------------------------------------------ index scores
// One wave scores KV block b of one sequence against all Hkv*NI index-query
// rows of the sequence (row = group*NI + head; 32 rows at 8 groups x 4
// heads; MT = ceil(rows / 16) MFMA tiles).  The block's index keys (B tokens
// x 128 bytes) are streamed with 1 KB wave-contiguous direct-to-LDS loads
// (global_load_lds_dwordx4, non-temporal): lane l of load i fills bytes
// i*1024 + 16*l of `stage`, i.e. token 8i + l/8 and chunk slot l%8, and reads
// the source chunk (l%8) ^ (l/8), so the LDS image is XOR-swizzled and the
// MFMA operand reads (16 tokens x one chunk per instruction) hit distinct
// banks.  The rows are the M side of v_mfma_f32_16x16x32_bf16; the 16x16
// score tiles fold into per-row running maxima and a DPP row reduction gives
// the block max of each group, which emit(g, value) receives (one lane per
// group calls it).
template <int B, int NI, int MT, class Emit>
__device__ __forceinline__ void index_block_scores(const uint16_t* __restrict__ idx_k,
                                                   int32_t page, const uint16_t* __restrict__ idx_q_s,
                                                   int num_kv_heads, uint8_t* stage, Emit emit) {
  constexpr int BYTES = B * 128;     // one block of index keys
  constexpr int NLD = BYTES / 1024;  // 1 KB wave loads per block
  constexpr int NT = B / 16;         // 16-token MFMA tiles per block
  const int lane = threadIdx.x & (kWave - 1);
  const uint8_t* src = reinterpret_cast<const uint8_t*>(idx_k) + (size_t)page * BYTES;
  const int src_off = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
#pragma unroll
  for (int i = 0; i < NLD; ++i) load_lds16_stream(src + i * 1024 + src_off, stage + i * 1024);

  // A operand: index-query rows; K split: dims ks*32 + 8*q4 .. +7, the same
  // for the keys below.
  const int R = num_kv_heads * NI;
  const int r16 = lane & 15, q4 = lane >> 4;
  // (no branches around the loads; padding rows read row R-1 and are zeroed)
  bf16x8 a[MT][2];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row = mt * 16 + r16;
    const uint16_t* p = idx_q_s + (size_t)min(row, R - 1) * 64 + q4 * 8;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a[mt][ks] = load_bf16x8(p + ks * 32);
  }
  wait_vmem();  // the LDS image and the queries are in place (one wave: no barrier)
  // nothing that reads the queries may be scheduled above the wait (a select
  // hoisted between the key loads makes the compiler wait for all of them)
  __builtin_amdgcn_sched_barrier(0);
#pragma unroll
  for (int mt = 0; mt < MT; ++mt)
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) a[mt][ks] = mt * 16 + r16 < R ? a[mt][ks] : zero_bf16x8();

  f32x4 rmax[MT];
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) rmax[mt] = f32x4{-INFINITY, -INFINITY, -INFINITY, -INFINITY};
#pragma unroll
  for (int nt = 0; nt < NT; ++nt) {
    const int t = nt * 16 + r16;  // B operand: token t
    bf16x8 kb[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = ks * 4 + q4;
      kb[ks] = __builtin_bit_cast(bf16x8,
                                  *reinterpret_cast<const u32x4*>(&stage[t * 128 + ((c ^ (t & 7)) << 4)]));
    }
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      acc = mfma16(a[mt][0], kb[0], acc);
      acc = mfma16(a[mt][1], kb[1], acc);
#pragma unroll
      for (int j = 0; j < 4; ++j) rmax[mt][j] = fmaxf(rmax[mt][j], acc[j]);
    }
  }
  // lane holds rows mt*16 + 4*q4 + j; reduce over the 16 token lanes, then
  // over the rows of each group.
#pragma unroll
  for (int mt = 0; mt < MT; ++mt) {
    const int row0 = mt * 16 + q4 * 4;
    if constexpr (NI >= 4) {
      float v = row16_max(max4(rmax[mt]));
      if constexpr (NI >= 8) v = fmaxf(v, xor_lane(v, 16));
      if constexpr (NI >= 16) v = fmaxf(v, xor_lane(v, 32));
      const int g = row0 / NI;
      if (r16 == 0 && (row0 % NI) == 0 && g < num_kv_heads) emit(g, v);
    } else {
      float v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) v[j] = row16_max(rmax[mt][j]);
      if (r16 == 0) {
        if constexpr (NI == 2) {
          const int g = row0 / 2;
          if (g < num_kv_heads) emit(g, fmaxf(v[0], v[1]));
          if (g + 1 < num_kv_heads) emit(g + 1, fmaxf(v[2], v[3]));
        } else {
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (row0 + j < num_kv_heads) emit(row0 + j, v[j]);
        }
      }
    }
  }
}

}  // namespace msa
