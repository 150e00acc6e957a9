// Device-side helpers shared by the MSA kernels (gfx950 / CDNA4, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace msa {

constexpr int kWave = 64;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16)+j], B[8*(l/16)+j][l%16]
// (j = 0..7) and D[4*(l/16)+j][l%16] (j = 0..3).
__device__ __forceinline__ f32x4 mfma16(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 half2 __attribute__((ext_vector_type(2)));
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
// LDS (address space 3) pointers, for addresses formed from byte offsets
typedef __attribute__((address_space(3))) const uint8_t* lds_u8;
typedef __attribute__((address_space(3))) const u32x4* lds_u32x4;

// v_mfma_f32_32x32x16_f16: the same lane layout as the bf16 form below.
__device__ __forceinline__ f32x16 mfma32_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_32x32x16_bf16: lane l holds A[l%32][8*(l/32)+j], B[8*(l/32)+j][l%32]
// and D[8*(v/4)+4*(l/32)+v%4][l%32] (v = 0..15).
__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ bf16x8 load_bf16x8(const uint16_t* p) {
  return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4*>(p));
}
// Direct global -> LDS copy of 16 bytes per lane (gfx950
// global_load_lds_dwordx4): lane l's bytes land at lds_base + 16*l; the LDS
// base must be the same for the whole wave.  Non-temporal (streamed once).
typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef __attribute__((address_space(1))) void* global_ptr_t;
constexpr int kCachePolicyNT = 2;
__device__ __forceinline__ void load_lds16_stream(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)lds_base, 16, 0, kCachePolicyNT);
}
// The same with the default cache policy (data read again by other workgroups).
__device__ __forceinline__ void load_lds16(const void* src, void* lds_base) {
  __builtin_amdgcn_global_load_lds((global_ptr_t)src, (lds_ptr_t)lds_base, 16, 0, 0);
}
// Wait for every outstanding vector-memory operation of this wave.
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0); }

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16
// lanes, lane u supplies the address of 4 consecutive 16-bit elements; lane i
// of the group receives element i%4 of the chunks addressed by lanes
// i/4, 4 + i/4, 8 + i/4 and 12 + i/4, in that order.  So if lane u = 4j + c
// addresses row r0 + j, columns c0 + 4c .. c0 + 4c + 3 of a row-major tile,
// lane i receives column c0 + i of rows r0 .. r0 + 3: the column a matrix-core
// operand needs when its K dimension runs along the rows.
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
__device__ __forceinline__ i16x4 lds_read_tr16(const void* lds_byte_addr) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_i16x4*)(__attribute__((address_space(3))) void*)(lds_byte_addr));
}
__device__ __forceinline__ i16x4 lds_read_tr16_l(lds_u8 p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}
// Two transpose reads (rows r0..r0+3, then r0+4..r0+7) as one 8-element operand.
__device__ __forceinline__ bf16x8 join_tr(i16x4 a, i16x4 b) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 v = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  return __builtin_bit_cast(bf16x8, u32x4{0u, 0u, 0u, 0u});
}

// Round-to-nearest-even float -> bfloat16 bits (inputs are finite).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
  uint32_t u = __builtin_bit_cast(uint32_t, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t h) {
  return __builtin_bit_cast(float, h << 16);
}

// Split x into hi + lo, both bfloat16, with hi = bf16(x) and lo = bf16(x - hi):
// x - (hi + lo) is below 2^-16 |x|.
__device__ __forceinline__ void split_bf16(float x, uint32_t& hi, uint32_t& lo) {
  hi = f32_to_bf16_bits(x);
  lo = f32_to_bf16_bits(x - bf16_bits_to_f32(hi));
}
__device__ __forceinline__ uint32_t pack2(uint32_t lo16, uint32_t hi16) {
  return lo16 | (hi16 << 16);
}

// DPP row rotate within 16-lane rows (row_ror:n has control 0x120 + n).
template <int N>
__device__ __forceinline__ float row_ror(float v) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, v), 0x120 + N, 0xF, 0xF, false));
}
// Max over the 16 lanes of each DPP row; every lane receives the result.
__device__ __forceinline__ float row16_max(float v) {
  v = fmaxf(v, row_ror<8>(v));
  v = fmaxf(v, row_ror<4>(v));
  v = fmaxf(v, row_ror<2>(v));
  v = fmaxf(v, row_ror<1>(v));
  return v;
}
__device__ __forceinline__ float row16_min(float v) {
  v = fminf(v, row_ror<8>(v));
  v = fminf(v, row_ror<4>(v));
  v = fminf(v, row_ror<2>(v));
  v = fminf(v, row_ror<1>(v));
  return v;
}
__device__ __forceinline__ float xor_lane(float v, int m) { return __shfl_xor(v, m, kWave); }

__device__ __forceinline__ float wave_max(float v) {
  v = row16_max(v);
  v = fmaxf(v, xor_lane(v, 16));
  return fmaxf(v, xor_lane(v, 32));
}
__device__ __forceinline__ float wave_min(float v) {
  v = row16_min(v);
  v = fminf(v, xor_lane(v, 16));
  return fminf(v, xor_lane(v, 32));
}

__device__ __forceinline__ int wave_min_i(int v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = min(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_max_i(int v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = max(v, __shfl_xor(v, m, kWave));
  return v;
}

__device__ __forceinline__ float max4(f32x4 v) { return fmaxf(fmaxf(v[0], v[1]), fmaxf(v[2], v[3])); }

}  // namespace msa
