// Measurement kernels (include/msa_probes.h): a plain HBM read stream and a
// bf16 MFMA issue loop, the practical peaks the attention path's kernels
// are compared with.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr uint32_t kProbeMagic = 0x9E3779B9u;

// Grid-stride pass over n16 16-byte words; eight loads in flight per
// iteration.  Consecutive threads read consecutive words, so one wave load
// instruction covers 1 KiB.
__global__ __launch_bounds__(256) void read_stream_kernel(const u32x4* __restrict__ src,
                                                          size_t n16, uint32_t* __restrict__ sink) {
  constexpr int kInFlight = 8;
  const size_t stride = (size_t)gridDim.x * 256;
  size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (; i + (kInFlight - 1) * stride < n16; i += kInFlight * stride) {
    u32x4 v[kInFlight];
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) v[u] = __builtin_nontemporal_load(src + i + u * stride);
#pragma unroll
    for (int u = 0; u < kInFlight; ++u) acc ^= v[u];
  }
  for (; i < n16; i += stride) acc ^= __builtin_nontemporal_load(src + i);
  const uint32_t v = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
  if (v == kProbeMagic) sink[0] = v;
}

// Four independent accumulator chains of v_mfma_f32_32x32x16_bf16 per wave.
// The operands depend on the lane (nothing folds at compile time) and are
// small (products stay exact, sums far from overflow).
__global__ __launch_bounds__(256) void mfma_loop_kernel(int32_t iters, float* __restrict__ sink) {
  const int lane = threadIdx.x & (kWave - 1);
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((lane + j) & 7) * 0.125f);
    b[j] = (__bf16)((float)((lane * 3 + j) & 7) * 0.0625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  for (int i = 0; i < iters; ++i) {
    c0 = mfma32(a, b, c0);
    c1 = mfma32(a, b, c1);
    c2 = mfma32(a, b, c2);
    c3 = mfma32(a, b, c3);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == 1.0e30f) sink[0] = s;
}

hipError_t launch_read_stream(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(256), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int32_t iters, int32_t workgroups, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

}  // namespace msa
