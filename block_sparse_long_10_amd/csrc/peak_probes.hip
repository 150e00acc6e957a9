// Measurement kernels (include/msa_probes.h): a plain HBM read stream and a
// bf16 MFMA issue loop, the practical peaks the attention path's kernels
// are compared with, and a chain of dependent loads, the latency that bounds
// the kernels made of short dependent steps.
#include "msa_device.h"
#include "msa_launch.h"

namespace msa {

constexpr uint32_t kProbeMagic = 0x9E3779B9u;

// One wave per workgroup; workgroup w reads the 16 KiB chunks w, w + grid,
// ... with sixteen 1 KiB wave loads in flight (consecutive lanes read
// consecutive 16-byte words), then the words past the last whole chunk.
__global__ __launch_bounds__(64) void read_stream_kernel(const u32x4* __restrict__ src,
                                                         size_t n16, uint32_t* __restrict__ sink) {
  constexpr int kLoads = 16;
  const size_t nchunk = n16 / (kLoads * 64);
  u32x4 acc = {0u, 0u, 0u, 0u};
  for (size_t c = blockIdx.x; c < nchunk; c += gridDim.x) {
    const u32x4* p = src + c * (kLoads * 64) + threadIdx.x;
    u32x4 v[kLoads];
#pragma unroll
    for (int u = 0; u < kLoads; ++u) v[u] = __builtin_nontemporal_load(p + u * 64);
#pragma unroll
    for (int u = 0; u < kLoads; ++u) acc ^= v[u];
  }
  for (size_t i = nchunk * (kLoads * 64) + (size_t)blockIdx.x * 64 + threadIdx.x; i < n16;
       i += (size_t)gridDim.x * 64)
    acc ^= __builtin_nontemporal_load(src + i);
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

// One lane follows `steps` links of a chain stored in next[0 .. n): p =
// next[p], so each load waits for the one before it (an entry outside
// [0, n) restarts the chain at 0, which keeps every load inside the table).
// The index is kept in a vector register, so that the loads take the vector
// memory path (the attention kernels' loads), not the scalar cache.  The
// last index reached is written to sink[0].
__global__ __launch_bounds__(64) void latency_chain_kernel(const int32_t* __restrict__ next,
                                                           int32_t n, int32_t steps, int32_t start,
                                                           int32_t* __restrict__ sink) {
  if (threadIdx.x != 0) return;
  int32_t p = start;
  for (int32_t i = 0; i < steps; ++i) {
    asm volatile("" : "+v"(p));
    p = next[p];
    if ((uint32_t)p >= (uint32_t)n) p = 0;
  }
  sink[0] = p;
}

hipError_t launch_read_stream(const void* src, size_t bytes, int32_t workgroups, uint32_t* sink,
                              hipStream_t stream) {
  hipLaunchKernelGGL(read_stream_kernel, dim3(workgroups), dim3(64), 0, stream,
                     static_cast<const u32x4*>(src), bytes / 16, sink);
  return hipGetLastError();
}

hipError_t launch_mfma_loop(int32_t iters, int32_t workgroups, float* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(workgroups), dim3(256), 0, stream, iters, sink);
  return hipGetLastError();
}

hipError_t launch_latency_chain(const int32_t* next, int32_t n, int32_t steps, int32_t start,
                                int32_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(latency_chain_kernel, dim3(1), dim3(64), 0, stream, next, n, steps, start,
                     sink);
  return hipGetLastError();
}

}  // namespace msa
