// Wall-clock marks of the timeline build (-DMSA_TIMELINE): the mark numbers
// are those of msa_timeline.h.  In the ordinary build every macro is empty.
//   MSA_MARK(m)        thread 0 of the watched decode attention workgroup
//                      (sequence 0, group 0, slot 1) stores the clock;
//   MSA_MARK_IF(c, m)  thread 0 of any workgroup for which c holds;
//   MSA_MARK_LATEST(m) thread 0 of every workgroup: the latest clock wins.
// Each translation unit keeps its own array (the marks are read per unit).
#pragma once

#include "msa_timeline.h"

#ifdef MSA_TIMELINE
#include <hip/hip_runtime.h>

namespace msa {

static __device__ unsigned long long timeline_marks[MSA_NUM_MARKS];

// The decode attention grid is (top_k, num_kv_heads, batch) with the
// (slot, group) index lin = x + y * top_k, group lin % num_kv_heads and slot
// lin / num_kv_heads: slot 1 of group 0 is lin = num_kv_heads = gridDim.y.
__device__ __forceinline__ bool timeline_watched() {
  return threadIdx.x == 0 && blockIdx.z == 0 && blockIdx.x + blockIdx.y * gridDim.x == gridDim.y;
}
__device__ __forceinline__ unsigned long long timeline_now() {
  return __builtin_amdgcn_s_memrealtime();
}

}  // namespace msa

#define MSA_MARK(m)                                                        \
  do {                                                                     \
    if (::msa::timeline_watched()) ::msa::timeline_marks[m] = ::msa::timeline_now(); \
  } while (0)
#define MSA_MARK_IF(c, m)                                                  \
  do {                                                                     \
    if (threadIdx.x == 0 && (c)) ::msa::timeline_marks[m] = ::msa::timeline_now(); \
  } while (0)
#define MSA_MARK_LATEST(m)                                                 \
  do {                                                                     \
    if (threadIdx.x == 0) atomicMax(&::msa::timeline_marks[m], ::msa::timeline_now()); \
  } while (0)
// Host side: copy out / clear this unit's array (synchronous copies).
#define MSA_TIMELINE_ACCESSORS(name)                                                  \
  hipError_t timeline_read_##name(unsigned long long* out) {                          \
    return hipMemcpyFromSymbol(out, HIP_SYMBOL(::msa::timeline_marks),                \
                               sizeof(unsigned long long) * MSA_NUM_MARKS);           \
  }                                                                                   \
  hipError_t timeline_clear_##name() {                                                \
    static const unsigned long long zero[MSA_NUM_MARKS] = {};                         \
    return hipMemcpyToSymbol(HIP_SYMBOL(::msa::timeline_marks), zero, sizeof zero);   \
  }

#else

#define MSA_MARK(m) ((void)0)
#define MSA_MARK_IF(c, m) ((void)0)
#define MSA_MARK_LATEST(m) ((void)0)

#endif
