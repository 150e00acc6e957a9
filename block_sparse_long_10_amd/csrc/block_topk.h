// Block TopK: the k best blocks of one (sequence or tile, group) by pooled
// index score, ranked by (score descending, block index ascending), with the
// own block always kept ("TopK" of the index branch in "MiniMax wird dünn",
// section 1, Schritt 1).
//
// One 256-thread workgroup selects from scores[0 .. own) in global memory:
//   1. range [lo, hi] of the scores (wave DPP reductions + LDS);
//   2. LDS histogram of 256 value bins over [lo, hi]; bin(v) is monotone
//      non-increasing in v, so every item of a lower bin outranks every item
//      of a higher bin;
//   3. a wave scan finds the bin b* holding the last needed item; items of
//      lower bins are kept, the items of b* are ranked exactly (score, index)
//      when they fit in LDS, otherwise [lo, hi] narrows to b*'s range and the
//      histogram repeats;
//   4. when the live range holds a single value, the lowest indices win
//      (ballot prefix counts in index order).
// The result (sorted ascending, own block included, -1 padded) lands in LDS.
#pragma once

#include "msa_device.h"

namespace msa {

constexpr int kTopkThreads = 256;
constexpr int kTopkBins = 256;
constexpr int kTopkCap = 256;
constexpr int kMaxTopK = 64;

struct TopkShared {
  unsigned hist[kTopkBins];
  float cand_v[kTopkCap];
  int cand_i[kTopkCap];
  int chosen[kMaxTopK];
  float red_a[kTopkThreads / kWave];
  float red_b[kTopkThreads / kWave];
  int wave_cnt[kTopkThreads / kWave];
  int n_chosen;
  int n_cand;
  int bstar;
  int c_lt;
  int c_eq;
};

__device__ __forceinline__ void push_chosen(TopkShared& sh, int i) {
  const int p = atomicAdd(&sh.n_chosen, 1);
  if (p < kMaxTopK) sh.chosen[p] = i;
}

__device__ __forceinline__ int topk_bin(float v, double hi, double scale) {
  double d = (hi - (double)v) * scale;
  return d >= (double)(kTopkBins - 1) ? kTopkBins - 1 : (int)d;
}

// Range of the live items (lo <= v <= hi, optionally restricted to one bin).
__device__ __forceinline__ void topk_range(const float* __restrict__ scores, int n, float lo,
                                           float hi, bool use_bin, double dhi, double scale,
                                           int bin, TopkShared& sh, float& out_lo, float& out_hi) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  float mx = -INFINITY, mn = INFINITY;
  for (int i = tid; i < n; i += kTopkThreads) {
    float v = scores[i];
    bool live = v >= lo && v <= hi;
    if (use_bin && live) live = topk_bin(v, dhi, scale) == bin;
    if (live) {
      mx = fmaxf(mx, v);
      mn = fminf(mn, v);
    }
  }
  mx = wave_max(mx);
  mn = wave_min(mn);
  if (lane == 0) {
    sh.red_a[wave] = mx;
    sh.red_b[wave] = mn;
  }
  __syncthreads();
  mx = sh.red_a[0];
  mn = sh.red_b[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / kWave; ++w) {
    mx = fmaxf(mx, sh.red_a[w]);
    mn = fminf(mn, sh.red_b[w]);
  }
  __syncthreads();
  out_lo = mn;
  out_hi = mx;
}

// Keep the `need` lowest indices among items equal to `val`.
__device__ __forceinline__ void topk_lowest_equal(const float* __restrict__ scores, int n,
                                                  float val, int need, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  int done = 0;
  for (int c0 = 0; c0 < n && done < need; c0 += kTopkThreads) {
    const int i = c0 + tid;
    const bool f = i < n && scores[i] == val;
    const unsigned long long m = __ballot(f);
    const int in_wave = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) sh.wave_cnt[wave] = __popcll(m);
    __syncthreads();
    int before = done, total = 0;
#pragma unroll
    for (int w = 0; w < kTopkThreads / kWave; ++w) {
      const int c = sh.wave_cnt[w];
      if (w < wave) before += c;
      total += c;
    }
    if (f && before + in_wave < need) push_chosen(sh, i);
    __syncthreads();
    done += total;
  }
}

// All threads of the workgroup call this with identical arguments.
// out_sel (LDS, k entries) receives the kept blocks, ascending, -1 padded.
__device__ void block_topk(const float* __restrict__ scores, int own, int k, int* out_sel,
                           TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int keep = min(k - 1, own);
  if (keep >= own) {  // every eligible block is kept
    for (int i = tid; i < k; i += kTopkThreads) out_sel[i] = i <= own ? i : -1;
    __syncthreads();
    return;
  }
  if (tid == 0) sh.n_chosen = 0;
  float lo, hi;
  topk_range(scores, own, -INFINITY, INFINITY, false, 0.0, 0.0, 0, sh, lo, hi);
  int need = keep;
  // every refinement strictly shrinks the boundary bin, so a few rounds
  // suffice; the cap only guards against non-finite scores
  for (int round = 0; need > 0 && round < 64; ++round) {
    if (!(lo < hi)) {
      topk_lowest_equal(scores, own, hi, need, sh);
      break;
    }
    for (int i = tid; i < kTopkBins; i += kTopkThreads) sh.hist[i] = 0u;
    if (tid == 0) {
      sh.bstar = kTopkBins;
      sh.c_lt = 0;
      sh.c_eq = 0;
    }
    __syncthreads();
    const double dhi = (double)hi;
    const double scale = (double)kTopkBins / (dhi - (double)lo);
    for (int i = tid; i < own; i += kTopkThreads) {
      const float v = scores[i];
      if (v >= lo && v <= hi) atomicAdd(&sh.hist[topk_bin(v, dhi, scale)], 1u);
    }
    __syncthreads();
    if (wave == 0) {  // find the bin holding the need-th item
      constexpr int kPer = kTopkBins / kWave;
      unsigned h[kPer];
      unsigned local = 0;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        h[j] = sh.hist[lane * kPer + j];
        local += h[j];
      }
      unsigned incl = local;
#pragma unroll
      for (int off = 1; off < kWave; off <<= 1) {
        const unsigned o = __shfl_up(incl, off, kWave);
        if (lane >= off) incl += o;
      }
      unsigned prev = incl - local;
#pragma unroll
      for (int j = 0; j < kPer; ++j) {
        if (prev < (unsigned)need && prev + h[j] >= (unsigned)need) {
          sh.bstar = lane * kPer + j;
          sh.c_lt = (int)prev;
          sh.c_eq = (int)h[j];
        }
        prev += h[j];
      }
      if (lane == 0) sh.n_cand = 0;
    }
    __syncthreads();
    const int bstar = sh.bstar, c_lt = sh.c_lt, c_eq = sh.c_eq;
    if (bstar >= kTopkBins) break;  // fewer live scores than needed (non-finite input)
    const bool fits = c_eq <= kTopkCap;
    for (int i = tid; i < own; i += kTopkThreads) {
      const float v = scores[i];
      if (!(v >= lo && v <= hi)) continue;
      const int b = topk_bin(v, dhi, scale);
      if (b < bstar) {
        push_chosen(sh, i);
      } else if (b == bstar && fits) {
        const int p = atomicAdd(&sh.n_cand, 1);
        if (p < kTopkCap) {
          sh.cand_v[p] = v;
          sh.cand_i[p] = i;
        }
      }
    }
    __syncthreads();
    need -= c_lt;
    if (fits) {
      if (tid < c_eq) {
        const float v = sh.cand_v[tid];
        const int idx = sh.cand_i[tid];
        int rank = 0;
        for (int j = 0; j < c_eq; ++j) {
          const float w = sh.cand_v[j];
          rank += (w > v) || (w == v && sh.cand_i[j] < idx);
        }
        if (rank < need) push_chosen(sh, idx);
      }
      __syncthreads();
      break;
    }
    float nlo, nhi;
    topk_range(scores, own, lo, hi, true, dhi, scale, bstar, sh, nlo, nhi);
    lo = nlo;
    hi = nhi;
  }
  __syncthreads();
  // sort the kept blocks (own included) ascending; with non-finite scores
  // fewer than keep may have been found, the rest is filled with -1
  const int found = min(sh.n_chosen, keep);
  if (tid <= found) {
    const int x = tid < found ? sh.chosen[tid] : own;
    int rank = 0;
    for (int j = 0; j <= found; ++j) rank += (j < found ? sh.chosen[j] : own) < x;
    out_sel[rank] = x;
  }
  for (int i = found + 1 + tid; i < k; i += kTopkThreads) out_sel[i] = -1;
  __syncthreads();
}

}  // namespace msa
