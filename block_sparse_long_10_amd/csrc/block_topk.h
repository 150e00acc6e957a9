// Block TopK: the k best blocks of one (sequence or tile, group) by pooled
// index score, ranked by (score descending, block index ascending), with the
// own block always kept ("TopK" of the index branch in "MiniMax wird dünn",
// section 1, Schritt 1).
//
// One 256-thread workgroup selects from scores[0 .. own).  A score's rank is
// that of its order-preserving 32-bit key (-0.0 folded into +0.0).
//
// Fast path (own <= 256*MAXV): the scores are loaded into registers, all
// loads at once (-inf in the slots past the row).  Each thread takes the max
// of its scores; an LDS histogram of the thread maxima (threads holding no
// score left out, so that short rows keep fine bins) gives T, the lowest key
// of the bin that completes k' = k-1 maxima; those k' distinct scores reach
// T, so it bounds the k'-th best score from below.  The few scores >= T are
// gathered to LDS (DPP prefix-sum offsets; every slot is written, the
// others to a write-off slot, so there is no branch per slot).  With at most
// four more than k' of them, the worst are dropped one at a time (wave
// minimum of the key, then maximum of the index among equal keys);
// otherwise they are sorted by (score, index) with a wave-wide DPP bitonic
// sort.  A second sort puts the winners in block order; each sort network
// is only as wide as its count.  If more than 64 scores reach T (heavy
// ties), or the row is longer
// than the registers hold, the general path runs instead, on keys re-read
// from memory (so the fast path's registers are free for the caller's other
// phases):
//   1. key range [lo, hi] (DPP/shuffle wave reductions + LDS);
//   2. LDS histogram of bin = (hi - key) >> shift, at most 256 bins; the bin
//      is monotone in the key, so every item of a lower bin outranks every
//      item of a higher bin;
//   3. a wave scan finds the bin b* holding the last needed item; items of
//      lower bins are kept; the items of b* are ranked exactly by
//      (key, index) when they fit in LDS, otherwise [lo, hi] narrows to b*'s
//      range (at least 2^7 times smaller) and the histogram repeats;
//   4. when the live range holds a single key, the lowest indices win
//      (ballot prefix counts in index order).
// The result (sorted ascending, own block included, -1 padded) lands in LDS.
#pragma once

#include "msa_device.h"
#include "timeline_marks.h"

namespace msa {

constexpr int kTopkThreads = 256;
constexpr int kTopkBins = 256;
constexpr int kTopkCap = 256;
constexpr int kMaxTopK = 64;

struct TopkShared {
  // the fast path's histogram, then (once the bound is known) its candidate
  // (score bits, index) pairs: slots below the count, and one write-off slot
  // per lane above kWave
  union {
    unsigned hist[kTopkBins];
    uint2 pair[kTopkBins / 2];
  };
  uint32_t cand_k[kTopkCap];
  int cand_i[kTopkCap];
  int chosen[kMaxTopK];
  uint32_t red_a[kTopkThreads / kWave];
  uint32_t red_b[kTopkThreads / kWave];
  int wave_cnt[kTopkThreads / kWave];
  int n_chosen;
  int n_cand;
  int bstar;
  int c_lt;
  int c_eq;
};

// Order-preserving map float -> uint32 (larger score, larger key).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __builtin_bit_cast(uint32_t, v);
  if ((u << 1) == 0u) u = 0u;  // -0.0 == +0.0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ uint32_t umax_(uint32_t a, uint32_t b) { return a > b ? a : b; }
__device__ __forceinline__ uint32_t umin_(uint32_t a, uint32_t b) { return a < b ? a : b; }

template <int N>
__device__ __forceinline__ uint32_t row_ror_u(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x120 + N, 0xF, 0xF, false);
}
// Wave maximum / minimum (every lane active): DPP rotations within each row
// of 16 lanes, then the four row results meet in scalar registers (lane
// reads instead of LDS permutes, which cost a round trip through the LDS
// unit each).  The result is wave-uniform.
__device__ __forceinline__ uint32_t rows_to_scalar_max(uint32_t v) {
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return umax_(umax_(a, b), umax_(c, d));
}
__device__ __forceinline__ uint32_t rows_to_scalar_min(uint32_t v) {
  const uint32_t a = __builtin_amdgcn_readlane(v, 0), b = __builtin_amdgcn_readlane(v, 16);
  const uint32_t c = __builtin_amdgcn_readlane(v, 32), d = __builtin_amdgcn_readlane(v, 48);
  return umin_(umin_(a, b), umin_(c, d));
}
__device__ __forceinline__ uint32_t wave_umax(uint32_t v) {
  v = umax_(v, row_ror_u<8>(v));
  v = umax_(v, row_ror_u<4>(v));
  v = umax_(v, row_ror_u<2>(v));
  v = umax_(v, row_ror_u<1>(v));
  return rows_to_scalar_max(v);
}
__device__ __forceinline__ uint32_t wave_umin(uint32_t v) {
  v = umin_(v, row_ror_u<8>(v));
  v = umin_(v, row_ror_u<4>(v));
  v = umin_(v, row_ror_u<2>(v));
  v = umin_(v, row_ror_u<1>(v));
  return rows_to_scalar_min(v);
}

// Inverse of order_key for keys of finite floats (-0.0 comes back as +0.0).
__device__ __forceinline__ float key_float(uint32_t k) {
  return __builtin_bit_cast(float, (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k);
}
constexpr uint32_t kKeyMinFinite = 0x00800000u;  // order_key(-FLT_MAX); -inf maps below it

// Scores held in registers for the fast path: item i = j*256 + tid lives in
// val[j] (-inf in the slots past the row).  The fast path compares the
// floats themselves and forms keys only for thread maxima and candidates.
template <int MAXV>
struct RegKeys {
  float val[MAXV];
  int n;
  // (every load is issued: slots past the row read its last score, or the
  // row's first entry when it is empty, and are then set to -inf; a load
  // under a branch per slot made the loads trickle out one by one)
  __device__ __forceinline__ void load(const float* __restrict__ s, int n_) {
    n = n_;
    const int tid = threadIdx.x;
    const int last = n > 0 ? n - 1 : 0;
#pragma unroll
    for (int j = 0; j < MAXV; ++j) {
      const int i = j * kTopkThreads + tid;
      const float v = s[min(i, last)];
      val[j] = i < n ? v : -INFINITY;
    }
  }
};

// Keys re-read from global memory: the general path (heavy ties, or rows
// longer than the registers hold).
struct GlobalKeys {
  const float* __restrict__ s;
  int n;
  template <class F>
  __device__ __forceinline__ void each(F&& f) const {
    for (int i = threadIdx.x; i < n; i += kTopkThreads) f(i, order_key(s[i]));
  }
  template <class F>
  __device__ __forceinline__ void chunks_in_order(F&& f) const {
    for (int c0 = 0; c0 < n; c0 += kTopkThreads) {
      const int i = c0 + (int)threadIdx.x;
      if (!f(i, i < n ? order_key(s[i]) : 0u, i < n)) break;
    }
  }
};

__device__ __forceinline__ void push_chosen(TopkShared& sh, int i) {
  const int p = atomicAdd(&sh.n_chosen, 1);
  if (p < kMaxTopK) sh.chosen[p] = i;
}

// Range [lo, hi] of the live keys (lo <= key <= hi, and bin == b when b >= 0).
template <class Src>
__device__ __forceinline__ void topk_range(const Src& src, uint32_t lo, uint32_t hi, int shift,
                                           int b, TopkShared& sh, uint32_t& out_lo,
                                           uint32_t& out_hi) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  uint32_t mx = 0u, mn = 0xFFFFFFFFu;
  src.each([&](int, uint32_t key) {
    bool live = key >= lo && key <= hi;
    if (b >= 0) live = live && (int)((hi - key) >> shift) == b;
    if (live) {
      mx = umax_(mx, key);
      mn = umin_(mn, key);
    }
  });
  mx = wave_umax(mx);
  mn = wave_umin(mn);
  if (lane == 0) {
    sh.red_a[wave] = mx;
    sh.red_b[wave] = mn;
  }
  __syncthreads();
  mx = sh.red_a[0];
  mn = sh.red_b[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / kWave; ++w) {
    mx = umax_(mx, sh.red_a[w]);
    mn = umin_(mn, sh.red_b[w]);
  }
  __syncthreads();
  out_lo = mn;
  out_hi = mx;
}

// Keep the `need` lowest indices among the items whose key equals val.
template <class Src>
__device__ __forceinline__ void topk_lowest_equal(const Src& src, uint32_t val, int need,
                                                  TopkShared& sh) {
  const int lane = threadIdx.x & (kWave - 1), wave = threadIdx.x / kWave;
  int done = 0;
  src.chunks_in_order([&](int i, uint32_t key, bool valid) -> bool {
    if (done >= need) return false;
    const bool f = valid && key == val;
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
    return true;
  });
}

// Lane exchange with lane ^ M across the wave (DPP for M <= 8, swizzle for
// 16, bpermute for 32).  row_ror:n reads lane i-n within a row of 16.
template <int M>
__device__ __forceinline__ uint32_t xor_exchange(uint32_t v) {
  const int iv = (int)v;
  if constexpr (M == 1) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0xB1, 0xF, 0xF, false);  // quad_perm 1,0,3,2
  } else if constexpr (M == 2) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x4E, 0xF, 0xF, false);  // quad_perm 2,3,0,1
  } else if constexpr (M == 4) {
    const int lo = __builtin_amdgcn_mov_dpp(iv, 0x12C, 0xF, 0xF, false);  // lane i+4
    const int hi = __builtin_amdgcn_mov_dpp(iv, 0x124, 0xF, 0xF, false);  // lane i-4
    return (uint32_t)((threadIdx.x & 4) ? hi : lo);
  } else if constexpr (M == 8) {
    return (uint32_t)__builtin_amdgcn_mov_dpp(iv, 0x128, 0xF, 0xF, false);  // row_ror:8
  } else if constexpr (M == 16) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle(iv, 0x401F);  // xor 16 within 32 lanes
  } else {
    return (uint32_t)__shfl_xor(iv, 32, kWave);
  }
}

// One compare-exchange stage of a bitonic sort of one 32-bit value per lane:
// lanes pair with lane ^ J; blocks of K lanes alternate direction so that the
// full sort (K = 64) is descending from lane 0.
template <int K, int J>
__device__ __forceinline__ void bitonic_stage(uint32_t& v) {
  const uint32_t o = xor_exchange<J>(v);
  const int lane = threadIdx.x & (kWave - 1);
  const bool take_max = ((lane & J) == 0) == ((lane & K) == 0);
  v = take_max ? umax_(v, o) : umin_(v, o);
}
template <int K>
__device__ __forceinline__ void bitonic_merge(uint32_t& v) {
  if constexpr (K >= 64) bitonic_stage<K, 32>(v);
  if constexpr (K >= 32) bitonic_stage<K, 16>(v);
  if constexpr (K >= 16) bitonic_stage<K, 8>(v);
  if constexpr (K >= 8) bitonic_stage<K, 4>(v);
  if constexpr (K >= 4) bitonic_stage<K, 2>(v);
  bitonic_stage<K, 1>(v);
}
// Sort the lane values of each group of W lanes (W = 16, 32 or 64)
// descending: lane 0 of the wave holds the largest of lanes 0 .. W-1.  (The
// other groups end up sorted too, in alternating directions.)
template <int W = 64>
__device__ __forceinline__ void wave_sort_desc(uint32_t& v) {
  bitonic_merge<2>(v);
  bitonic_merge<4>(v);
  bitonic_merge<8>(v);
  bitonic_merge<16>(v);
  if constexpr (W >= 32) bitonic_merge<32>(v);
  if constexpr (W >= 64) bitonic_merge<64>(v);
}

// The same for (key, index) pairs ordered by key descending, then index
// ascending (the selection order).
template <int K, int J>
__device__ __forceinline__ void bitonic_stage2(uint32_t& key, uint32_t& idx) {
  const uint32_t ok = xor_exchange<J>(key), oi = xor_exchange<J>(idx);
  const int lane = threadIdx.x & (kWave - 1);
  const bool take_max = ((lane & J) == 0) == ((lane & K) == 0);
  const bool other_first = ok > key || (ok == key && oi < idx);
  const bool take_other = take_max == other_first;
  key = take_other ? ok : key;
  idx = take_other ? oi : idx;
}
template <int K>
__device__ __forceinline__ void bitonic_merge2(uint32_t& key, uint32_t& idx) {
  if constexpr (K >= 64) bitonic_stage2<K, 32>(key, idx);
  if constexpr (K >= 32) bitonic_stage2<K, 16>(key, idx);
  if constexpr (K >= 16) bitonic_stage2<K, 8>(key, idx);
  if constexpr (K >= 8) bitonic_stage2<K, 4>(key, idx);
  if constexpr (K >= 4) bitonic_stage2<K, 2>(key, idx);
  bitonic_stage2<K, 1>(key, idx);
}
// Sort the (key, index) pairs of each group of W lanes into selection order:
// lane 0 first.
template <int W = 64>
__device__ __forceinline__ void wave_sort_pairs(uint32_t& key, uint32_t& idx) {
  bitonic_merge2<2>(key, idx);
  bitonic_merge2<4>(key, idx);
  bitonic_merge2<8>(key, idx);
  bitonic_merge2<16>(key, idx);
  if constexpr (W >= 32) bitonic_merge2<32>(key, idx);
  if constexpr (W >= 64) bitonic_merge2<64>(key, idx);
}

// Wave inclusive prefix sum with DPP: row shifts, then row broadcasts.
__device__ __forceinline__ int wave_incl_scan(int v) {
  v += __builtin_amdgcn_update_dpp(0, v, 0x111, 0xF, 0xF, false);  // row_shr:1
  v += __builtin_amdgcn_update_dpp(0, v, 0x112, 0xF, 0xF, false);  // row_shr:2
  v += __builtin_amdgcn_update_dpp(0, v, 0x114, 0xF, 0xF, false);  // row_shr:4
  v += __builtin_amdgcn_update_dpp(0, v, 0x118, 0xF, 0xF, false);  // row_shr:8
  v += __builtin_amdgcn_update_dpp(0, v, 0x142, 0xA, 0xF, false);  // row_bcast:15
  v += __builtin_amdgcn_update_dpp(0, v, 0x143, 0xC, 0xF, false);  // row_bcast:31
  return v;
}

// Fast path; returns false (leaving out_sel untouched) when more than 64
// keys reach the bound.  Requires 1 <= keep < own.  Without ORDERED the
// kept blocks before the own one come in a fixed order of the path's own
// (gather or score order) instead of ascending: for callers that only need
// the same set in the same order in every workgroup.
// (timeline marks: the unordered form runs only in the decode attention kernel)
#define MSA_TOPK_MARK(m)                \
  do {                                  \
    if constexpr (!ORDERED) MSA_MARK(m); \
  } while (0)
template <int MAXV, bool ORDERED>
__device__ __forceinline__ bool topk_fast(const RegKeys<MAXV>& src, int own, int keep, int k,
                                          int* out_sel, TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  // thread max (tree, on the floats; slots past the row hold -inf) and the
  // range of the 256 thread maxima as keys
  float mx[MAXV];
#pragma unroll
  for (int j = 0; j < MAXV; ++j) mx[j] = src.val[j];
#pragma unroll
  for (int w = MAXV / 2; w >= 1; w /= 2)
#pragma unroll
    for (int j = 0; j < w; ++j) mx[j] = fmaxf(mx[j], mx[j + w]);
  // (threads with no score of the row hold -inf: they are left out of the
  // range and the histogram, so that a short row keeps fine bins; at least
  // keep < own threads hold a score)
  const uint32_t m = order_key(mx[0]);
  MSA_TOPK_MARK(MSA_MARK_SCORES_IN);
  const bool has = m >= kKeyMinFinite;
  const uint32_t wmax = wave_umax(m), wmin = wave_umin(has ? m : 0xFFFFFFFFu);
  if (lane == 0) {
    sh.red_a[wave] = wmax;
    sh.red_b[wave] = wmin;
  }
  for (int i = tid; i < kTopkBins; i += kTopkThreads) sh.hist[i] = 0u;
  __syncthreads();
  MSA_TOPK_MARK(MSA_MARK_RANGE);
  uint32_t hi = sh.red_a[0], lo = sh.red_b[0];
#pragma unroll
  for (int w = 1; w < kTopkThreads / kWave; ++w) {
    hi = umax_(hi, sh.red_a[w]);
    lo = umin_(lo, sh.red_b[w]);
  }
  // histogram of the thread maxima, bin = (hi - m) >> shift (at most 256
  // bins, monotone): T = lowest key of the bin that completes `keep` maxima;
  // those `keep` distinct scores reach T, so T bounds the keep-th best score.
  const uint32_t span = hi - lo;
  const int bits = span == 0u ? 0 : 32 - __builtin_clz(span);
  const int shift = bits > 8 ? bits - 8 : 0;
  if (has) atomicAdd(&sh.hist[(hi - m) >> shift], 1u);
  __syncthreads();
  if (wave == 0) {
    constexpr int kPer = kTopkBins / kWave;
    unsigned h[kPer], local = 0;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      h[j] = sh.hist[lane * kPer + j];
      local += h[j];
    }
    unsigned prev = (unsigned)wave_incl_scan((int)local) - local;
#pragma unroll
    for (int j = 0; j < kPer; ++j) {
      if (prev < (unsigned)keep && prev + h[j] >= (unsigned)keep) sh.bstar = lane * kPer + j;
      prev += h[j];
    }
  }
  __syncthreads();
  MSA_TOPK_MARK(MSA_MARK_BIN);
  const uint32_t edge = ((uint32_t)(sh.bstar + 1) << shift) - 1u;  // hi - key <= edge
  // the bound as a float (at least -FLT_MAX, so the -inf of empty slots
  // never reaches it): key >= t  <=>  score >= tf for finite scores
  const uint32_t t = umax_(hi - umin_(edge, hi - kKeyMinFinite), kKeyMinFinite);
  const float tf = key_float(t);
  // count, scan and gather the scores >= tf
  int cnt = 0;
#pragma unroll
  for (int j = 0; j < MAXV; ++j) cnt += src.val[j] >= tf;
  const int incl = wave_incl_scan(cnt);
  if (lane == kWave - 1) sh.wave_cnt[wave] = incl;
  __syncthreads();
  MSA_TOPK_MARK(MSA_MARK_COUNTED);
  int base = incl - cnt, total = 0;
#pragma unroll
  for (int w = 0; w < kTopkThreads / kWave; ++w) {
    const int c = sh.wave_cnt[w];
    if (w < wave) base += c;
    total += c;
  }
  if (total > kWave) return false;  // uniform
  // every thread writes every slot j, to its place in the candidate list or
  // to its lane's write-off slot (no branch per slot); the histogram was last
  // read before the barrier that published bstar
#pragma unroll
  for (int j = 0; j < MAXV; ++j) {
    const bool c = src.val[j] >= tf;
    sh.pair[c ? base : kWave + lane] =
        uint2{__builtin_bit_cast(uint32_t, src.val[j]), (uint32_t)(j * kTopkThreads + tid)};
    base += c ? 1 : 0;
  }
  __syncthreads();
  MSA_TOPK_MARK(MSA_MARK_GATHERED);
  if (wave == 0) {
    // total >= keep candidates (T bounds the keep-th best score).  A few
    // too many: the worst are dropped one at a time (lowest key, then
    // highest index); more: the candidates are sorted into selection order
    // and the first keep taken.  The winners' indices are then put in
    // ascending order (sort networks only as wide as needed).
    const uint2 pr = sh.pair[lane];
    bool live = lane < total;
    uint32_t key = live ? order_key(__builtin_bit_cast(float, pr.x)) : 0u;
    uint32_t idx = live ? pr.y : 0x7FFFFFFFu;
    const int drop = total - keep;  // uniform
    uint32_t v;
    int width = total;
    if (drop <= 4) {
      for (int d = 0; d < drop; ++d) {
        const uint32_t kmin = wave_umin(live ? key : 0xFFFFFFFFu);
        const uint32_t imax = wave_umax(live && key == kmin ? idx : 0u);
        live = live && !(key == kmin && idx == imax);
      }
      if constexpr (!ORDERED) {  // the winners in gather order
        const uint64_t lm = __ballot(live);
        const int r = __builtin_amdgcn_mbcnt_hi((uint32_t)(lm >> 32),
                                                __builtin_amdgcn_mbcnt_lo((uint32_t)lm, 0u));
        if (live) out_sel[r] = (int)idx;
      }
      v = live ? ~idx : 0u;
    } else {
      if (total <= 32) wave_sort_pairs<32>(key, idx);
      else wave_sort_pairs<64>(key, idx);
      if constexpr (!ORDERED) {  // the winners in score order
        if (lane < keep) out_sel[lane] = (int)idx;
      }
      v = lane < keep ? ~idx : 0u;
      width = keep;
    }
    if constexpr (ORDERED) {
      if (width <= 16) wave_sort_desc<16>(v);
      else if (width <= 32) wave_sort_desc<32>(v);
      else wave_sort_desc<64>(v);
      if (lane < keep) out_sel[lane] = (int)~v;
    }
    if (lane == 0) out_sel[keep] = own;
    for (int i = keep + 1 + lane; i < k; i += kWave) out_sel[i] = -1;
    MSA_TOPK_MARK(MSA_MARK_SELECTED);
  }
  __syncthreads();
  return true;
}
#undef MSA_TOPK_MARK

// Sort keep+1 kept blocks (chosen[0..found) and own) ascending into out_sel.
__device__ __forceinline__ void topk_write_sorted(const TopkShared& sh, int found, int own, int k,
                                                  int* out_sel) {
  const int tid = threadIdx.x;
  if (tid <= found) {
    const int x = tid < found ? sh.chosen[tid] : own;
    int rank = 0;
    for (int j = 0; j <= found; ++j) rank += (j < found ? sh.chosen[j] : own) < x;
    out_sel[rank] = x;
  }
  for (int i = found + 1 + tid; i < k; i += kTopkThreads) out_sel[i] = -1;
  __syncthreads();
}

// All 256 threads call this with identical arguments; src holds scores of
// blocks 0 .. own-1.  out_sel (LDS, k entries) receives the kept blocks.
template <class Src>
__device__ __forceinline__ void topk_select(const Src& src, int own, int k, int* out_sel,
                                            TopkShared& sh) {
  const int tid = threadIdx.x, lane = tid & (kWave - 1), wave = tid / kWave;
  const int keep = min(k - 1, own);
  if (keep >= own) {  // every eligible block is kept
    for (int i = tid; i < k; i += kTopkThreads) out_sel[i] = i <= own ? i : -1;
    __syncthreads();
    return;
  }
  if (tid == 0) sh.n_chosen = 0;
  uint32_t lo, hi;
  topk_range(src, 0u, 0xFFFFFFFFu, 0, -1, sh, lo, hi);
  int need = keep;
  // each refinement shrinks hi - lo at least 2^7-fold: at most 5 rounds
  for (int round = 0; need > 0 && round < 8; ++round) {
    if (lo == hi) {
      topk_lowest_equal(src, hi, need, sh);
      break;
    }
    const uint32_t span = hi - lo;
    const int bits = 32 - __builtin_clz(span);
    const int shift = bits > 8 ? bits - 8 : 0;
    for (int i = tid; i < kTopkBins; i += kTopkThreads) sh.hist[i] = 0u;
    if (tid == 0) {
      sh.bstar = kTopkBins;
      sh.c_lt = 0;
      sh.c_eq = 0;
    }
    __syncthreads();
    src.each([&](int, uint32_t key) {
      if (key >= lo && key <= hi) atomicAdd(&sh.hist[(hi - key) >> shift], 1u);
    });
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
    if (bstar >= kTopkBins) break;  // cannot happen for well-formed input
    const bool fits = c_eq <= kTopkCap;
    src.each([&](int i, uint32_t key) {
      if (!(key >= lo && key <= hi)) return;
      const int b = (int)((hi - key) >> shift);
      if (b < bstar) {
        push_chosen(sh, i);
      } else if (b == bstar && fits) {
        const int p = atomicAdd(&sh.n_cand, 1);
        if (p < kTopkCap) {
          sh.cand_k[p] = key;
          sh.cand_i[p] = i;
        }
      }
    });
    __syncthreads();
    need -= c_lt;
    if (fits) {
      if (tid < c_eq) {
        const uint32_t key = sh.cand_k[tid];
        const int idx = sh.cand_i[tid];
        int rank = 0;
        for (int j = 0; j < c_eq; ++j) {
          const uint32_t o = sh.cand_k[j];
          rank += (o > key) || (o == key && sh.cand_i[j] < idx);
        }
        if (rank < need) push_chosen(sh, idx);
      }
      __syncthreads();
      break;
    }
    uint32_t nlo, nhi;
    topk_range(src, lo, hi, shift, bstar, sh, nlo, nhi);
    lo = nlo;
    hi = nhi;
  }
  __syncthreads();
  // with non-finite scores fewer than keep may have been found; -1 fills
  topk_write_sorted(sh, min(sh.n_chosen, keep), own, k, out_sel);
}

// TopK of scores[0 .. own) held in global memory.  Up to 256 * REGS
// candidates live in registers (REGS per thread: 32, or 4 for kernels that
// only meet rows of at most 1024 blocks, which then do an eighth of the
// work); WIDE kernels also keep up to 16384 there (64 per thread), otherwise
// longer rows are re-read from memory.  Each register variant is a separate
// copy of the selection code, so kernels on a latency-critical path keep only
// the one they need.
template <bool WIDE, bool ORDERED = true, int REGS = 32>
__device__ __forceinline__ void block_topk(const float* __restrict__ scores, int own, int k,
                                           int* out_sel, TopkShared& sh) {
  const int keep = min(k - 1, own);
  if (keep >= own || keep == 0) {
    GlobalKeys src{scores, own};  // nothing to rank
    topk_select(src, own, k, out_sel, sh);
  } else if (own <= kTopkThreads * REGS) {
    RegKeys<REGS> src;
    src.load(scores, own);
    if (!topk_fast<REGS, ORDERED>(src, own, keep, k, out_sel, sh))
      topk_select(GlobalKeys{scores, own}, own, k, out_sel, sh);
  } else if (WIDE && own <= kTopkThreads * 64) {
    RegKeys<64> src;
    src.load(scores, own);
    if (!topk_fast<64, ORDERED>(src, own, keep, k, out_sel, sh))
      topk_select(GlobalKeys{scores, own}, own, k, out_sel, sh);
  } else {
    GlobalKeys src{scores, own};
    topk_select(src, own, k, out_sel, sh);
  }
}

// TopK with forced blocks: blocks [0, n_sink) and the n_local blocks just
// before the own block are kept unranked and count toward k; the other
// eligible blocks form the contiguous range [lo, hi), ranked by block_topk as
// if hi were the own block with a budget of k - (number forced).  Without
// forced blocks that is the plain selection, written straight to out_sel (one
// copy of the selection code either way).  tmp is an LDS array of kMaxTopK
// entries.  Result as block_topk's (ascending, or as ORDERED allows; own
// block included, -1 padded).
template <bool WIDE, bool ORDERED = true, int REGS = 32>
__device__ __forceinline__ void block_topk_forced(const float* __restrict__ scores, int own, int k,
                                                  int n_sink, int n_local, int* out_sel,
                                                  int* tmp, TopkShared& sh) {
  const int lo = min(n_sink, own);
  const int hi = max(own - n_local, lo);
  const int forced = lo + (own - hi);
  const int kr = k - forced;  // >= 1: the host checks sink + local <= k - 1
  block_topk<WIDE, ORDERED, REGS>(scores + lo, hi - lo, kr, forced == 0 ? out_sel : tmp, sh);
  if (forced == 0) return;  // uniform
  const int chosen = min(kr - 1, hi - lo);  // tmp[0 .. chosen) are relative block ids
  for (int i = threadIdx.x; i < k; i += kTopkThreads) {
    int b;
    if (i < lo) b = i;
    else if (i < lo + chosen) b = lo + tmp[i - lo];
    else if (i <= lo + chosen + (own - hi)) b = hi + (i - lo - chosen);
    else b = -1;
    out_sel[i] = b;
  }
  __syncthreads();
}

}  // namespace msa
