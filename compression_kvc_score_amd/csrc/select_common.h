// Device helpers shared by the selection kernels and the selection inside the
// fused scan launch (TideKV, Fig. 3 caption: the top K_l - |R_mand|
// non-mandatory keys plus the mandatory sink and recent keys): ranking-key
// formats, workgroup scans, the per-head geometry of the mandatory set, and
// the radix digit pick.
#pragma once

#include "kvc_internal.h"
#include "wave_ops.h"

namespace kvc {
namespace {

// Ranking keys: uint32 patterns ordered like the values. Softmax scores are
// >= +0, so their IEEE-754 patterns already are; signed scores (the raw
// inner-product modes) map negatives to their complement and set the sign
// bit of the others (-0 is taken as +0). The histogram bin is the 12 bits
// above the LOW pattern bits that the radix rounds resolve (10 bits, then
// LOW - 10); listed candidates keep a sub-chunk tag in the bits above LOW.
template <bool SIGNED>
struct KeyFmt {
  static constexpr int LOW = SIGNED ? 20 : 19;
  static constexpr uint32_t LOW_MASK = (1u << LOW) - 1u;
  static constexpr int R2 = LOW - 10;
  static constexpr uint32_t R2_BINS = 1u << R2;
  __device__ static __forceinline__ uint32_t key(float v) {
    uint32_t u = __float_as_uint(v);
    if constexpr (SIGNED) {
      if (u == 0x80000000u) u = 0u;
      return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    } else {
      return u;
    }
  }
  __device__ static __forceinline__ uint32_t bin(uint32_t key) { return (key >> LOW) & (kHistBins - 1); }
};

// Workgroup barrier. LDS_ONLY: it orders LDS accesses alone and leaves this
// thread's global loads and stores in flight (__syncthreads waits for them).
template <bool LDS_ONLY>
__device__ __forceinline__ void wg_sync() {
  if constexpr (LDS_ONLY) asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
  else __syncthreads();
}

// Exclusive prefix sum over a workgroup of NW wavefronts, one value per
// thread; also returns the total. Uses `scratch` (NW entries) in LDS.
template <int NW, bool LDS_ONLY = false>
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(v);
  if (lane == 63) scratch[wave] = incl;
  wg_sync<LDS_ONLY>();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    const uint32_t t = scratch[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  total = all;
  wg_sync<LDS_ONLY>();
  return before + incl - v;
}

// Sums over a workgroup of NW wavefronts of two values per thread (every
// thread gets both). Uses `scratch` (2 * NW entries) in LDS.
template <int NW, bool LDS_ONLY = false>
__device__ void block_sum2(uint32_t& x, uint32_t& y, uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t ix = wave_inclusive_sum(x), iy = wave_inclusive_sum(y);
  if (lane == 63) {
    scratch[wave] = ix;
    scratch[NW + wave] = iy;
  }
  wg_sync<LDS_ONLY>();
  x = 0u;
  y = 0u;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    x += scratch[w];
    y += scratch[NW + w];
  }
  wg_sync<LDS_ONLY>();
}

// Sums over a workgroup of NW wavefronts of N values per thread (every
// thread gets all N). Uses `scratch` (N * NW entries) in LDS.
template <int NW, int N, bool LDS_ONLY = false>
__device__ void block_sums(uint32_t (&x)[N], uint32_t* scratch) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
  for (int i = 0; i < N; ++i) {
    const uint32_t inc = wave_inclusive_sum(x[i]);
    if (lane == 63) scratch[i * NW + wave] = inc;
  }
  wg_sync<LDS_ONLY>();
#pragma unroll
  for (int i = 0; i < N; ++i) {
    x[i] = 0u;
#pragma unroll
    for (int w = 0; w < NW; ++w) x[i] += scratch[i * NW + w];
  }
  wg_sync<LDS_ONLY>();
}

struct HeadGeom {
  int64_t s, sink_end, rec_begin;
  int64_t budget;
  uint32_t k_sel;  // candidates to choose (budget - mandatory); 0 when keeping all
  bool keep_all;
};

__device__ __forceinline__ HeadGeom head_geom(const SelectArgs& a, int head) {
  HeadGeom h;
  h.s = a.s;
  h.budget = a.heads.budget[head];
  h.keep_all = h.budget >= h.s;
  h.sink_end = a.n_sink < h.s ? a.n_sink : h.s;
  h.rec_begin = h.s - a.n_recent;
  if (h.rec_begin < h.sink_end) h.rec_begin = h.sink_end;
  const int64_t n_mand = h.sink_end + (h.s - h.rec_begin);
  h.k_sel = h.keep_all ? 0u : (uint32_t)(h.budget - n_mand);
  return h;
}

__device__ __forceinline__ bool is_candidate(const HeadGeom& h, int64_t j) {
  return j >= h.sink_end && j < h.rec_begin;
}

// Mandatory keys in [lo, hi).
__device__ __forceinline__ uint32_t mandatory_in(const HeadGeom& h, int64_t lo, int64_t hi) {
  if (hi > h.s) hi = h.s;
  if (lo >= hi) return 0u;
  const int64_t sink = h.sink_end > lo ? (h.sink_end < hi ? h.sink_end : hi) - lo : 0;
  const int64_t rb = h.rec_begin > lo ? h.rec_begin : lo;
  const int64_t rec = hi > rb ? hi - rb : 0;
  return (uint32_t)(sink + rec);
}

// Ranking value of key j: the score, or its centred max over [j - r, j + r].
__device__ __forceinline__ float rank_value(const float* row, int64_t s, int64_t j, int r) {
  float m = row[j];
  for (int t = 1; t <= r; ++t) {
    if (j - t >= 0) m = fmaxf(m, row[j - t]);
    if (j + t < s) m = fmaxf(m, row[j + t]);
  }
  return m;
}

// Run by one wavefront: among the NB bins of `hist` (counts), walked from the
// highest bin down, find the bin d holding the rem-th element and the rank of
// that element inside d; lane 0 of the bin's owner writes (d, rank) to out.
template <int NB>
__device__ void pick_digit_wave(const uint32_t* hist, uint32_t rem, uint32_t* out) {
  constexpr int BPL = NB / kWave;  // bins per lane, consecutive and descending
  const int lane = threadIdx.x & 63;
  uint32_t c[BPL], loc = 0;
#pragma unroll
  for (int q = 0; q < BPL; ++q) {
    c[q] = hist[NB - 1 - BPL * lane - q];
    loc += c[q];
  }
  const uint32_t incl = wave_inclusive_sum(loc);
  uint32_t before = incl - loc;
  if (before < rem && rem <= incl) {
#pragma unroll
    for (int q = 0; q < BPL; ++q) {
      if (before < rem && rem <= before + c[q]) {
        out[0] = (uint32_t)(NB - 1 - BPL * lane - q);
        out[1] = rem - before;
      }
      before += c[q];
    }
  }
}

}  // namespace
}  // namespace kvc
