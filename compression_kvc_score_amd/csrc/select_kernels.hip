// Selection of the retained keys (TideKV, Fig. 3 caption): per KV head, the
// mandatory sink and recent keys plus the top K_h - |mandatory| other keys by
// (score descending, index ascending), written in ascending key order.
//
// Scores are finite and >= +0, so their IEEE-754 bit patterns read as uint32
// order the same way as the values. The selection spreads over every CU:
//
//  hist     a 4096-bin histogram of the candidates' top bits (bits 30..19:
//           exponent and 4 mantissa bits) per KV head. Workgroups take
//           4096-key chunks, count in LDS and add their non-empty bins to the
//           global histogram. (Inside the whole-layer call, pass 2 builds the
//           same histogram while it writes the scores; with a max-pool this
//           kernel also writes the pooled values.)
//  filter   every chunk workgroup finds, from its head's histogram, the bin b*
//           holding the k-th best candidate, counts its candidates above b*,
//           and lists the patterns of its candidates inside b* in its own
//           slot (no atomics).
//  select   every chunk workgroup reads its head's short lists (a few
//           thousand patterns), radix-selects in LDS the exact pattern T of
//           the k-th best candidate and how many candidates equal to T are
//           taken (the lowest indices: ties go to the lower index), derives
//           its output offset from the counts of the chunks before it, and
//           writes its kept indices in ascending order. If a slot or the
//           lists overflow (heavily tied scores), it selects by a radix over
//           the head's whole score row instead -- same result, slower.
//
// All counts are integers, so the output does not depend on the order in
// which workgroups run.

#include "kvc_internal.h"
#include "wave_ops.h"

namespace kvc {
namespace {

constexpr int kThreads = kSelectThreads;  // 1024
constexpr int kWaves = kThreads / kWave;  // 16
constexpr int kChunk = kSelectChunk;      // 4096 keys per chunk, 4 per thread

__device__ __forceinline__ uint32_t bin_of(uint32_t bits) { return (bits >> 19) & (kHistBins - 1); }

// Exclusive prefix sum over the workgroup of one value per thread; also
// returns the total. Uses `scratch` (kWaves + 1 entries) in LDS.
__device__ uint32_t block_exclusive_scan(uint32_t v, uint32_t* scratch, uint32_t& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const uint32_t incl = wave_inclusive_sum(v);
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  uint32_t before = 0, all = 0;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) {
    const uint32_t t = scratch[w];
    before += w < wave ? t : 0u;
    all += t;
  }
  total = all;
  __syncthreads();
  return before + incl - v;
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

// Ranking value of key j: the score, or its centred max over [j - r, j + r].
__device__ __forceinline__ float rank_value(const float* row, int64_t s, int64_t j, int r) {
  float m = row[j];
  for (int t = 1; t <= r; ++t) {
    if (j - t >= 0) m = fmaxf(m, row[j - t]);
    if (j + t < s) m = fmaxf(m, row[j + t]);
  }
  return m;
}

// Find the bin holding the k-th largest candidate from the head's histogram.
// Returns b* and the number of candidates in higher bins. Uses `scratch`.
__device__ void find_bin(const uint32_t* hist, uint32_t k, uint32_t* scratch, uint32_t& bstar,
                         uint32_t& above) {
  __shared__ uint32_t s_b, s_above;
  // thread t owns bins 4095-4t .. 4092-4t (descending)
  uint32_t c[4], loc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = hist[kHistBins - 1 - 4 * threadIdx.x - q];
    loc += c[q];
  }
  uint32_t total;
  uint32_t before = block_exclusive_scan(loc, scratch, total);
  if (before < k && k <= before + loc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (before < k && k <= before + c[q]) {
        s_b = kHistBins - 1 - 4 * threadIdx.x - q;
        s_above = before;
      }
      before += c[q];
    }
  }
  __syncthreads();
  bstar = s_b;
  above = s_above;
  __syncthreads();
}

// ---------------------------------------------------------------------------
// init: clear the per-head histograms and candidate counters.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) init_kernel(SelectArgs a, int hkv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < hkv * kHistBins) a.hist[i] = 0u;
}

// ---------------------------------------------------------------------------
// hist: per-chunk LDS histogram of candidate ranking values, merged into the
// head's global histogram; writes pooled values when pooling.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) hist_kernel(SelectArgs a) {
  __shared__ uint32_t lh[kHistBins];
  const int head = blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  const HeadGeom h = head_geom(a, head);
  if (h.keep_all || h.k_sel == 0) return;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads) lh[i] = 0u;
  __syncthreads();
  const float* row = a.scores + (int64_t)head * h.s;
  float* prow = a.pooled ? a.pooled + (int64_t)head * h.s : nullptr;
  const int64_t j0 = (int64_t)chunk * kChunk + 4 * threadIdx.x;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    if (j >= h.s) break;
    const float v = a.pool_radius > 0 ? rank_value(row, h.s, j, a.pool_radius) : row[j];
    if (prow) prow[j] = v;
    if (j >= h.sink_end && j < h.rec_begin) atomicAdd(&lh[bin_of(__float_as_uint(v))], 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)head * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// ---------------------------------------------------------------------------
// filter: per chunk, count the candidates above b* and list, in key order,
// the patterns of those inside b* (in the chunk's own slot: no atomics).
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) filter_kernel(SelectArgs a) {
  __shared__ uint32_t scratch[kWaves + 1];
  const int head = blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  const HeadGeom h = head_geom(a, head);
  if (h.keep_all || h.k_sel == 0) return;
  // this thread's four values, loaded before the histogram scan so that the
  // two memory round trips overlap
  const float* vals = a.vals + (int64_t)head * h.s;
  const int64_t j0 = (int64_t)chunk * kChunk + 4 * threadIdx.x;
  uint32_t bits[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    bits[e] = (j < h.s && j >= h.sink_end && j < h.rec_begin) ? __float_as_uint(vals[j]) : 0u;
  }
  uint32_t bstar, above_all;
  find_bin(a.hist + (int64_t)head * kHistBins, h.k_sel, scratch, bstar, above_all);

  uint32_t above = 0, nin = 0;
  bool in[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    in[e] = false;
    if (j < h.s && j >= h.sink_end && j < h.rec_begin) {
      const uint32_t b = bin_of(bits[e]);
      above += b > bstar;
      in[e] = b == bstar;
      nin += in[e];
    }
  }
  uint32_t n_in;
  uint32_t pos = block_exclusive_scan(nin, scratch, n_in);
  uint32_t* slot = a.slots + ((int64_t)head * a.n_chunks + chunk) * kSlotCap;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (in[e]) {
      if (pos < (uint32_t)kSlotCap) slot[pos] = bits[e];
      ++pos;
    }
  }
  uint32_t n_above;
  block_exclusive_scan(above, scratch, n_above);
  if (threadIdx.x == 0) {
    a.chunk_above[(int64_t)head * a.n_chunks + chunk] = n_above;
    a.chunk_in[(int64_t)head * a.n_chunks + chunk] = n_in;
  }
}

// Mandatory keys inside chunk c.
__device__ __forceinline__ uint32_t chunk_mandatory(const HeadGeom& h, int64_t c) {
  const int64_t lo = c * kChunk;
  int64_t hi = lo + kChunk;
  if (hi > h.s) hi = h.s;
  const int64_t sink = (h.sink_end > lo ? (h.sink_end < hi ? h.sink_end : hi) - lo : 0);
  const int64_t rec = (hi > h.rec_begin ? hi - (h.rec_begin > lo ? h.rec_begin : lo) : 0);
  return (uint32_t)(sink + rec);
}

// Slow path: k-th largest candidate pattern by a radix over the whole score
// row of the head (8 bits per round from the top).
__device__ uint32_t radix_over_row(const HeadGeom& h, const uint32_t* bits, uint32_t k,
                                   uint32_t* hist256, uint32_t& above) {
  __shared__ uint32_t s_digit, s_rem;
  uint32_t prefix = 0u, mask = 0u, rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += kThreads) hist256[i] = 0u;
    __syncthreads();
    for (int64_t j = h.sink_end + threadIdx.x; j < h.rec_begin; j += kThreads) {
      const uint32_t u = bits[j];
      if ((u & mask) == prefix) atomicAdd(&hist256[(u >> shift) & 255u], 1u);
    }
    __syncthreads();
    if (threadIdx.x < 64) {
      const int l = threadIdx.x;
      uint32_t c[4], loc = 0;
#pragma unroll
      for (int q = 0; q < 4; ++q) { c[q] = hist256[255 - 4 * l - q]; loc += c[q]; }
      const uint32_t incl = wave_inclusive_sum(loc);
      uint32_t before = incl - loc;
      if (before < rem && rem <= incl) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          if (before < rem && rem <= before + c[q]) {
            s_digit = 255u - 4u * l - q;
            s_rem = rem - before;
          }
          before += c[q];
        }
      }
    }
    __syncthreads();
    prefix |= s_digit << shift;
    mask |= 255u << shift;
    rem = s_rem;
    __syncthreads();
  }
  above = k - rem;  // candidates strictly above the threshold pattern
  return prefix;
}

// Sum over the workgroup of one value per thread (all threads get it).
__device__ __forceinline__ uint32_t block_sum(uint32_t v, uint32_t* scratch) {
  uint32_t tot;
  block_exclusive_scan(v, scratch, tot);
  return tot;
}

// ---------------------------------------------------------------------------
// select: each chunk workgroup resolves its head's exact threshold from the
// listed candidates (the same computation in every workgroup of the head),
// derives its output offset from the counts of the chunks before it, and
// writes its kept indices in ascending order.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) select_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* cbits = reinterpret_cast<uint32_t*>(smem);  // kCandCap listed patterns
  uint32_t* coff = cbits + kCandCap;                    // n_chunks + 1 list offsets
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t scratch[kWaves + 1];
  __shared__ uint32_t s_digit, s_rem, s_flag;

  const int head = blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  const HeadGeom h = head_geom(a, head);
  int32_t* out = a.idx_out + a.heads.offset[head];
  const int64_t j0 = (int64_t)chunk * kChunk + 4 * threadIdx.x;
  if (h.keep_all) {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (j0 + e < h.s) out[j0 + e] = (int32_t)(j0 + e);
    return;
  }
  const float* vals = a.vals + (int64_t)head * h.s;
  const uint32_t* rowbits = reinterpret_cast<const uint32_t*>(vals);
  const int nc = a.n_chunks;
  const uint32_t* c_in = a.chunk_in + (int64_t)head * nc;
  const uint32_t* c_above = a.chunk_above + (int64_t)head * nc;
  // this thread's four values, needed last, are loaded first
  uint32_t vbits[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    vbits[e] = (h.k_sel > 0 && j < h.s && j >= h.sink_end && j < h.rec_begin) ? __float_as_uint(vals[j]) : 0u;
  }

  uint32_t thr = 0xFFFFFFFFu, need_eq = 0u;  // k_sel == 0: no candidate is chosen
  // counts of the chunks before this one: kept = mandatory + above + taken equals
  uint32_t prev_gt = 0, prev_eq = 0;
  uint32_t eq_before = 0;  // equal candidates in chunks before this one
  if (h.k_sel > 0) {
    // list offsets; overflow if a chunk's slot or the whole list is too small
    if (threadIdx.x == 0) s_flag = 0u;
    __syncthreads();
    uint32_t n_total = 0;
    uint32_t above_local = 0;
    for (int c = threadIdx.x; c < nc; c += kThreads) above_local += c_above[c];
    for (int base = 0; base < nc; base += kThreads) {
      const int c = base + threadIdx.x;
      const uint32_t n = c < nc ? c_in[c] : 0u;
      if (n > (uint32_t)kSlotCap) s_flag = 1u;
      uint32_t t;
      const uint32_t o = n_total + block_exclusive_scan(n, scratch, t);
      if (c < nc) coff[c] = o;
      n_total += t;
    }
    if (threadIdx.x == 0) coff[nc] = n_total;
    if (n_total > (uint32_t)kCandCap) s_flag = 1u;
    __syncthreads();
    const bool overflow = s_flag != 0u;

    if (!overflow) {
      const uint32_t above_all = block_sum(above_local, scratch);
      uint32_t rem = h.k_sel - above_all;  // rank of the threshold inside the list
      // gather the listed patterns of all chunks, chunk by chunk
      for (uint32_t i = threadIdx.x; i < n_total; i += kThreads) {
        int lo = 0, hi = nc - 1;  // last chunk with coff[c] <= i
        while (lo < hi) {
          const int mid = (lo + hi + 1) >> 1;
          if (coff[mid] <= i) lo = mid; else hi = mid - 1;
        }
        cbits[i] = a.slots[((int64_t)head * nc + lo) * kSlotCap + (i - coff[lo])];
      }
      // the listed patterns share bits 31..19; radix over bits 18..9, then 8..0
      uint32_t prefix = 0u, mask = 0u;
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int shift = p == 0 ? 9 : 0;
        const uint32_t nb = p == 0 ? 1024u : 512u;
        for (uint32_t i = threadIdx.x; i < 1024u; i += kThreads) hist[i] = 0u;
        __syncthreads();
        for (uint32_t i = threadIdx.x; i < n_total; i += kThreads) {
          const uint32_t u = cbits[i] & 0x7FFFFu;
          if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
        }
        __syncthreads();
        const uint32_t b = nb - 1 - threadIdx.x;
        const uint32_t cnt = threadIdx.x < nb ? hist[b] : 0u;
        uint32_t tot;
        const uint32_t before = block_exclusive_scan(cnt, scratch, tot);
        if (threadIdx.x < nb && before < rem && rem <= before + cnt) {
          s_digit = b;
          s_rem = rem - before;
        }
        __syncthreads();
        prefix |= s_digit << shift;
        mask |= (nb - 1) << shift;
        rem = s_rem;
        __syncthreads();
      }
      thr = (cbits[0] & ~0x7FFFFu) | prefix;
      need_eq = rem;
      // above / equal counts of the listed entries of the chunks before this one
      const uint32_t lim = coff[chunk];
      uint32_t g = 0, q = 0;
      for (uint32_t i = threadIdx.x; i < lim; i += kThreads) {
        g += cbits[i] > thr;
        q += cbits[i] == thr;
      }
      for (int c = threadIdx.x; c < chunk; c += kThreads) g += c_above[c];
      prev_gt = block_sum(g, scratch);
      prev_eq = block_sum(q, scratch);
    } else {
      uint32_t above;
      thr = radix_over_row(h, rowbits, h.k_sel, hist, above);
      need_eq = h.k_sel - above;
      const int64_t lim = (int64_t)chunk * kChunk < h.rec_begin ? (int64_t)chunk * kChunk : h.rec_begin;
      uint32_t g = 0, q = 0;
      for (int64_t j = h.sink_end + threadIdx.x; j < lim; j += kThreads) {
        const uint32_t u = rowbits[j];
        g += u > thr;
        q += u == thr;
      }
      prev_gt = block_sum(g, scratch);
      prev_eq = block_sum(q, scratch);
    }
    eq_before = prev_eq;
  }
  // output offset of this chunk: mandatory keys, candidates above the
  // threshold and the equal candidates taken, all in the chunks before it
  uint32_t mand_before = 0;
  for (int c = threadIdx.x; c < chunk; c += kThreads) mand_before += chunk_mandatory(h, c);
  mand_before = block_sum(mand_before, scratch);
  const uint32_t taken_before = need_eq < eq_before ? need_eq : eq_before;
  const int64_t out_base = (int64_t)mand_before + prev_gt + taken_before;

  uint32_t flags[4];  // 1: kept, 2: equal to the threshold (kept in index order)
  uint32_t neq = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    flags[e] = 0u;
    if (j >= h.s) continue;
    if (j < h.sink_end || j >= h.rec_begin) { flags[e] = 1u; continue; }
    if (h.k_sel == 0) continue;
    const uint32_t u = vbits[e];
    if (u > thr) flags[e] = 1u;
    else if (u == thr) { flags[e] = 2u; ++neq; }
  }
  uint32_t tot;
  uint32_t eq_rank = eq_before + block_exclusive_scan(neq, scratch, tot);
  uint32_t nkeep = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (flags[e] == 2u) {
      flags[e] = eq_rank < need_eq ? 1u : 0u;
      ++eq_rank;
    }
    nkeep += flags[e];
  }
  const uint32_t pos0 = block_exclusive_scan(nkeep, scratch, tot);
  int64_t o = out_base + pos0;
  const int64_t limit = h.budget;  // never past this head's rows
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (flags[e]) {
      if (o < limit) out[o] = (int32_t)(j0 + e);
      ++o;
    }
  }
}

}  // namespace

size_t select_lds_bytes(int n_chunks) {
  return (size_t)kCandCap * 4 + (size_t)(n_chunks + 1) * 4;
}

hipError_t launch_select(const Layer& L, const SelectArgs& a, bool need_hist, hipStream_t st) {
  SelectArgs args = a;
  void* kargs[] = {&args};
  const dim3 chunks((unsigned)(L.hkv * a.n_chunks));
  hipError_t e;
  if (need_hist) {
    int hkv = L.hkv;
    void* iargs[] = {&args, &hkv};
    e = hipLaunchKernel(reinterpret_cast<const void*>(&init_kernel),
                        dim3((unsigned)((L.hkv * kHistBins + 255) / 256)), dim3(256), iargs, 0, st);
    if (e != hipSuccess) return e;
    e = hipLaunchKernel(reinterpret_cast<const void*>(&hist_kernel), chunks, dim3(kThreads), kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchKernel(reinterpret_cast<const void*>(&filter_kernel), chunks, dim3(kThreads), kargs, 0, st);
  if (e != hipSuccess) return e;
  const size_t lds = select_lds_bytes(a.n_chunks);
  e = ensure_lds(reinterpret_cast<const void*>(&select_kernel), lds);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&select_kernel), chunks, dim3(kThreads), kargs, lds, st);
}

}  // namespace kvc
