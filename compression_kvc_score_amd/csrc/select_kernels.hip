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
//           and appends the candidates inside b* to a short per-head list.
//  resolve  one workgroup per head radix-selects, among the listed
//           candidates and in LDS, the exact pattern T of the k-th best and
//           how many candidates equal to T are taken (the lowest indices:
//           ties go to the lower index). From per-chunk counts it lays out
//           every chunk's output range. If a bin holds more candidates than
//           the list can take (heavily tied scores), it selects by a radix
//           over the head's whole score row instead -- same result, slower.
//  compact  every chunk workgroup writes its kept indices, ascending, to its
//           range.
//
// All counts are integers and the candidate list is only used as a multiset,
// so the output does not depend on the order in which workgroups run.

#include "kvc_internal.h"

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
  uint32_t incl = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  if (lane == 63) scratch[wave] = incl;
  __syncthreads();
  if (wave == 0) {
    const uint32_t w = lane < kWaves ? scratch[lane] : 0u;
    uint32_t wi = w;
#pragma unroll
    for (int off = 1; off < kWaves; off <<= 1) {
      const uint32_t o = __shfl_up(wi, off);
      if (lane >= off) wi += o;
    }
    if (lane < kWaves) scratch[lane] = wi - w;  // exclusive wave offsets
    if (lane == kWaves - 1) scratch[kWaves] = wi;
  }
  __syncthreads();
  const uint32_t res = scratch[wave] + incl - v;
  total = scratch[kWaves];
  __syncthreads();
  return res;
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
  if (i < hkv) a.cand_count[i] = 0u;
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
// filter: count candidates above b* per chunk, list the candidates inside b*.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) filter_kernel(SelectArgs a) {
  __shared__ uint32_t scratch[kWaves + 1];
  const int head = blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  const HeadGeom h = head_geom(a, head);
  if (h.keep_all || h.k_sel == 0) return;
  uint32_t bstar, above_all;
  find_bin(a.hist + (int64_t)head * kHistBins, h.k_sel, scratch, bstar, above_all);

  const float* vals = a.vals + (int64_t)head * h.s;
  const int64_t j0 = (int64_t)chunk * kChunk + 4 * threadIdx.x;
  uint32_t above = 0, nin = 0;
  uint32_t bits[4];
  bool in[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    in[e] = false;
    bits[e] = 0u;
    if (j < h.s && j >= h.sink_end && j < h.rec_begin) {
      bits[e] = __float_as_uint(vals[j]);
      const uint32_t b = bin_of(bits[e]);
      above += b > bstar;
      in[e] = b == bstar;
      nin += in[e];
    }
  }
  // wave-aggregated append of the in-bin candidates
  const int lane = threadIdx.x & 63;
  uint32_t incl = nin;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t o = __shfl_up(incl, off);
    if (lane >= off) incl += o;
  }
  const uint32_t wave_total = __shfl(incl, 63);
  uint32_t base = 0;
  if (lane == 63 && wave_total) base = atomicAdd(&a.cand_count[head], wave_total);
  base = __shfl(base, 63);
  uint32_t pos = base + incl - nin;
  uint2* list = a.cand + (int64_t)head * kCandCap;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (in[e]) {
      if (pos < (uint32_t)kCandCap) list[pos] = make_uint2(bits[e], (uint32_t)(j0 + e));
      ++pos;
    }
  }
  uint32_t tot;
  block_exclusive_scan(above, scratch, tot);
  if (threadIdx.x == 0) a.chunk_above[(int64_t)head * a.n_chunks + chunk] = tot;
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

// Slow path of resolve: k-th largest candidate pattern by a radix over the
// whole score row of the head (8 bits per round from the top).
__device__ uint32_t radix_over_row(const SelectArgs& a, const HeadGeom& h, const uint32_t* bits,
                                   uint32_t k, uint32_t* hist256, uint32_t* scratch,
                                   uint32_t& above) {
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
      uint32_t incl = loc;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const uint32_t o = __shfl_up(incl, off);
        if (l >= off) incl += o;
      }
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

// ---------------------------------------------------------------------------
// resolve: exact threshold per head and every chunk's output range.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) resolve_kernel(SelectArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint32_t* cbits = reinterpret_cast<uint32_t*>(smem);        // kCandCap
  uint32_t* gt_c = cbits + kCandCap;                           // n_chunks
  uint32_t* eq_c = gt_c + a.n_chunks;                          // n_chunks
  __shared__ uint32_t hist[1024];
  __shared__ uint32_t scratch[kWaves + 1];
  __shared__ uint32_t s_digit, s_rem;

  const int head = blockIdx.x;
  const HeadGeom h = head_geom(a, head);
  SelectHead* out = a.head_out + head;
  int64_t* ranges = a.chunk_range + (int64_t)head * a.n_chunks * 2;
  if (h.keep_all) return;  // compact writes 0..s-1 directly

  for (int c = threadIdx.x; c < a.n_chunks; c += kThreads) { gt_c[c] = 0u; eq_c[c] = 0u; }
  uint32_t thr = 0xFFFFFFFFu, need_eq = 0u;  // k_sel == 0: choose no candidate
  const uint32_t* rowbits = reinterpret_cast<const uint32_t*>(a.vals + (int64_t)head * h.s);
  const uint32_t n_cand = h.k_sel ? a.cand_count[head] : 0u;
  const bool overflow = n_cand > (uint32_t)kCandCap;
  __syncthreads();

  if (h.k_sel > 0 && !overflow) {
    // candidates above b*, over all chunks
    uint32_t above_local = 0;
    for (int c = threadIdx.x; c < a.n_chunks; c += kThreads)
      above_local += a.chunk_above[(int64_t)head * a.n_chunks + c];
    uint32_t above_all;
    block_exclusive_scan(above_local, scratch, above_all);
    uint32_t rem = h.k_sel - above_all;  // rank of the threshold inside the listed candidates
    const uint2* list = a.cand + (int64_t)head * kCandCap;
    for (uint32_t i = threadIdx.x; i < n_cand; i += kThreads) cbits[i] = list[i].x;
    // the listed candidates share bits 30..19; radix over bits 18..9 then 8..0
    uint32_t prefix = 0u, mask = 0u;
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int shift = p == 0 ? 9 : 0;
      const uint32_t nb = p == 0 ? 1024u : 512u;
      for (uint32_t i = threadIdx.x; i < 1024u; i += kThreads) hist[i] = 0u;
      __syncthreads();
      for (uint32_t i = threadIdx.x; i < n_cand; i += kThreads) {
        const uint32_t u = cbits[i] & 0x7FFFFu;
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & (nb - 1)], 1u);
      }
      __syncthreads();
      // descending scan over nb bins, one bin per thread
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
    thr = (cbits[0] & ~0x7FFFFu) | prefix;  // listed candidates all carry b* in bits 31..19
    need_eq = rem;
    // per-chunk counts of listed candidates above / equal to the threshold
    for (uint32_t i = threadIdx.x; i < n_cand; i += kThreads) {
      const uint2 e = list[i];
      const int64_t c = (int64_t)e.y / kChunk;
      if (e.x > thr) atomicAdd(&gt_c[c], 1u);
      else if (e.x == thr) atomicAdd(&eq_c[c], 1u);
    }
    __syncthreads();
    for (int c = threadIdx.x; c < a.n_chunks; c += kThreads)
      gt_c[c] += a.chunk_above[(int64_t)head * a.n_chunks + c];
    __syncthreads();
  } else if (h.k_sel > 0) {
    uint32_t above;
    thr = radix_over_row(a, h, rowbits, h.k_sel, hist, scratch, above);
    need_eq = h.k_sel - above;
    for (int64_t j = h.sink_end + threadIdx.x; j < h.rec_begin; j += kThreads) {
      const uint32_t u = rowbits[j];
      if (u > thr) atomicAdd(&gt_c[j / kChunk], 1u);
      else if (u == thr) atomicAdd(&eq_c[j / kChunk], 1u);
    }
    __syncthreads();
  }

  // chunk ranges: equal candidates are taken in index order until need_eq
  uint32_t eq_run = 0, out_run = 0;
  for (int base = 0; base < a.n_chunks; base += kThreads) {
    const int c = base + threadIdx.x;
    const uint32_t e = c < a.n_chunks ? eq_c[c] : 0u;
    uint32_t etot;
    const uint32_t eb = eq_run + block_exclusive_scan(e, scratch, etot);
    uint32_t take = 0;
    if (need_eq > eb) take = need_eq - eb < e ? need_eq - eb : e;
    const uint32_t kept = c < a.n_chunks ? chunk_mandatory(h, c) + gt_c[c] + take : 0u;
    uint32_t ktot;
    const uint32_t ob = out_run + block_exclusive_scan(kept, scratch, ktot);
    if (c < a.n_chunks) {
      ranges[2 * c] = ob;
      ranges[2 * c + 1] = eb;
    }
    eq_run += etot;
    out_run += ktot;
  }
  if (threadIdx.x == 0) {
    out->thr = thr;
    out->need_eq = need_eq;
  }
}

// ---------------------------------------------------------------------------
// compact: kept indices of one chunk, ascending, at the chunk's output range.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(kThreads) compact_kernel(SelectArgs a) {
  __shared__ uint32_t scratch[kWaves + 1];
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
  const uint32_t thr = a.head_out[head].thr;
  const uint32_t need_eq = a.head_out[head].need_eq;
  const int64_t* rg = a.chunk_range + ((int64_t)head * a.n_chunks + chunk) * 2;
  const int64_t out_base = rg[0];
  const uint32_t eq_base = (uint32_t)rg[1];
  const float* vals = a.vals + (int64_t)head * h.s;

  uint32_t flags[4];  // 1: definitely kept, 2: equal to the threshold
  uint32_t neq = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    flags[e] = 0u;
    if (j >= h.s) continue;
    if (j < h.sink_end || j >= h.rec_begin) { flags[e] = 1u; continue; }
    if (h.k_sel == 0) continue;
    const uint32_t u = __float_as_uint(vals[j]);
    if (u > thr) flags[e] = 1u;
    else if (u == thr) { flags[e] = 2u; ++neq; }
  }
  uint32_t tot;
  uint32_t eq_rank = eq_base + block_exclusive_scan(neq, scratch, tot);
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

size_t resolve_lds_bytes(int n_chunks) {
  return (size_t)kCandCap * 4 + (size_t)n_chunks * 8;
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
  const size_t lds = resolve_lds_bytes(a.n_chunks);
  e = ensure_lds(reinterpret_cast<const void*>(&resolve_kernel), lds);
  if (e != hipSuccess) return e;
  e = hipLaunchKernel(reinterpret_cast<const void*>(&resolve_kernel), dim3((unsigned)L.hkv),
                      dim3(kThreads), kargs, lds, st);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(reinterpret_cast<const void*>(&compact_kernel), chunks, dim3(kThreads), kargs, 0, st);
}

}  // namespace kvc
