// Selection of the retained keys (TideKV, Fig. 3 caption): per KV head, the
// mandatory sink and recent keys plus the top K_h - |mandatory| other keys by
// (score descending, index ascending), written in ascending key order.
//
// Scores are finite and >= +0, so their IEEE-754 bit patterns read as uint32
// order the same way as the values. One 1024-thread workgroup per KV head:
//  1. radix select, 8 bits per round from the top, over the candidate keys'
//     patterns finds the pattern T of the k-th best candidate and how many
//     candidates equal to T must be taken (`need_eq`);
//  2. an ordered compaction keeps mandatory keys, candidates above T, and the
//     first `need_eq` candidates equal to T in index order -- the lower index
//     wins ties -- and writes the kept indices in ascending order.
// The optional max-pool over scores runs first as its own pass.

#include "kvc_internal.h"

namespace kvc {
namespace {

__global__ void __launch_bounds__(256) pool_kernel(PoolArgs a) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= a.total) return;
  const int64_t j = i % a.s;
  const float* row = a.in + (i - j);
  float m = row[j];
  for (int t = 1; t <= a.radius; ++t) {
    if (j - t >= 0) m = fmaxf(m, row[j - t]);
    if (j + t < a.s) m = fmaxf(m, row[j + t]);
  }
  a.out[i] = m;
}

constexpr int kThreads = kSelectThreads;
constexpr int kWaves = kThreads / kWave;

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
    uint32_t w = lane < kWaves ? scratch[lane] : 0u;
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

__global__ void __launch_bounds__(kThreads) select_kernel(SelectArgs a) {
  __shared__ uint32_t hist[256];
  __shared__ uint32_t scan_scratch[kWaves + 1];
  __shared__ uint32_t s_digit, s_remaining;

  const int head = blockIdx.x;
  const int64_t s = a.s;
  const int64_t budget = a.heads.budget[head];
  int32_t* out = a.idx_out + a.heads.offset[head];
  const float* vals = a.vals + (int64_t)head * s;
  const int tid = threadIdx.x;

  if (budget >= s) {
    for (int64_t j = tid; j < s; j += kThreads) out[j] = (int32_t)j;
    return;
  }
  const int64_t sink_end = a.n_sink < s ? a.n_sink : s;
  int64_t rec_begin = s - a.n_recent;
  if (rec_begin < sink_end) rec_begin = sink_end;
  // candidates: [sink_end, rec_begin); mandatory: the rest
  const int64_t n_mand = sink_end + (s - rec_begin);
  const uint32_t k_sel = (uint32_t)(budget - n_mand);

  // ---- 1. radix select of the k_sel-th largest candidate pattern ----
  uint32_t prefix = 0u, mask = 0u, remaining = k_sel;
  const uint32_t* bits = reinterpret_cast<const uint32_t*>(vals);
  if (k_sel > 0) {
    for (int shift = 24; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kThreads) hist[i] = 0u;
      __syncthreads();
      for (int64_t j = sink_end + tid; j < rec_begin; j += kThreads) {
        const uint32_t u = bits[j];
        if ((u & mask) == prefix) atomicAdd(&hist[(u >> shift) & 255u], 1u);
      }
      __syncthreads();
      if (tid < 64) {
        // lane l covers digits 255-4l .. 252-4l (descending)
        uint32_t c[4], loc = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) { c[q] = hist[255 - 4 * tid - q]; loc += c[q]; }
        uint32_t incl = loc;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const uint32_t o = __shfl_up(incl, off);
          if (tid >= off) incl += o;
        }
        uint32_t before = incl - loc;  // candidates on strictly higher digits
        if (before < remaining && remaining <= incl) {
#pragma unroll
          for (int q = 0; q < 4; ++q) {
            if (before < remaining && remaining <= before + c[q]) {
              s_digit = 255u - 4u * tid - q;
              s_remaining = remaining - before;
            }
            before += c[q];
          }
        }
      }
      __syncthreads();
      prefix |= s_digit << shift;
      mask |= 255u << shift;
      remaining = s_remaining;
      __syncthreads();
    }
  }
  const uint32_t thr = prefix;
  const uint32_t need_eq = k_sel > 0 ? remaining : 0u;

  // ---- 2. ordered compaction over contiguous per-thread segments ----
  const int64_t seg = (s + kThreads - 1) / kThreads;
  const int64_t j0 = (int64_t)tid * seg;
  const int64_t j1 = j0 + seg < s ? j0 + seg : s;
  uint32_t n_def = 0, n_eq = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const bool cand = j >= sink_end && j < rec_begin;
    if (!cand) { ++n_def; continue; }
    if (k_sel == 0) continue;
    const uint32_t u = bits[j];
    n_def += u > thr;
    n_eq += u == thr;
  }
  uint32_t eq_total;
  const uint32_t eq_before = block_exclusive_scan(n_eq, scan_scratch, eq_total);
  uint32_t take_eq = 0;
  if (need_eq > eq_before) {
    take_eq = need_eq - eq_before;
    if (take_eq > n_eq) take_eq = n_eq;
  }
  uint32_t kept_total;
  const uint32_t out_base = block_exclusive_scan(n_def + take_eq, scan_scratch, kept_total);
  uint32_t o = out_base, eq_seen = 0;
  for (int64_t j = j0; j < j1; ++j) {
    const bool cand = j >= sink_end && j < rec_begin;
    bool keep = !cand;
    if (cand && k_sel > 0) {
      const uint32_t u = bits[j];
      if (u > thr) keep = true;
      else if (u == thr) { keep = eq_seen < take_eq; ++eq_seen; }
    }
    if (keep) {
      if (o < (uint32_t)budget) out[o] = (int32_t)j;  // never past this head's rows
      ++o;
    }
  }
}

}  // namespace

hipError_t launch_pool(const PoolArgs& a, hipStream_t st) {
  PoolArgs args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)((a.total + 255) / 256));
  return hipLaunchKernel(reinterpret_cast<const void*>(&pool_kernel), grid, dim3(256), kargs, 0, st);
}

hipError_t launch_select(const Layer& L, const SelectArgs& a, hipStream_t st) {
  SelectArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&select_kernel), dim3((unsigned)L.hkv),
                         dim3(kThreads), kargs, 0, st);
}

}  // namespace kvc
