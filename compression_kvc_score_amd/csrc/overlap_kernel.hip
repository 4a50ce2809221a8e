// Overlap coefficient of two retained index sets (HeteroCache summary, Key
// Contributions item 1): per KV head, |A & B| / min(|A|, |B|). Both sets of a
// head are ascending and of the same size. One workgroup per head copies B
// into LDS (when it fits) and each thread looks its entries of A up in it by
// binary search; the hits are summed over the workgroup.

#include "kvc_internal.h"
#include "wave_ops.h"

namespace kvc {
namespace {

constexpr int kOThreads = 1024;
constexpr int kOCap = 15360;  // entries of B held in LDS (60 KiB)

// Position of the first entry >= x among B[0, n) (ascending).
template <typename P>
__device__ __forceinline__ int64_t lower_bound(P B, int64_t n, int32_t x) {
  int64_t lo = 0, hi = n;
  while (lo < hi) {
    const int64_t mid = (lo + hi) >> 1;
    if (B[mid] < x) lo = mid + 1; else hi = mid;
  }
  return lo;
}

__global__ void __launch_bounds__(kOThreads) overlap_kernel(OverlapArgs a) {
  __shared__ uint32_t part[kOThreads / kWave];
  __shared__ int32_t lb[kOCap];
  const int head = blockIdx.x;
  const int64_t o = a.heads.offset[head];
  const int64_t n = a.heads.offset[head + 1] - o;
  const int32_t* A = a.idx_a + o;
  const int32_t* B = a.idx_b + o;
  const bool in_lds = n <= kOCap;
  if (in_lds) {
    for (int64_t i = threadIdx.x; i < n; i += kOThreads) lb[i] = B[i];
    __syncthreads();
  }
  uint32_t hits = 0;
  for (int64_t i = threadIdx.x; i < n; i += kOThreads) {
    const int32_t x = A[i];
    if (in_lds) {
      const int64_t p = lower_bound(lb, n, x);
      hits += p < n && lb[p] == x;
    } else {
      const int64_t p = lower_bound(B, n, x);
      hits += p < n && B[p] == x;
    }
  }
  const uint32_t tot = wave_total(wave_inclusive_sum(hits));
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = tot;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0;
    for (int w = 0; w < kOThreads / kWave; ++w) t += part[w];
    a.out[head] = n > 0 ? __fdiv_rn((float)t, (float)n) : 1.f;
  }
}

}  // namespace

hipError_t launch_overlap(const OverlapArgs& a, int hkv, hipStream_t st) {
  OverlapArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&overlap_kernel), dim3((unsigned)hkv), dim3(kOThreads), kargs,
                         0, st);
}

}  // namespace kvc
