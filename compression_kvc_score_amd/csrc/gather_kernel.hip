// Gather of the retained cache (TideKV, Fig. 2 caption): the selected K and V
// rows copied bit for bit into dense head-major blocks, and their absolute
// positions. One thread moves one 16-byte chunk of K and the same chunk of V;
// consecutive threads cover consecutive chunks of a row, so both the reads
// (one contiguous row segment per key) and the writes are coalesced.

#include <algorithm>

#include "kvc_internal.h"

namespace kvc {
namespace {

__global__ void __launch_bounds__(256) gather_kernel(GatherArgs a) {
  const int cpr = a.d / 8;  // 16-byte chunks per row
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.total_rows * cpr) return;
  const int64_t row = t / cpr;
  const int c = (int)(t % cpr);
  int g = 0;
  while (g + 1 < a.hkv && a.heads.offset[g + 1] <= row) ++g;
  int64_t j = a.idx[row];
  j = j < 0 ? 0 : (j >= a.s ? a.s - 1 : j);  // keep every read inside K and V
  const uint4 kv = *reinterpret_cast<const uint4*>(a.k + j * a.k_tok + (int64_t)g * a.k_head + c * 8);
  const uint4 vv = *reinterpret_cast<const uint4*>(a.v + j * a.v_tok + (int64_t)g * a.v_head + c * 8);
  *reinterpret_cast<uint4*>(a.k_out + row * a.d + c * 8) = kv;
  *reinterpret_cast<uint4*>(a.v_out + row * a.d + c * 8) = vv;
  if (c == 0) a.pos_out[row] = (int32_t)(a.pos_offset + j);
}

// Immediate eviction appends each prompt chunk behind the keys a head has
// retained so far (TideKV, Fig. 1 caption, schedule (c)); the arena is
// head-major, so one thread moves one 16-byte chunk of a K row and of the V
// row, reading the token-major chunk and writing the arena tail coalesced.
// One launch serves up to two chunks (blockIdx.y picks the chunk).
__global__ void __launch_bounds__(256) append_kernel(AppendJobs jobs) {
  const AppendArgs& a = jobs.job[blockIdx.y];
  const int cpr = a.d / 8;
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= a.n * a.hkv * cpr) return;
  const int c = (int)(t % cpr);
  const int64_t r = t / cpr;
  const int g = (int)(r / a.n);
  const int64_t tok = r % a.n;
  const int64_t dst = ((int64_t)g * a.cap + a.row0 + tok) * a.d + c * 8;
  const uint4 kv = *reinterpret_cast<const uint4*>(a.k + tok * a.k_tok + (int64_t)g * a.k_head + c * 8);
  const uint4 vv = *reinterpret_cast<const uint4*>(a.v + tok * a.v_tok + (int64_t)g * a.v_head + c * 8);
  *reinterpret_cast<uint4*>(a.k_arena + dst) = kv;
  *reinterpret_cast<uint4*>(a.v_arena + dst) = vv;
  if (c == 0) a.pos_arena[(int64_t)g * a.cap + a.row0 + tok] = (int32_t)(a.pos0 + tok);
}

}  // namespace

hipError_t launch_append(const AppendArgs* jobs, int n_jobs, hipStream_t st) {
  AppendJobs args{};
  int n = 0;
  int64_t threads = 0;
  for (int i = 0; i < n_jobs && n < 2; ++i) {
    if (jobs[i].n == 0) continue;
    args.job[n++] = jobs[i];
    threads = std::max<int64_t>(threads, jobs[i].n * jobs[i].hkv * (jobs[i].d / 8));
  }
  if (n == 0) return hipSuccess;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)((threads + 255) / 256), (unsigned)n);
  return hipLaunchKernel(reinterpret_cast<const void*>(&append_kernel), grid, dim3(256), kargs, 0, st);
}

hipError_t launch_gather(const GatherArgs& a, hipStream_t st) {
  if (a.total_rows == 0) return hipSuccess;
  GatherArgs args = a;
  void* kargs[] = {&args};
  const int64_t threads = a.total_rows * (a.d / 8);
  const dim3 grid((unsigned)((threads + 255) / 256));
  return hipLaunchKernel(reinterpret_cast<const void*>(&gather_kernel), grid, dim3(256), kargs, 0, st);
}

}  // namespace kvc
