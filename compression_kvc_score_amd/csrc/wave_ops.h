// Wavefront-wide integer scans and counts for gfx9 wave64, built from DPP row
// operations and ballots instead of LDS permutes (a __shfl_up/__shfl_xor step
// is a ds_bpermute round trip through LDS; these stay in the VALU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvc {

// DPP controls (GFX9 encoding): row_shr:n = 0x110 + n; row_bcast:15 = 0x142
// (lane 15 of each row to the next row); row_bcast:31 = 0x143 (lane 31 to
// rows 2 and 3).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint32_t dpp_or_zero(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, ROW_MASK, 0xF, false);
}

// Inclusive prefix sum over the 64 lanes (all lanes active).
__device__ __forceinline__ uint32_t wave_inclusive_sum(uint32_t x) {
  x += dpp_or_zero<0x111, 0xF>(x);
  x += dpp_or_zero<0x112, 0xF>(x);
  x += dpp_or_zero<0x114, 0xF>(x);
  x += dpp_or_zero<0x118, 0xF>(x);
  x += dpp_or_zero<0x142, 0xA>(x);
  x += dpp_or_zero<0x143, 0xC>(x);
  return x;
}

__device__ __forceinline__ uint32_t wave_total(uint32_t incl) {
  return (uint32_t)__builtin_amdgcn_readlane((int)incl, 63);
}

// Number of lanes where pred holds, in every lane (a ballot and a popcount).
__device__ __forceinline__ uint32_t wave_count(bool pred) { return (uint32_t)__popcll(__ballot(pred)); }

// Set lanes of mask below this lane.
__device__ __forceinline__ uint32_t lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

}  // namespace kvc
