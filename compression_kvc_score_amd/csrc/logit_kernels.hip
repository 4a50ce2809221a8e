// Raw inner-product scores (HillInfer, Algorithmic Simplification: ranking
// needs only the order of the keys and the softmax is monotonic, so keys are
// ranked by Q.K^T alone, without exponentiation or scaling) and their INT8
// form (HillInfer, Streaming Execution and Asymmetric Precision: the products
// in INT8 for the ranking only, the streamed keys cast on the fly, the
// original rows retrieved afterwards).
//
// With W window queries in G heads per KV head, the score of key j is the sum
// of the logits of the rows that see it: one dot product of K[j] with the
// pooled query of those rows -- all W*G rows for the prefix keys j <= S-W, the
// rows i >= j-(S-W) for the later window keys. One launch streams K once:
//
//  - main workgroups own one KV head and a range of prefix keys. Their
//    prologue sums the head's window queries in fp64 (exact for bf16 inputs
//    whose magnitudes span fewer than 2^45) and rounds the pooled query once
//    to fp32; INT8 quantises it per vector.
//  - D/8 lanes share a key row, one 16-byte load each, so a row is one
//    contiguous 256-byte segment; eight rows are in flight per lane group.
//    The partial products are summed over the row's lanes by DPP steps in a
//    fixed order. INT8 rows are quantised by the same lanes (the row maximum
//    by DPP, the codes by round-half-even of x * 127/max) and multiplied with
//    dot4 instructions, exactly.
//  - one more workgroup per window key j = S-W+t (t >= 1) forms the pooled
//    query of rows t .. W-1 the same way and scores that key.
//
// With a histogram buffer the scan also counts the candidates' ranking keys
// per head (signed-key bins of the selection).

#include "kvc_internal.h"
#include "wave_ops.h"

namespace kvc {
namespace {

constexpr int kLThreads = 512;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// 8 bf16 values of one 16-byte load as fp32 (exact).
__device__ __forceinline__ void unpack8(const uint4& v, float (&x)[8]) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    x[2 * i] = bf16_lo(w[i]);
    x[2 * i + 1] = bf16_hi(w[i]);
  }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, false));
}
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
  return __builtin_amdgcn_update_dpp(0, x, CTRL, 0xF, 0xF, false);
}
template <int CTRL>
__device__ __forceinline__ float dpp_keep(float x) {  // every lane reads inside its row
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(x), __float_as_int(x), CTRL, 0xF, 0xF, false));
}

// Sum over a group of LPR (8 or 16) consecutive lanes: an inclusive scan by
// row shifts; the group's last lane holds the total (fixed order).
template <int LPR>
__device__ __forceinline__ float group_sum(float x) {
  x += dpp_f<0x111>(x);
  x += dpp_f<0x112>(x);
  x += dpp_f<0x114>(x);
  if constexpr (LPR == 16) x += dpp_f<0x118>(x);
  return x;
}
template <int LPR>
__device__ __forceinline__ int group_sum_i(int x) {
  x += dpp_i<0x111>(x);
  x += dpp_i<0x112>(x);
  x += dpp_i<0x114>(x);
  if constexpr (LPR == 16) x += dpp_i<0x118>(x);
  return x;
}
// Maximum over the group, in every lane of it: quad swaps, then the mirror
// of each half row (and of the row for 16 lanes).
template <int LPR>
__device__ __forceinline__ float group_max_all(float x) {
  x = fmaxf(x, dpp_keep<0xB1>(x));   // quad_perm [1,0,3,2]
  x = fmaxf(x, dpp_keep<0x4E>(x));   // quad_perm [2,3,0,1]
  x = fmaxf(x, dpp_keep<0x141>(x));  // row_half_mirror
  if constexpr (LPR == 16) x = fmaxf(x, dpp_keep<0x140>(x));  // row_mirror
  return x;
}

// Symmetric INT8 codes of this lane's 8 values given the vector's max |x|
// (the rule of the oracle: round-half-even of x * fp32(127 / max)), packed
// four to a word. Adding 1.5 * 2^23 to the separately rounded product (the
// compiler would otherwise fuse the two into one rounding) leaves
// exactly that rounded integer in the low mantissa bits (|x * r| <= 127), so
// its low byte is the two's-complement code; an all-zero vector (r = 0) gives
// zero codes.
__device__ __forceinline__ void quantize8(const float (&x)[8], float amax, int (&packed)[2]) {
  constexpr float kMagic = 12582912.0f;  // 1.5 * 2^23
  const float r = amax > 0.f ? __fdiv_rn(127.f, amax) : 0.f;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    uint32_t p = 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float prod = x[4 * h + i] * r;
      asm volatile("" : "+v"(prod));  // keep the product's own rounding: no fused multiply-add
      const uint32_t c = __float_as_uint(prod + kMagic) & 0xFFu;
      p |= c << (8 * i);
    }
    packed[h] = (int)p;
  }
}

__device__ __forceinline__ float step_of(float amax) { return amax > 0.f ? __fdiv_rn(amax, 127.f) : 0.f; }

__device__ __forceinline__ uint32_t signed_bin(float v) {
  uint32_t u = __float_as_uint(v);
  if (u == 0x80000000u) u = 0u;
  const uint32_t key = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return key >> 20;  // the selection's bins for signed keys
}

// Score of one key row (this lane's 8 values) against the pooled query.
template <int LPR, bool I8>
__device__ __forceinline__ float row_score(const uint4& kraw, const float (&qf)[8], const int (&q8)[2],
                                           float step_q) {
  float x[8];
  unpack8(kraw, x);
  if constexpr (!I8) {
    float p = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) p = fmaf(qf[i], x[i], p);
    return group_sum<LPR>(p);
  } else {
    float am = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) am = fmaxf(am, fabsf(x[i]));
    am = group_max_all<LPR>(am);
    int k8[2];
    quantize8(x, am, k8);
    int dot = __builtin_amdgcn_sdot4(q8[0], k8[0], 0, false);
    dot = __builtin_amdgcn_sdot4(q8[1], k8[1], dot, false);
    dot = group_sum_i<LPR>(dot);
    return __fmul_rn(__fmul_rn((float)dot, step_q), step_of(am));
  }
}

template <int D, bool I8, bool HIST>
__global__ void __launch_bounds__(kLThreads) logit_scan_kernel(LogitArgs a) {
  constexpr int LPR = D / 8;                   // lanes per key row
  constexpr int GROUPS = kLThreads / LPR;      // key rows per pass
  constexpr int U = 8;                         // rows in flight per lane group
  __shared__ double part[GROUPS][D];
  __shared__ float qbar[D];
  __shared__ float s_amax;
  __shared__ uint32_t lh[HIST ? kHistBins : 1];
  const int grp = threadIdx.x / LPR, l = threadIdx.x % LPR;
  const int s = a.s, w = a.w, G = a.g;
  const int nmain = a.hkv * a.n_split;
  const bool window_wg = (int)blockIdx.x >= nmain;
  // main: (head, split), rows from 0; window: (head, t), rows from t
  const int head = window_wg ? ((int)blockIdx.x - nmain) / (w - 1) : (int)blockIdx.x / a.n_split;
  const int split = window_wg ? 0 : (int)blockIdx.x % a.n_split;
  const int t_first = window_wg ? 1 + ((int)blockIdx.x - nmain) % (w - 1) : 0;
  const int first_win = s - w + 1;  // keys from here on are seen by fewer than all rows
  float* out = a.scores + (int64_t)head * s;
  const uint16_t* kh = a.k + (int64_t)head * a.k_head + 8 * l;

  if constexpr (HIST) {
    for (int i = threadIdx.x; i < kHistBins; i += kLThreads) lh[i] = 0u;
  }

  // ---- pooled query of rows t_first .. W-1: lane group grp sums flattened
  // rows r = t_first*G + grp, + GROUPS, ... (row r = window query r / G of
  // head head*G + r % G), exactly in fp64
  double acc[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  for (int r = t_first * G + grp; r < w * G; r += GROUPS) {
    const uint4 v = *reinterpret_cast<const uint4*>(a.q + (int64_t)(r / G) * a.q_tok +
                                                    (int64_t)(head * G + r % G) * a.q_head + 8 * l);
    float x[8];
    unpack8(v, x);
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] += (double)x[i];
  }
#pragma unroll
  for (int i = 0; i < 8; ++i) part[grp][8 * l + i] = acc[i];
  __syncthreads();
  if (threadIdx.x < D) {
    double t = 0.0;
    for (int g2 = 0; g2 < GROUPS; ++g2) t += part[g2][threadIdx.x];
    qbar[threadIdx.x] = (float)t;
  }
  __syncthreads();
  float qf[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) qf[i] = qbar[8 * l + i];
  int q8[2] = {0, 0};
  float step_q = 0.f;
  if constexpr (I8) {
    if (threadIdx.x < kWave) {
      float m = 0.f;
      for (int i = threadIdx.x; i < D; i += kWave) m = fmaxf(m, fabsf(qbar[i]));
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
      if (threadIdx.x == 0) s_amax = m;
    }
    __syncthreads();
    quantize8(qf, s_amax, q8);
    step_q = step_of(s_amax);
  }

  if (!window_wg) {
    // ---- prefix keys [kb, ke), all seen by every window row
    const int kb = split * a.keys_per_wg;
    const int ke = min(kb + a.keys_per_wg, first_win);
    // two register buffers of U rows per lane group: the next rows load while
    // the current ones are scored; loads are clamped into the range (never
    // conditional), so the compiler can count the ones in flight
    constexpr int STEP = GROUPS * U;
    uint4 ka[U], kb2[U];
    auto load = [&](uint4 (&buf)[U], int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = min(base + u * GROUPS + grp, ke - 1);
        buf[u] = *reinterpret_cast<const uint4*>(kh + (int64_t)key * a.k_tok);
      }
    };
    auto score = [&](const uint4 (&buf)[U], int base) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int key = base + u * GROUPS + grp;
        const float sc = row_score<LPR, I8>(buf[u], qf, q8, step_q);
        if (l == LPR - 1 && key < ke) {
          out[key] = sc;
          if (HIST && key >= a.sink_end && key < a.rec_begin) atomicAdd(&lh[signed_bin(sc)], 1u);
        }
      }
    };
    if (kb < ke) load(ka, kb);
    for (int base = kb; base < ke; base += 2 * STEP) {
      if (base + STEP < ke) load(kb2, base + STEP);
      score(ka, base);
      if (base + STEP < ke) {
        if (base + 2 * STEP < ke) load(ka, base + 2 * STEP);
        score(kb2, base + STEP);
      }
    }
  } else if (grp == 0) {
    // ---- the window key j = S-W+t_first, seen by rows t_first .. W-1
    const int key = s - w + t_first;
    const uint4 kraw = *reinterpret_cast<const uint4*>(kh + (int64_t)key * a.k_tok);
    const float sc = row_score<LPR, I8>(kraw, qf, q8, step_q);
    if (l == LPR - 1) {
      out[key] = sc;
      if (HIST && key >= a.sink_end && key < a.rec_begin) atomicAdd(&lh[signed_bin(sc)], 1u);
    }
  }

  if constexpr (HIST) {
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)head * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += kLThreads)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
  }
}

template <int D, bool I8>
const void* logit_fn(bool hist) {
  return hist ? reinterpret_cast<const void*>(&logit_scan_kernel<D, I8, true>)
              : reinterpret_cast<const void*>(&logit_scan_kernel<D, I8, false>);
}

}  // namespace

hipError_t launch_logit_scan(const Layer& L, const LogitArgs& a, bool int8, hipStream_t st) {
  LogitArgs args = a;
  void* kargs[] = {&args};
  const bool hist = a.hist != nullptr;
  const void* fn = L.d == 128 ? (int8 ? logit_fn<128, true>(hist) : logit_fn<128, false>(hist))
                              : (int8 ? logit_fn<64, true>(hist) : logit_fn<64, false>(hist));
  const dim3 grid((unsigned)(L.hkv * (a.n_split + L.w - 1)));  // + one workgroup per window key
  return hipLaunchKernel(fn, grid, dim3(kLThreads), kargs, 0, st);
}

}  // namespace kvc
