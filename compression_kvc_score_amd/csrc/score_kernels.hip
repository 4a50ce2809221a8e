// Two-pass blockwise scoring on gfx950 (TideKV, Fig. 3 caption).
//
// Work decomposition (both passes): one workgroup of up to 8 wavefronts
// scans `blocks_per_wg` consecutive key blocks of one KV head; in every block
// each wavefront owns one or more 32-key tiles. The G*W query rows of the
// head (its window queries) are staged once per workgroup in LDS and stay
// stationary; K streams from HBM straight into VGPRs in the bf16 MFMA operand
// layout, one tile ahead of the math.
//
// The contraction Q_win . K^T runs on v_mfma_f32_32x32x16_bf16. The k-index
// of the MFMA is a sum index, so any assignment of head-dimension chunks to
// k-slots works as long as Q and K use the same one: lane half h (lanes
// 32h..32h+31) feeds the contiguous half [h*D/2, (h+1)*D/2) of a row, one
// 16-byte chunk per MFMA step. Each lane therefore loads one contiguous
// D-byte run of its key row.
//
// Pass 1 computes K-tile x Q^T so that every lane owns one query row and 16
// keys of each tile: the online (max, sum-exp) state is lane-private and the
// cross-lane merge happens once per workgroup. Pass 2 computes Q x K^T so
// that every lane owns one key and 16 query rows: the per-key pooling over
// the group's window rows is an in-register sum plus one lane-half exchange.
// exp runs in base 2 on v_exp_f32 with the scale folded into one FMA.
//
// Latency hiding: the next tile's loads are issued unconditionally before
// the current tile is computed (so the compiler never waits on them early),
// and within a tile the MFMAs of row tile t+1 are issued before the VALU
// work of row tile t.

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroups are dispatched round-robin over the 8 XCDs. Give each XCD a
// contiguous run of work items so that the workgroups of one KV head share
// that XCD's L2 (its staged queries and normalisers).
__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  if ((nb & 7) != 0) return bid;
  return (bid & 7) * (nb >> 3) + (bid >> 3);
}

// Merge two (max, sum) log-sum-exp states in base-2 units scaled by c.
__device__ __forceinline__ void lse_merge(float& m, float& z, float m2, float z2, float c) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;  // both empty
  z = z * exp2_raw((m - mn) * c) + z2 * exp2_raw((m2 - mn) * c);
  m = mn;
}

template <int D>
__device__ __forceinline__ void stage_queries(const ScoreArgs& a, int head, int rows_pad,
                                              uint16_t* qs) {
  constexpr int CH = D / 8;       // 16-byte chunks per row
  constexpr int PITCH = D + 8;    // +16 B per row: ds_read_b128 across rows is conflict free
  for (int idx = threadIdx.x; idx < rows_pad * CH; idx += blockDim.x) {
    const int r = idx / CH, c = idx % CH;
    uint4 v = make_uint4(0u, 0u, 0u, 0u);
    if (r < a.rows) {
      const int hh = r / a.w, i = r % a.w;
      const int h = head * a.g + hh;
      v = *reinterpret_cast<const uint4*>(a.q + (int64_t)i * a.q_tok + (int64_t)h * a.q_head + c * 8);
    }
    *reinterpret_cast<uint4*>(qs + r * PITCH + c * 8) = v;
  }
}

// Lane's K operand for one 32-key tile: key `key` (clamped into range; the
// caller masks keys >= s), half `half` of the head dimension.
template <int D>
__device__ __forceinline__ void load_key_frag(const ScoreArgs& a, int head, int key, int half,
                                              uint4 (&kf)[D / 16]) {
  const int kk = key < a.s ? key : a.s - 1;
  const uint16_t* src = a.k + (int64_t)kk * a.k_tok + (int64_t)head * a.k_head + half * (D / 2);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) kf[c] = *reinterpret_cast<const uint4*>(src + 8 * c);
}

// The 32-key tiles one wavefront visits: in each of the workgroup's blocks,
// tiles wave, wave + nwaves, ... (block / 32 / nwaves of them), in increasing
// key order. The first `clean` tiles hold only keys that every window query
// sees; the rest (at the end of the prompt) need the causal mask. kbase(k)
// of any k >= n names keys past the range, which loads clamp into it.
struct TileSeq {
  int b0, block, nwaves, tpw, wave;
  int n, clean;
  __device__ __forceinline__ int kbase(int k) const {
    const int b = b0 + k / tpw, j = k % tpw;
    return b * block + (j * nwaves + wave) * kKeyTile;
  }
};

__device__ __forceinline__ TileSeq tile_seq(const ScoreArgs& a, int split, int wave, int nwaves,
                                            int first_hidden) {
  TileSeq q;
  q.b0 = split * a.blocks_per_wg;
  const int b1 = min(q.b0 + a.blocks_per_wg, a.n_blocks);
  q.block = a.block;
  q.nwaves = nwaves;
  q.tpw = a.block / (kKeyTile * nwaves);
  q.wave = wave;
  q.n = (b1 - q.b0) * q.tpw;
  q.clean = q.n;
  while (q.clean > 0 && q.kbase(q.clean - 1) + kKeyTile > first_hidden) --q.clean;
  return q;
}

// One row tile of the Q_win.K^T contraction for the lane's 32-key tile.
// KROWS: the MFMA rows are the keys (pass 1: lane = one query row, 16 keys);
// otherwise the rows are the query rows (pass 2: lane = one key, 16 rows).
template <int D, bool KROWS>
__device__ __forceinline__ f32x16_t contract_row_tile(const uint16_t* qs, const uint4 (&kf)[D / 16],
                                                      int t, int half, int l32) {
  constexpr int PITCH = D + 8;
  constexpr int NCH = D / 16;
  const uint16_t* qrow = qs + (t * kRowTile + l32) * PITCH + half * (D / 2);
  f32x16_t acc = {};
#pragma unroll
  for (int st = 0; st < NCH; ++st) {
    const uint4 qf = *reinterpret_cast<const uint4*>(qrow + st * 8);
    acc = KROWS ? mfma32x32x16(kf[st], qf, acc) : mfma32x32x16(qf, kf[st], acc);
  }
  return acc;
}

__device__ __forceinline__ float max16(const f32x16_t& v) {
  const float a = fmaxf(fmaxf(v[0], v[1]), v[2]);
  const float b = fmaxf(fmaxf(v[3], v[4]), v[5]);
  const float c = fmaxf(fmaxf(v[6], v[7]), v[8]);
  const float d = fmaxf(fmaxf(v[9], v[10]), v[11]);
  const float e = fmaxf(fmaxf(v[12], v[13]), v[14]);
  return fmaxf(fmaxf(fmaxf(a, b), c), fmaxf(fmaxf(d, e), v[15]));
}

// ---------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------

// Online (max, sum-exp) update of the lane's query row in one row tile with
// the 16 logits it holds (keys kbase + 8*(e/4) + 4*half + e%4).
template <bool EDGE>
__device__ __forceinline__ void lse_update(const ScoreArgs& a, f32x16_t acc, int kbase, int half,
                                           int qpos, float& mrun, float& zrun) {
  if constexpr (EDGE) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + 4 * half + (e & 3);
      if (key >= a.s || key > qpos) acc[e] = -INFINITY;
    }
  }
  const float mnew = fmaxf(mrun, max16(acc));
  if (EDGE && mnew == -INFINITY) return;  // nothing visible to this row yet
  const float mc = mnew * a.c;
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int e = 0; e < 16; e += 2) {
    s0 += exp2_raw(fmaf(acc[e], a.c, -mc));
    s1 += exp2_raw(fmaf(acc[e + 1], a.c, -mc));
  }
  zrun = zrun * exp2_raw((mrun - mnew) * a.c) + (s0 + s1);
  mrun = mnew;
}

template <int D, int NRT, bool EDGE>
__device__ __forceinline__ void pass1_tile(const ScoreArgs& a, const uint16_t* qs,
                                           const uint4 (&kf)[D / 16], int kbase, int half,
                                           int l32, const int (&qpos)[NRT],
                                           float (&mrun)[NRT], float (&zrun)[NRT]) {
  f32x16_t acc[2];
  acc[0] = contract_row_tile<D, true>(qs, kf, 0, half, l32);
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    if (t + 1 < NRT) acc[(t + 1) & 1] = contract_row_tile<D, true>(qs, kf, t + 1, half, l32);
    lse_update<EDGE>(a, acc[t & 1], kbase, half, qpos[t], mrun[t], zrun[t]);
    __builtin_amdgcn_sched_barrier(0);  // at most two row tiles of operands live
  }
}

// Split-local (max, sum-exp) per query row.
template <int D, int NRT>
__global__ void __launch_bounds__(512) pass1_kernel(ScoreArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem);
  constexpr int NCH = D / 16;
  constexpr int ROWS_PAD = NRT * kRowTile;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int head = work / a.n_split;
  const int split = work % a.n_split;
  // The first workgroup of each head clears that head's selection histogram,
  // which pass 2 fills after this kernel has finished.
  if (a.hist != nullptr && split == 0) {
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) a.hist[(int64_t)head * kHistBins + i] = 0u;
  }
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nwaves = blockDim.x >> 6;
  const int first_hidden = a.s - a.w + 1;  // keys from here on are after some window query
  const TileSeq seq = tile_seq(a, split, wave, nwaves, first_hidden);
  uint4 ka[NCH], kb[NCH];
  load_key_frag<D>(a, head, seq.kbase(0) + l32, half, ka);  // streams in during staging
  stage_queries<D>(a, head, ROWS_PAD, qs);
  __syncthreads();

  float mrun[NRT], zrun[NRT];
  int qpos[NRT];  // prompt position of this lane's query row in tile t (-1: padding row)
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    mrun[t] = -INFINITY;
    zrun[t] = 0.f;
    const int r = t * kRowTile + l32;
    qpos[t] = r < a.rows ? a.s - a.w + (r % a.w) : -1;
  }

  int k = 0;
  for (; k + 1 < seq.clean; k += 2) {
    load_key_frag<D>(a, head, seq.kbase(k + 1) + l32, half, kb);
    pass1_tile<D, NRT, false>(a, qs, ka, seq.kbase(k), half, l32, qpos, mrun, zrun);
    load_key_frag<D>(a, head, seq.kbase(k + 2) + l32, half, ka);
    pass1_tile<D, NRT, false>(a, qs, kb, seq.kbase(k + 1), half, l32, qpos, mrun, zrun);
  }
  if (k < seq.clean) pass1_tile<D, NRT, false>(a, qs, ka, seq.kbase(k), half, l32, qpos, mrun, zrun);
  for (k = seq.clean; k < seq.n; ++k) {
    load_key_frag<D>(a, head, seq.kbase(k) + l32, half, ka);
    pass1_tile<D, NRT, true>(a, qs, ka, seq.kbase(k), half, l32, qpos, mrun, zrun);
  }

  // Lanes l and l+32 hold the same query row over different keys.
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const float mo = __shfl_xor(mrun[t], 32);
    const float zo = __shfl_xor(zrun[t], 32);
    lse_merge(mrun[t], zrun[t], mo, zo, a.c);
  }

  // Merge the wavefronts in a fixed order through LDS (the staged queries are dead).
  __syncthreads();
  float2* red = reinterpret_cast<float2*>(smem);
  if (half == 0) {
#pragma unroll
    for (int t = 0; t < NRT; ++t) red[wave * ROWS_PAD + t * kRowTile + l32] = make_float2(mrun[t], zrun[t]);
  }
  __syncthreads();
  for (int r = threadIdx.x; r < a.rows; r += blockDim.x) {
    float m = -INFINITY, z = 0.f;
    for (int wv = 0; wv < nwaves; ++wv) {
      const float2 p = red[wv * ROWS_PAD + r];
      lse_merge(m, z, p.x, p.y, a.c);
    }
    reinterpret_cast<float2*>(a.part)[((int64_t)head * a.n_split + split) * ROWS_PAD + r] = make_float2(m, z);
  }
}

// ---------------------------------------------------------------------------
// Combine the split partials of each query row into (m, Z), natural-log units.
// One workgroup per (KV head, 32-row tile): 8 lanes per row share the splits.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) combine_kernel(ScoreArgs a, int rows_pad) {
  __shared__ float2 red[8][kRowTile];
  const int head = blockIdx.x / (rows_pad / kRowTile);
  const int tile = blockIdx.x % (rows_pad / kRowTile);
  const int rl = threadIdx.x & 31, sl = threadIdx.x >> 5;
  const int r = tile * kRowTile + rl;
  const float2* part = reinterpret_cast<const float2*>(a.part) + (int64_t)head * a.n_split * rows_pad;

  float2 v[kMaxSplit / 8];
#pragma unroll
  for (int u = 0; u < kMaxSplit / 8; ++u) {
    const int sp = sl + 8 * u;
    v[u] = (sp < a.n_split && r < a.rows) ? part[(int64_t)sp * rows_pad + r] : make_float2(-INFINITY, 0.f);
  }
  float m = -INFINITY, z = 0.f;
#pragma unroll
  for (int u = 0; u < kMaxSplit / 8; ++u) lse_merge(m, z, v[u].x, v[u].y, a.c);
  red[sl][rl] = make_float2(m, z);
  __syncthreads();
  if (sl == 0 && r < a.rows) {
    for (int k = 1; k < 8; ++k) lse_merge(m, z, red[k][rl].x, red[k][rl].y, a.c);
    const int hh = r / a.w, i = r % a.w;
    const int h = head * a.g + hh;
    a.m_out[(int64_t)h * a.w + i] = m * a.scale;
    a.z_out[(int64_t)h * a.w + i] = z;
  }
}

// ---------------------------------------------------------------------------
// Pass 2
// ---------------------------------------------------------------------------

// Add the lane key's normalised weights of row tile t (rows
// t*32 + 8*(e/4) + 4*half + e%4) to the running sums.
template <bool EDGE>
__device__ __forceinline__ void weight_sum(const ScoreArgs& a, const f32x16_t& acc,
                                           const float* bias, int t, int key, int half,
                                           float& s0, float& s1) {
  const float* bt = bias + t * kRowTile + 4 * half;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    const float4 bq = *reinterpret_cast<const float4*>(bt + 8 * q4);
    const float bb[4] = {bq.x, bq.y, bq.z, bq.w};
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float p = exp2_raw(fmaf(acc[4 * q4 + e4], a.c, -bb[e4]));
      if constexpr (EDGE) {
        const int r = t * kRowTile + 8 * q4 + 4 * half + e4;
        const int qp = a.s - a.w + (r % a.w);
        if (key >= a.s || r >= a.rows || key > qp) p = 0.f;
      }
      if (e4 & 1) s1 += p; else s0 += p;
    }
  }
}

// One 32-key tile of pass 2: the lane's key collects exp(l - m)/Z over all
// query rows of the head; lanes l and l+32 then add their row halves.
template <int D, int NRT, bool EDGE>
__device__ __forceinline__ void pass2_tile(const ScoreArgs& a, const uint16_t* qs,
                                           const float* bias, const uint4 (&kf)[D / 16],
                                           int kbase, int half, int l32, float* out,
                                           uint32_t* lh) {
  const int key = kbase + l32;
  float s0 = 0.f, s1 = 0.f;
  // With many row tiles, re-read the per-row bias from LDS for every tile
  // rather than letting it be hoisted into registers for the whole scan.
  if constexpr (NRT > 4) asm volatile("" ::: "memory");
  f32x16_t acc[2];
  acc[0] = contract_row_tile<D, false>(qs, kf, 0, half, l32);
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    if (t + 1 < NRT) acc[(t + 1) & 1] = contract_row_tile<D, false>(qs, kf, t + 1, half, l32);
    weight_sum<EDGE>(a, acc[t & 1], bias, t, key, half, s0, s1);
    __builtin_amdgcn_sched_barrier(0);
  }
  float sum = s0 + s1;
  sum += __shfl_xor(sum, 32);
  if (half == 0 && key < a.s) {
    out[key] = sum;
    if (lh != nullptr && key >= a.sink_end && key < a.rec_begin)
      atomicAdd(&lh[(__float_as_uint(sum) >> 19) & (kHistBins - 1)], 1u);
  }
}

// Normalised weights summed per key over the group's window rows.
template <int D, int NRT>
__global__ void __launch_bounds__(512) pass2_kernel(ScoreArgs a) {
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int PITCH = D + 8;
  constexpr int NCH = D / 16;
  constexpr int ROWS_PAD = NRT * kRowTile;
  uint16_t* qs = reinterpret_cast<uint16_t*>(smem);
  float* bias = reinterpret_cast<float*>(smem + ROWS_PAD * PITCH * 2);
  uint32_t* lh = a.hist != nullptr ? reinterpret_cast<uint32_t*>(bias + ROWS_PAD) : nullptr;

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int head = work / a.n_split;
  const int split = work % a.n_split;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = lane >> 5, l32 = lane & 31;
  const int nwaves = blockDim.x >> 6;
  const int first_hidden = a.s - a.w + 1;
  const TileSeq seq = tile_seq(a, split, wave, nwaves, first_hidden);
  uint4 ka[NCH], kb[NCH];
  load_key_frag<D>(a, head, seq.kbase(0) + l32, half, ka);  // streams in during staging

  if (lh != nullptr)
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x) lh[i] = 0u;
  stage_queries<D>(a, head, ROWS_PAD, qs);
  // p = exp(l - m) / Z = 2^(dot * c - (m * log2 e + log2 Z)); padding rows get +inf (p = 0).
  for (int r = threadIdx.x; r < ROWS_PAD; r += blockDim.x) {
    float bv = INFINITY;
    if (r < a.rows) {
      const int hh = r / a.w, i = r % a.w;
      const int64_t o = (int64_t)(head * a.g + hh) * a.w + i;
      bv = fmaf(a.m_in[o], kLog2e, __log2f(a.z_in[o]));
    }
    bias[r] = bv;
  }
  __syncthreads();

  float* out = a.scores + (int64_t)head * a.s;
  int k = 0;
  for (; k + 1 < seq.clean; k += 2) {
    load_key_frag<D>(a, head, seq.kbase(k + 1) + l32, half, kb);
    pass2_tile<D, NRT, false>(a, qs, bias, ka, seq.kbase(k), half, l32, out, lh);
    load_key_frag<D>(a, head, seq.kbase(k + 2) + l32, half, ka);
    pass2_tile<D, NRT, false>(a, qs, bias, kb, seq.kbase(k + 1), half, l32, out, lh);
  }
  if (k < seq.clean) pass2_tile<D, NRT, false>(a, qs, bias, ka, seq.kbase(k), half, l32, out, lh);
  for (k = seq.clean; k < seq.n; ++k) {
    load_key_frag<D>(a, head, seq.kbase(k) + l32, half, ka);
    pass2_tile<D, NRT, true>(a, qs, bias, ka, seq.kbase(k), half, l32, out, lh);
  }
  if (lh != nullptr) {
    __syncthreads();
    uint32_t* gh = a.hist + (int64_t)head * kHistBins;
    for (int i = threadIdx.x; i < kHistBins; i += blockDim.x)
      if (lh[i]) atomicAdd(&gh[i], lh[i]);
  }
}

template <int D>
const void* pass1_fn(int nrt) {
  switch (nrt) {
    case 1: return reinterpret_cast<const void*>(&pass1_kernel<D, 1>);
    case 2: return reinterpret_cast<const void*>(&pass1_kernel<D, 2>);
    case 3: return reinterpret_cast<const void*>(&pass1_kernel<D, 3>);
    case 4: return reinterpret_cast<const void*>(&pass1_kernel<D, 4>);
    case 5: return reinterpret_cast<const void*>(&pass1_kernel<D, 5>);
    case 6: return reinterpret_cast<const void*>(&pass1_kernel<D, 6>);
    case 7: return reinterpret_cast<const void*>(&pass1_kernel<D, 7>);
    case 8: return reinterpret_cast<const void*>(&pass1_kernel<D, 8>);
    default: return nullptr;
  }
}

template <int D>
const void* pass2_fn(int nrt) {
  switch (nrt) {
    case 1: return reinterpret_cast<const void*>(&pass2_kernel<D, 1>);
    case 2: return reinterpret_cast<const void*>(&pass2_kernel<D, 2>);
    case 3: return reinterpret_cast<const void*>(&pass2_kernel<D, 3>);
    case 4: return reinterpret_cast<const void*>(&pass2_kernel<D, 4>);
    case 5: return reinterpret_cast<const void*>(&pass2_kernel<D, 5>);
    case 6: return reinterpret_cast<const void*>(&pass2_kernel<D, 6>);
    case 7: return reinterpret_cast<const void*>(&pass2_kernel<D, 7>);
    case 8: return reinterpret_cast<const void*>(&pass2_kernel<D, 8>);
    default: return nullptr;
  }
}

hipError_t launch_scan(const void* fn, const Layer& L, const ScoreArgs& a, size_t lds,
                       hipStream_t st) {
  if (fn == nullptr) return hipErrorInvalidValue;
  const hipError_t e = ensure_lds(fn, lds);
  if (e != hipSuccess) return e;
  ScoreArgs args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)(L.hkv * L.n_split));
  const dim3 blk((unsigned)(scan_waves(L) * kWave));
  return hipLaunchKernel(fn, grid, blk, kargs, lds, st);
}

}  // namespace

size_t pass1_lds_bytes(const Layer& L) {
  const size_t rows_pad = (size_t)L.row_tiles * kRowTile;
  const size_t q = rows_pad * (L.d + 8) * 2;
  const size_t red = (size_t)scan_waves(L) * rows_pad * sizeof(float2);
  return q > red ? q : red;
}

size_t pass2_lds_bytes(const Layer& L) {
  const size_t rows_pad = (size_t)L.row_tiles * kRowTile;
  return rows_pad * (L.d + 8) * 2 + rows_pad * sizeof(float) + kHistBins * sizeof(uint32_t);
}

int per_head_wgs_per_cu(const Layer& L) {
  const void* f1 = L.d == 128 ? pass1_fn<128>(L.row_tiles) : pass1_fn<64>(L.row_tiles);
  const void* f2 = L.d == 128 ? pass2_fn<128>(L.row_tiles) : pass2_fn<64>(L.row_tiles);
  if (f1 == nullptr || f2 == nullptr) return 0;
  const size_t l1 = pass1_lds_bytes(L), l2 = pass2_lds_bytes(L);
  if (ensure_lds(f1, l1) != hipSuccess || ensure_lds(f2, l2) != hipSuccess) return 0;
  const int threads = scan_waves(L) * kWave;
  int b1 = 0, b2 = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b1, f1, threads, l1) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&b2, f2, threads, l2) != hipSuccess) return 0;
  return std::min(b1, b2);
}

hipError_t launch_pass1(const Layer& L, const ScoreArgs& a, hipStream_t st) {
  const void* fn = L.d == 128 ? pass1_fn<128>(L.row_tiles) : pass1_fn<64>(L.row_tiles);
  return launch_scan(fn, L, a, pass1_lds_bytes(L), st);
}

hipError_t launch_pass2(const Layer& L, const ScoreArgs& a, hipStream_t st) {
  const void* fn = L.d == 128 ? pass2_fn<128>(L.row_tiles) : pass2_fn<64>(L.row_tiles);
  return launch_scan(fn, L, a, pass2_lds_bytes(L), st);
}

hipError_t launch_combine(const Layer& L, const ScoreArgs& a, hipStream_t st) {
  ScoreArgs args = a;
  int rows_pad = L.row_tiles * kRowTile;
  void* kargs[] = {&args, &rows_pad};
  const dim3 grid((unsigned)(L.hkv * L.row_tiles));
  return hipLaunchKernel(reinterpret_cast<const void*>(&combine_kernel), grid, dim3(256), kargs, 0, st);
}

}  // namespace kvc
