// Streaming form of the two scans (TideKV, Fig. 3 caption) for query-row
// counts G*W <= 128: used whenever its register budget allows.
//
// A workgroup of 8 wavefronts owns HG KV heads (a head pair when Hkv is even)
// and a contiguous token range. K flows through a two-stage LDS ring with
// direct global->LDS loads: a stage holds TOK tokens x HG heads, and every
// load instruction moves 1 KiB made of whole HG*256-byte token segments, so
// DRAM sees long contiguous runs even though K is token-major. Each wavefront
// keeps its head's G*W window-query rows in VGPRs (the MFMA operand layout,
// loaded once) and takes one 32-key tile of its head from every stage.
//
// LDS layout of a stage: token r occupies R16 16-byte slots; logical chunk
// (head h, chunk c) sits in slot (h*CPH + c) XOR (r mod 16), so the 32 lanes
// that read one chunk column of 32 tokens hit distinct banks.
//
// The MFMA k-slot assignment matches the per-head scans: at step st, lane
// half h feeds head-dimension chunk 2*st + h of both operands.

#include "kvc_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

// Workgroup barrier that orders LDS traffic only. __syncthreads(), and even a
// workgroup fence restricted to LDS, also drains every outstanding
// global->LDS copy, the next stage's included, and so serialises the ring;
// those copies are waited for explicitly (wait_stage) by the wavefront that
// issued them. The memory clobber keeps the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS reads inside the ring loop are issued as inline assembly. For a plain
// LDS load the compiler cannot tell which ring stage it touches, so it waits
// for every outstanding global->LDS copy, the stage still being filled
// included; these reads rely on the stage's explicit wait and the barrier
// instead, and lds_settle() orders their results before any use.
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ u32x4_t lds_read_b128(const void* p) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

// Wait for this wavefront's LDS reads; every value passed through here is
// read only after the wait.
template <int N>
__device__ __forceinline__ void lds_settle(u32x4_t (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Wait for every outstanding global load of this wavefront and re-define the
// given registers after the wait. Without this the compiler cannot prove, in
// the ring loop, that the query registers loaded before it have arrived (the
// global->LDS copies issued since share their counter) and waits for all
// loads, the next stage's included, before the first MFMA of every stage.
template <int N, int M>
__device__ __forceinline__ void vm_settle(uint4 (&q)[N][M]) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < M; ++j) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, q[i][j]);
      asm volatile("" : "+v"(v));
      q[i][j] = __builtin_bit_cast(uint4, v);
    }
}

__device__ __forceinline__ void vm_settle(float& x) { asm volatile("" : "+v"(x)); }

// LDS atomic add without return, as inline assembly for the same reason as
// the reads above (a plain LDS atomic would first drain the ring's copies).
__device__ __forceinline__ void lds_add_u32(uint32_t* p, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

__device__ __forceinline__ int xcd_remap(int bid, int nb) {
  if ((nb & 7) != 0) return bid;
  return (bid & 7) * (nb >> 3) + (bid >> 3);
}

__device__ __forceinline__ void lse_merge(float& m, float& z, float m2, float z2, float c) {
  const float mn = fmaxf(m, m2);
  if (mn == -INFINITY) return;
  z = z * exp2_raw((m - mn) * c) + z2 * exp2_raw((m2 - mn) * c);
  m = mn;
}

template <int D, int HG>
struct Cfg {
  static constexpr int WPH = 8 / HG;              // wavefronts per head
  static constexpr int TOK = kKeyTile * WPH;      // tokens per stage
  static constexpr int CPH = D / 8;               // 16-byte chunks per head row
  static constexpr int R16 = HG * CPH;            // 16-byte slots per token in a stage
  static constexpr int XS = R16 < 16 ? R16 : 16;  // swizzle span
  static constexpr int STAGE = TOK * R16 * 16;    // bytes per stage
  static constexpr int NI = STAGE / (1024 * 8);   // load instructions per wave per stage
  static constexpr int NCH = D / 16;              // MFMA k-steps
};

template <int D, int HG>
__device__ __forceinline__ int slot_of(int r, int h, int c) {
  using C = Cfg<D, HG>;
  return r * C::R16 + ((h * C::CPH + c) ^ (r & (C::XS - 1)));
}

// This wavefront's share of one stage's loads (tokens from tok0; tokens past
// the prompt are clamped to its last key and masked by the consumer).
template <int D, int HG>
__device__ __forceinline__ void stage_issue(const ScoreArgs& a, int h0, int tok0, int wave, int lane,
                                            unsigned char* dst) {
  using C = Cfg<D, HG>;
#pragma unroll
  for (int j = 0; j < C::NI; ++j) {
    const int p = (wave * C::NI + j) * 64 + lane;  // slot this lane fills
    const int r = p / C::R16, q = p % C::R16;
    const int lc = q ^ (r & (C::XS - 1));
    const int h = lc / C::CPH, c = lc % C::CPH;
    int tok = tok0 + r;
    tok = tok < a.s ? tok : a.s - 1;
    const uint16_t* src = a.k + (int64_t)tok * a.k_tok + (int64_t)(h0 + h) * a.k_head + c * 8;
    __builtin_amdgcn_global_load_lds(src, (lds_void*)(dst + (wave * C::NI + j) * 1024), 16, 0, 0);
  }
}

// Wait until this wavefront's loads of the stage being consumed have landed:
// at most `ahead` later stages' loads may still be in flight.
template <int NI>
__device__ __forceinline__ void wait_stage(bool next_in_flight) {
  // s_waitcnt immediate: vmcnt in bits 3:0 and 15:14, expcnt 6:4, lgkmcnt 11:8
  if (next_in_flight) __builtin_amdgcn_s_waitcnt(0x0F70 | (NI & 15) | ((NI >> 4) << 14));
  else __builtin_amdgcn_s_waitcnt(0x0F70);
}

// The wavefront's head rows of Q_win in MFMA operand layout: row tile t, step st.
template <int D, int NRT>
__device__ __forceinline__ void load_query_regs(const ScoreArgs& a, int head, int half, int l32,
                                                uint4 (&qr)[NRT][D / 16]) {
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const int r = t * kRowTile + l32;
    const bool ok = r < a.rows;
    const int hh = ok ? r / a.w : 0, i = ok ? r % a.w : 0;
    const uint16_t* src = a.q + (int64_t)i * a.q_tok + (int64_t)(head * a.g + hh) * a.q_head;
#pragma unroll
    for (int st = 0; st < D / 16; ++st)
      qr[t][st] = ok ? *reinterpret_cast<const uint4*>(src + (2 * st + half) * 8) : make_uint4(0u, 0u, 0u, 0u);
  }
}

template <int D, int HG>
__device__ __forceinline__ void load_key_regs(const unsigned char* stage, int hl, int kt, int half,
                                              int l32, uint4 (&kf)[D / 16]) {
  const int r = kt * kKeyTile + l32;
  u32x4_t raw[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st) raw[st] = lds_read_b128(stage + slot_of<D, HG>(r, hl, 2 * st + half) * 16);
  lds_settle(raw);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) kf[st] = make_uint4(raw[st][0], raw[st][1], raw[st][2], raw[st][3]);
}

template <int D, int NRT, bool KROWS>
__device__ __forceinline__ f32x16_t contract(const uint4 (&qr)[NRT][D / 16], const uint4 (&kf)[D / 16],
                                             int t) {
  f32x16_t acc = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    acc = KROWS ? mfma32x32x16(kf[st], qr[t][st], acc) : mfma32x32x16(qr[t][st], kf[st], acc);
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

struct Range {
  int t0, nst;  // first token, stages
};

__device__ __forceinline__ Range wg_range(const ScoreArgs& a, int split, int tok_per_stage) {
  Range r;
  r.t0 = split * a.blocks_per_wg * tok_per_stage;
  int t1 = r.t0 + a.blocks_per_wg * tok_per_stage;
  t1 = t1 < a.s ? t1 : a.s;
  r.nst = (t1 - r.t0 + tok_per_stage - 1) / tok_per_stage;
  return r;
}

// ---------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------
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
  if (EDGE && mnew == -INFINITY) return;
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
__device__ __forceinline__ void pass1_tile(const ScoreArgs& a, const uint4 (&qr)[NRT][D / 16],
                                           const uint4 (&kf)[D / 16], int kbase, int half,
                                           const int (&qpos)[NRT], float (&mrun)[NRT],
                                           float (&zrun)[NRT]) {
  if constexpr (NRT <= 2) {
    // software-pipelined: the MFMAs of row tile t+1 overlap the VALU of t
    f32x16_t acc[2];
    acc[0] = contract<D, NRT, true>(qr, kf, 0);
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      if (t + 1 < NRT) acc[(t + 1) & 1] = contract<D, NRT, true>(qr, kf, t + 1);
      lse_update<EDGE>(a, acc[t & 1], kbase, half, qpos[t], mrun[t], zrun[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // register budget: one accumulator; the second wavefront on the SIMD
    // overlaps its MFMAs with this one's VALU
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      lse_update<EDGE>(a, contract<D, NRT, true>(qr, kf, t), kbase, half, qpos[t], mrun[t], zrun[t]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

template <int D, int NRT, int HG>
__global__ void __launch_bounds__(512) pass1_stream_kernel(ScoreArgs a) {
  using C = Cfg<D, HG>;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int ROWS_PAD = NRT * kRowTile;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = work / a.n_split, split = work % a.n_split;
  const int h0 = grp * HG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront-uniform: SGPRs
  const int half = lane >> 5, l32 = lane & 31;
  const int hl = wave / C::WPH, kt = wave % C::WPH;
  const int head = h0 + hl;
  const int first_hidden = a.s - a.w + 1;
  const Range rg = wg_range(a, split, C::TOK);

  if (a.hist != nullptr && split == 0)
    for (int i = threadIdx.x; i < HG * kHistBins; i += blockDim.x) a.hist[(int64_t)h0 * kHistBins + i] = 0u;

  stage_issue<D, HG>(a, h0, rg.t0, wave, lane, smem);
  uint4 qr[NRT][D / 16];
  load_query_regs<D, NRT>(a, head, half, l32, qr);
  vm_settle(qr);
  if (rg.nst > 1) stage_issue<D, HG>(a, h0, rg.t0 + C::TOK, wave, lane, smem + C::STAGE);

  float mrun[NRT], zrun[NRT];
  int qpos[NRT];
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    mrun[t] = -INFINITY;
    zrun[t] = 0.f;
    const int r = t * kRowTile + l32;
    qpos[t] = r < a.rows ? a.s - a.w + (r % a.w) : -1;
  }

  for (int st = 0; st < rg.nst; ++st) {
    wait_stage<C::NI>(st + 1 < rg.nst);
    lds_barrier();
    const unsigned char* stage = smem + (st & 1) * C::STAGE;
    const int kbase = rg.t0 + st * C::TOK + kt * kKeyTile;
    if (kbase < a.s) {
      uint4 kf[D / 16];
      load_key_regs<D, HG>(stage, hl, kt, half, l32, kf);
      if (kbase + kKeyTile <= first_hidden)
        pass1_tile<D, NRT, false>(a, qr, kf, kbase, half, qpos, mrun, zrun);
      else
        pass1_tile<D, NRT, true>(a, qr, kf, kbase, half, qpos, mrun, zrun);
    }
    lds_barrier();
    if (st + 2 < rg.nst) stage_issue<D, HG>(a, h0, rg.t0 + (st + 2) * C::TOK, wave, lane, smem + (st & 1) * C::STAGE);
  }

  // lanes l and l+32 share a query row; then the WPH wavefronts of a head
#pragma unroll
  for (int t = 0; t < NRT; ++t) {
    const float mo = __shfl_xor(mrun[t], 32);
    const float zo = __shfl_xor(zrun[t], 32);
    lse_merge(mrun[t], zrun[t], mo, zo, a.c);
  }
  float2* red = reinterpret_cast<float2*>(smem);  // the ring is idle now
  if (half == 0) {
#pragma unroll
    for (int t = 0; t < NRT; ++t) red[wave * ROWS_PAD + t * kRowTile + l32] = make_float2(mrun[t], zrun[t]);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * a.rows; idx += blockDim.x) {
    const int h = idx / a.rows, r = idx % a.rows;
    float m = -INFINITY, z = 0.f;
    for (int k = 0; k < C::WPH; ++k) {
      const float2 p = red[(h * C::WPH + k) * ROWS_PAD + r];
      lse_merge(m, z, p.x, p.y, a.c);
    }
    reinterpret_cast<float2*>(a.part)[((int64_t)(h0 + h) * a.n_split + split) * ROWS_PAD + r] = make_float2(m, z);
  }
}

// ---------------------------------------------------------------------------
// Pass 2
// ---------------------------------------------------------------------------
// qpos: per row, the prompt position of its query (-1 for padding rows),
// read from LDS inside the loop so that nothing per row lives in registers.
template <bool EDGE>
__device__ __forceinline__ void weight_sum(const ScoreArgs& a, const f32x16_t& acc, const float* bias,
                                           const int* qpos, int t, int key, int half, float& s0,
                                           float& s1) {
  const int o = t * kRowTile + 4 * half;
  u32x4_t bq[4];
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) bq[q4] = lds_read_b128(bias + o + 8 * q4);
  lds_settle(bq);
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    u32x4_t qv = {0u, 0u, 0u, 0u};
    if constexpr (EDGE) {
      u32x4_t q1[1] = {lds_read_b128(qpos + o + 8 * q4)};
      lds_settle(q1);
      qv = q1[0];
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float p = exp2_raw(fmaf(acc[4 * q4 + e4], a.c, -__uint_as_float(bq[q4][e4])));
      if constexpr (EDGE) {
        if (key >= a.s || key > (int)qv[e4]) p = 0.f;
      }
      if (e4 & 1) s1 += p; else s0 += p;
    }
  }
}

template <int D, int NRT, bool EDGE>
__device__ __forceinline__ float pass2_tile(const ScoreArgs& a, const uint4 (&qr)[NRT][D / 16],
                                            const uint4 (&kf)[D / 16], const float* bias,
                                            const int* qpos, int key, int half) {
  float s0 = 0.f, s1 = 0.f;
  if constexpr (NRT <= 2) {
    f32x16_t acc[2];
    acc[0] = contract<D, NRT, false>(qr, kf, 0);
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      if (t + 1 < NRT) acc[(t + 1) & 1] = contract<D, NRT, false>(qr, kf, t + 1);
      weight_sum<EDGE>(a, acc[t & 1], bias, qpos, t, key, half, s0, s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int t = 0; t < NRT; ++t) {
      weight_sum<EDGE>(a, contract<D, NRT, false>(qr, kf, t), bias, qpos, t, key, half, s0, s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float s = s0 + s1;
  return s + __shfl_xor(s, 32);
}

template <int D, int NRT, int HG>
__global__ void __launch_bounds__(512) pass2_stream_kernel(ScoreArgs a) {
  using C = Cfg<D, HG>;
  extern __shared__ __align__(16) unsigned char smem[];
  constexpr int ROWS_PAD = NRT * kRowTile;
  float* bias_all = reinterpret_cast<float*>(smem + 2 * C::STAGE);          // [HG][ROWS_PAD]
  int* qpos_all = reinterpret_cast<int*>(bias_all + HG * ROWS_PAD);         // [HG][ROWS_PAD]
  uint32_t* hist2 = reinterpret_cast<uint32_t*>(qpos_all + HG * ROWS_PAD);  // [HG][kHistBins/2], u16 pairs

  const int work = xcd_remap(blockIdx.x, gridDim.x);
  const int grp = work / a.n_split, split = work % a.n_split;
  const int h0 = grp * HG;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront-uniform: SGPRs
  const int half = lane >> 5, l32 = lane & 31;
  const int hl = wave / C::WPH, kt = wave % C::WPH;
  const int head = h0 + hl;
  const int first_hidden = a.s - a.w + 1;
  const Range rg = wg_range(a, split, C::TOK);

  stage_issue<D, HG>(a, h0, rg.t0, wave, lane, smem);
  uint4 qr[NRT][D / 16];
  load_query_regs<D, NRT>(a, head, half, l32, qr);
  // this thread's normaliser (one bias entry per thread)
  static_assert(HG * ROWS_PAD <= 512, "one bias entry per thread");
  const int bidx = threadIdx.x;
  float mv = 0.f, zv = 1.f;
  bool real_row = false;
  if (bidx < HG * ROWS_PAD) {
    const int h = bidx / ROWS_PAD, r = bidx % ROWS_PAD;
    if (r < a.rows) {
      const int64_t o = (int64_t)((h0 + h) * a.g + r / a.w) * a.w + r % a.w;
      mv = a.m_in[o];
      zv = a.z_in[o];
      real_row = true;
    }
  }
  vm_settle(qr);
  vm_settle(mv);
  vm_settle(zv);

  // p = 2^(dot * c - (m * log2 e + log2 Z)); padding rows get +inf (p = 0)
  if (bidx < HG * ROWS_PAD) {
    bias_all[bidx] = real_row ? mv * kLog2e + __log2f(zv) : INFINITY;
    qpos_all[bidx] = real_row ? a.s - a.w + (bidx % ROWS_PAD) % a.w : -1;
  }
  const bool with_hist = a.hist != nullptr;
  if (with_hist)
    for (int i = threadIdx.x; i < HG * kHistBins / 2; i += blockDim.x) hist2[i] = 0u;
  if (rg.nst > 1) stage_issue<D, HG>(a, h0, rg.t0 + C::TOK, wave, lane, smem + C::STAGE);
  const float* bias = bias_all + hl * ROWS_PAD;
  const int* qpos = qpos_all + hl * ROWS_PAD;
  uint32_t* lh = hist2 + hl * (kHistBins / 2);
  float* out = a.scores + (int64_t)head * a.s;

  for (int st = 0; st < rg.nst; ++st) {
    wait_stage<C::NI>(st + 1 < rg.nst);
    lds_barrier();
    const unsigned char* stage = smem + (st & 1) * C::STAGE;
    const int kbase = rg.t0 + st * C::TOK + kt * kKeyTile;
    if (kbase < a.s) {
      uint4 kf[D / 16];
      load_key_regs<D, HG>(stage, hl, kt, half, l32, kf);
      const int key = kbase + l32;
      const float sum = kbase + kKeyTile <= first_hidden
                            ? pass2_tile<D, NRT, false>(a, qr, kf, bias, qpos, key, half)
                            : pass2_tile<D, NRT, true>(a, qr, kf, bias, qpos, key, half);
      if (half == 0 && key < a.s) {
        out[key] = sum;
        if (with_hist && key >= a.sink_end && key < a.rec_begin) {
          const uint32_t b = (__float_as_uint(sum) >> 19) & (kHistBins - 1);
          lds_add_u32(&lh[b >> 1], 1u << ((b & 1) * 16));
        }
      }
    }
    lds_barrier();
    if (st + 2 < rg.nst) stage_issue<D, HG>(a, h0, rg.t0 + (st + 2) * C::TOK, wave, lane, smem + (st & 1) * C::STAGE);
  }
  if (with_hist) {
    __syncthreads();
    for (int i = threadIdx.x; i < HG * kHistBins / 2; i += blockDim.x) {
      const uint32_t v = hist2[i];
      if (v == 0u) continue;
      const int h = i / (kHistBins / 2), b = 2 * (i % (kHistBins / 2));
      uint32_t* gh = a.hist + (int64_t)(h0 + h) * kHistBins;
      if (v & 0xFFFFu) atomicAdd(&gh[b], v & 0xFFFFu);
      if (v >> 16) atomicAdd(&gh[b + 1], v >> 16);
    }
  }
}

template <int D, int HG>
const void* pass1_stream_fn(int nrt) {
  switch (nrt) {
    case 1: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 1, HG>);
    case 2: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 2, HG>);
    case 3: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 3, HG>);
    case 4: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 4, HG>);
    default: return nullptr;
  }
}

template <int D, int HG>
const void* pass2_stream_fn(int nrt) {
  switch (nrt) {
    case 1: return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 1, HG>);
    case 2: return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 2, HG>);
    case 3: return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 3, HG>);
    case 4: return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 4, HG>);
    default: return nullptr;
  }
}

const void* stream_fn(bool pass1, const Layer& L) {
  if (L.d == 128) {
    if (L.stream_hg == 2) return pass1 ? pass1_stream_fn<128, 2>(L.row_tiles) : pass2_stream_fn<128, 2>(L.row_tiles);
    return pass1 ? pass1_stream_fn<128, 1>(L.row_tiles) : pass2_stream_fn<128, 1>(L.row_tiles);
  }
  if (L.stream_hg == 2) return pass1 ? pass1_stream_fn<64, 2>(L.row_tiles) : pass2_stream_fn<64, 2>(L.row_tiles);
  return pass1 ? pass1_stream_fn<64, 1>(L.row_tiles) : pass2_stream_fn<64, 1>(L.row_tiles);
}

size_t stage_bytes(const Layer& L) {
  const int tok = kKeyTile * 8 / L.stream_hg;
  return (size_t)tok * L.stream_hg * (L.d / 8) * 16;
}

}  // namespace

int stream_tokens(int hg) { return kKeyTile * 8 / hg; }

size_t pass1_stream_lds_bytes(const Layer& L) {
  const size_t ring = 2 * stage_bytes(L);
  const size_t red = (size_t)8 * L.row_tiles * kRowTile * sizeof(float2);
  return ring > red ? ring : red;
}

size_t pass2_stream_lds_bytes(const Layer& L) {
  const size_t rows_pad = (size_t)L.row_tiles * kRowTile;
  return 2 * stage_bytes(L) + L.stream_hg * rows_pad * (sizeof(float) + sizeof(int)) +
         (size_t)L.stream_hg * (kHistBins / 2) * sizeof(uint32_t);
}

hipError_t launch_stream(bool pass1, const Layer& L, const ScoreArgs& a, hipStream_t st) {
  const void* fn = stream_fn(pass1, L);
  if (fn == nullptr) return hipErrorInvalidValue;
  const size_t lds = pass1 ? pass1_stream_lds_bytes(L) : pass2_stream_lds_bytes(L);
  const hipError_t e = ensure_lds(fn, lds);
  if (e != hipSuccess) return e;
  ScoreArgs args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)(L.hkv / L.stream_hg * L.n_split));
  return hipLaunchKernel(fn, grid, dim3(8 * kWave), kargs, lds, st);
}

}  // namespace kvc
