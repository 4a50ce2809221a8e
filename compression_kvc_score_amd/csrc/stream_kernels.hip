// Streaming form of the two scans (TideKV, Fig. 3 caption) for query-row
// counts G*W <= 128, and up to 192 at D = 128 (three row tiles per
// wavefront): used whenever its register budget allows.
//
// A workgroup of 8 wavefronts owns HG KV heads (a head pair, or one head as
// the host chooses) and a contiguous token range. K flows through a ring of kRingSlots LDS
// slots filled by direct global->LDS loads: a slot holds TOKS tokens x HG
// heads (32 KiB), and every load instruction moves 1 KiB made of whole
// HG*D*2-byte token segments, so DRAM sees long contiguous runs even though K
// is token-major. Up to kRingSlots-1 slots are in flight while one is
// consumed; one LDS-only barrier per slot recycles the slot consumed before.
//
// The wavefronts of a head split a slot's key tiles and, when a slot holds
// fewer tiles than that, the head's query-row tiles as well (RS row groups):
// a wavefront keeps only its own row tiles of Q_win in VGPRs (MFMA operand
// layout, loaded once) and contracts them with its 32-key tile of every slot.
//
// LDS layout of a slot: token r occupies R16 16-byte chunks; logical chunk
// (head h, chunk c) sits in chunk (h*CPH + c) XOR (r mod XS), so the 32 lanes
// that read one chunk column of 32 tokens hit distinct banks.
//
// The MFMA k-slot assignment matches the per-head scans: at step st, lane
// half h feeds head-dimension chunk 2*st + h of both operands.

#include <algorithm>
#include <type_traits>

#include "kvc_internal.h"
#include "scan_select.h"

// 0 selects the job-at-a-time loops everywhere (for comparisons).
#ifndef KVC_SLOT_PIPE
#define KVC_SLOT_PIPE 1
#endif

namespace kvc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kSlotBytes = 32768;      // one ring slot
constexpr int kRingSlots = 4;          // slots in the ring
constexpr int kRingBytes = kSlotBytes * kRingSlots;

__device__ __forceinline__ f32x16_t mfma32x32x16(uint4 a, uint4 b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ float exp2_raw(float x) { return __builtin_amdgcn_exp2f(x); }

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

// Workgroup barrier that orders LDS traffic only. __syncthreads(), and even a
// workgroup fence restricted to LDS, also drains every outstanding
// global->LDS copy, the later slots' included, and so serialises the ring;
// those copies are waited for explicitly (wait_slots) by the wavefront that
// issued them. The memory clobber keeps the compiler from moving memory
// operations across the barrier.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// LDS accesses inside the ring loop are issued as inline assembly. For a
// plain LDS access the compiler cannot tell which ring slot it touches, so it
// waits for every outstanding global->LDS copy first; these rely on the
// slot's explicit wait and the barrier instead, and lds_settle() orders their
// results before any use.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return (uint32_t)(size_t)(const __attribute__((address_space(3))) char*)p;
}

__device__ __forceinline__ u32x4_t lds_read_b128(const void* p) {
  u32x4_t v;
  asm volatile("ds_read_b128 %0, %1" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

__device__ __forceinline__ float lds_read_f32(const void* p) {
  float v;
  asm volatile("ds_read_b32 %0, %1" : "=v"(v) : "v"(lds_addr(p)) : "memory");
  return v;
}

__device__ __forceinline__ void lds_write_f32(void* p, float v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

__device__ __forceinline__ void lds_add_u32(uint32_t* p, uint32_t v) {
  asm volatile("ds_add_u32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}

// Wait for this wavefront's LDS reads; every value passed through here is
// read only after the wait.
template <typename T, int N>
__device__ __forceinline__ void lds_settle(T (&v)[N]) {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
  for (int i = 0; i < N; ++i) asm volatile("" : "+v"(v[i]));
}

// Wait for every outstanding global load of this wavefront and re-define the
// given registers after the wait. Without this the compiler cannot prove, in
// the ring loop, that registers loaded before it have arrived (the
// global->LDS copies issued since share their counter) and waits for all
// copies before their first use in every iteration.
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

template <int NI, int K>
__device__ __forceinline__ void wait_slots(int later);

// As vm_settle, but the `later` slots of ring copies issued after the
// registers' loads may stay in flight.
template <int NI, int N, int M>
__device__ __forceinline__ void vm_settle_after(uint4 (&q)[N][M], int later) {
  wait_slots<NI, kRingSlots - 1>(later);
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < M; ++j) {
      u32x4_t v = __builtin_bit_cast(u32x4_t, q[i][j]);
      asm volatile("" : "+v"(v));
      q[i][j] = __builtin_bit_cast(uint4, v);
    }
}

// s_waitcnt with vmcnt = N (bits 3:0 and 15:14), expcnt and lgkmcnt not waited on.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt(0x0F70 | (N & 15) | ((N >> 4) << 14));
}

// Wait until at most `later` slots' copies (NI instructions each) are still
// in flight for this wavefront; `later` is wavefront-uniform.
template <int NI, int K>
__device__ __forceinline__ void wait_slots(int later) {
  if constexpr (K == 0) {
    wait_vmcnt<0>();
  } else {
    if (later >= K) wait_vmcnt<K * NI>();
    else wait_slots<NI, K - 1>(later);
  }
}

template <int D, int HG>
struct Ring {
  static constexpr int WAVES = 8;                       // wavefronts per workgroup
  static constexpr int CPH = D / 8;                     // 16-byte chunks per head row
  static constexpr int R16 = HG * CPH;                  // chunks per token in a slot
  static constexpr int XS = R16 < 16 ? R16 : 16;        // swizzle span
  static constexpr int TOKS = kSlotBytes / (R16 * 16);  // tokens per slot
  static constexpr int KT = TOKS / kKeyTile;            // key tiles per head per slot
  static constexpr int WPH = WAVES / HG;                // wavefronts per head
  static constexpr int RS = WPH / KT;                   // row groups sharing a key tile
  static constexpr int NI = kSlotBytes / (WAVES * 1024);   // copies per wavefront per slot
  static_assert(KT >= 1 && WPH % KT == 0 && RS >= 1, "slot geometry");
  static_assert(kSlotBytes % (WAVES * 1024) == 0, "whole copy instructions per wavefront");
  static_assert(64 % R16 == 0, "a copy instruction covers whole tokens");
};

// Wavefront roles: head within the group, key tile within a slot, and row
// group (row tiles rg, rg + RS, ...).
struct Role {
  int hl, kt, rg;
};

template <int D, int HG>
__device__ __forceinline__ Role role_of(int wave) {
  using R = Ring<D, HG>;
  const int sub = wave % R::WPH;
  return Role{wave / R::WPH, sub % R::KT, sub / R::KT};
}

// Per-lane byte offsets of this wavefront's copies within a full slot,
// relative to (first token of the slot, first head of the group); the host
// only picks this path when they fit in 32 bits.
template <int D, int HG>
__device__ __forceinline__ void copy_offsets(const ScoreArgs& a, int wave, int lane,
                                             uint32_t (&off)[Ring<D, HG>::NI]) {
  using R = Ring<D, HG>;
#pragma unroll
  for (int j = 0; j < R::NI; ++j) {
    const int p = (wave * R::NI + j) * 64 + lane;
    const int r = p / R::R16, q = p % R::R16;
    const int lc = q ^ (r & (R::XS - 1));
    const int h = lc / R::CPH, c = lc % R::CPH;
    // the host takes this path only when a slot's span fits in 32 bits
    off[j] = ((uint32_t)r * (uint32_t)a.k_tok + (uint32_t)h * (uint32_t)a.k_head + (uint32_t)(c * 8)) * 2u;
  }
}

// Copies of the slot that starts at token tok0 into the LDS buffer dst.
// Tokens past the prompt are clamped to its last key and masked by the
// consumer.
template <int D, int HG>
__device__ __forceinline__ void slot_issue(const ScoreArgs& a, int h0, int tok0, int wave, int lane,
                                           const uint32_t* off, unsigned char* dst) {
  using R = Ring<D, HG>;
  const char* base = reinterpret_cast<const char*>(a.k + (int64_t)tok0 * a.k_tok + (int64_t)h0 * a.k_head);
  if (tok0 + R::TOKS <= a.s) {
#pragma unroll
    for (int j = 0; j < R::NI; ++j)
      __builtin_amdgcn_global_load_lds(base + off[j], (lds_void*)(dst + (wave * R::NI + j) * 1024), 16, 0, 0);
  } else {
    // the same copies with the token of every lane past the prompt moved back
    // to the last key (a copy instruction covers 64 / R16 whole tokens)
    const int rl = lane / R::R16;
#pragma unroll
    for (int j = 0; j < R::NI; ++j) {
      const int tok = tok0 + (wave * R::NI + j) * (64 / R::R16) + rl;
      const int64_t back = tok < a.s ? 0 : (int64_t)(a.s - 1 - tok) * a.k_tok * 2;
      __builtin_amdgcn_global_load_lds(base + off[j] + back, (lds_void*)(dst + (wave * R::NI + j) * 1024), 16, 0, 0);
    }
  }
}

// The wavefront's row tiles (rg, rg + RS, ...) of its head's Q_win rows in
// MFMA operand layout; rows past G*W (and tiles past nrt) are zero.
template <int D, int NRTW, int RS>
__device__ __forceinline__ void load_query_regs(const ScoreArgs& a, int head, int rg, int nrt, int half,
                                                int l32, uint4 (&qr)[NRTW][D / 16]) {
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    const int t = rg + RS * i;
    const int r = t * kRowTile + l32;
    const bool full = t < nrt && (t + 1) * kRowTile <= a.rows;  // wavefront-uniform
    const bool ok = t < nrt && r < a.rows;
    const int hh = ok ? r / a.w : 0, wi = ok ? r % a.w : 0;
    const uint16_t* src = a.q + (int64_t)wi * a.q_tok + (int64_t)(head * a.g + hh) * a.q_head;
    if (full) {
#pragma unroll
      for (int st = 0; st < D / 16; ++st) qr[i][st] = *reinterpret_cast<const uint4*>(src + (2 * st + half) * 8);
    } else {
#pragma unroll
      for (int st = 0; st < D / 16; ++st)
        qr[i][st] = ok ? *reinterpret_cast<const uint4*>(src + (2 * st + half) * 8) : make_uint4(0u, 0u, 0u, 0u);
    }
  }
}

// This lane's MFMA operand chunks of key tile kt of head hl in a slot. The
// reads are only issued here; key_settle() waits for them.
template <int D, int HG>
__device__ __forceinline__ void key_issue(const unsigned char* slot, int hl, int kt, int half, int l32,
                                          u32x4_t (&raw)[D / 16]) {
  using R = Ring<D, HG>;
  const int r = kt * kKeyTile + l32;
#pragma unroll
  for (int st = 0; st < D / 16; ++st) {
    const int chunk = r * R::R16 + ((hl * R::CPH + 2 * st + half) ^ (r & (R::XS - 1)));
    raw[st] = lds_read_b128(slot + chunk * 16);
  }
}

// This lane's MFMA operand chunks of key tile kt of head hl in a slot, read
// and waited for in one statement: the registers are defined only after the
// wait, so a copy the compiler makes of them can never read a register that an
// LDS read has not yet written.
template <int D, int HG>
__device__ __forceinline__ void key_read(const unsigned char* slot, int hl, int kt, int half, int l32,
                                         u32x4_t (&kf)[D / 16]) {
  using R = Ring<D, HG>;
  const int r = kt * kKeyTile + l32;
  uint32_t ad[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    ad[st] = lds_addr(slot + (r * R::R16 + ((hl * R::CPH + 2 * st + half) ^ (r & (R::XS - 1)))) * 16);
  if constexpr (D == 128) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %9\n\tds_read_b128 %2, %10\n\tds_read_b128 %3, %11\n\t"
        "ds_read_b128 %4, %12\n\tds_read_b128 %5, %13\n\tds_read_b128 %6, %14\n\tds_read_b128 %7, %15\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]), "=&v"(kf[6]),
          "=&v"(kf[7])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7])
        : "memory");
  } else {
    static_assert(D == 64, "head dimension");
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b128 %2, %6\n\tds_read_b128 %3, %7\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3])
        : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3])
        : "memory");
  }
}

// As key_read, and one float read from `extra` in the same round trip (its
// value, like the fragments, is defined only after the wait).
template <int D, int HG>
__device__ __forceinline__ void key_read_x(const unsigned char* slot, int hl, int kt, int half, int l32,
                                           u32x4_t (&kf)[D / 16], const float* extra, float& xv) {
  using R = Ring<D, HG>;
  static_assert(D == 128, "the two-row-group pass 2 runs with D = 128");
  const int r = kt * kKeyTile + l32;
  uint32_t ad[D / 16];
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    ad[st] = lds_addr(slot + (r * R::R16 + ((hl * R::CPH + 2 * st + half) ^ (r & (R::XS - 1)))) * 16);
  asm volatile(
      "ds_read_b32 %8, %17\n\t"
      "ds_read_b128 %0, %9\n\tds_read_b128 %1, %10\n\tds_read_b128 %2, %11\n\tds_read_b128 %3, %12\n\t"
      "ds_read_b128 %4, %13\n\tds_read_b128 %5, %14\n\tds_read_b128 %6, %15\n\tds_read_b128 %7, %16\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(kf[0]), "=&v"(kf[1]), "=&v"(kf[2]), "=&v"(kf[3]), "=&v"(kf[4]), "=&v"(kf[5]), "=&v"(kf[6]),
        "=&v"(kf[7]), "=&v"(xv)
      : "v"(ad[0]), "v"(ad[1]), "v"(ad[2]), "v"(ad[3]), "v"(ad[4]), "v"(ad[5]), "v"(ad[6]), "v"(ad[7]),
        "v"(lds_addr(extra))
      : "memory");
}

template <int D>
__device__ __forceinline__ void key_settle(u32x4_t (&raw)[D / 16], uint4 (&kf)[D / 16]) {
  lds_settle(raw);
#pragma unroll
  for (int st = 0; st < D / 16; ++st) kf[st] = __builtin_bit_cast(uint4, raw[st]);
}

template <int D, int HG>
__device__ __forceinline__ void load_key_regs(const unsigned char* slot, int hl, int kt, int half, int l32,
                                              uint4 (&kf)[D / 16]) {
  u32x4_t raw[D / 16];
  key_issue<D, HG>(slot, hl, kt, half, l32, raw);
  key_settle<D>(raw, kf);
}

template <int D, int NRTW, bool KROWS>
__device__ __forceinline__ f32x16_t contract(const uint4 (&qr)[NRTW][D / 16], const uint4 (&kf)[D / 16], int i) {
  f32x16_t acc = {};
#pragma unroll
  for (int st = 0; st < D / 16; ++st)
    acc = KROWS ? mfma32x32x16(kf[st], qr[i][st], acc) : mfma32x32x16(qr[i][st], kf[st], acc);
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

// x + (x of lane l ^ 32): one swap of the wavefront halves in the VALU (a
// __shfl_xor is an LDS permute round trip).
__device__ __forceinline__ float add_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// Slot-level software pipeline, for wavefronts that own at most two row
// tiles: iteration n works through the exponentials of slot n's dot products
// (already in registers) while the MFMAs of slot n+1 run beside them, the row
// tiles' MFMA chains alternating so that no MFMA waits for the one before it
// in its chain. The key fragments of slot n+1 are read from LDS at the top of
// iteration n and waited for only after the first VALU work of slot n. Per
// row and per key the arithmetic runs in the same order as one job at a time,
// so the results are bitwise those of the job-at-a-time form.
// ---------------------------------------------------------------------------

// MFMA m of a slot (m = step * NRTW + tile) into the next accumulators.
template <int D, int NRTW, bool KROWS, int M>
__device__ __forceinline__ void slot_mfma(f32x16_t (&nxt)[NRTW], const uint4 (&qr)[NRTW][D / 16],
                                          const u32x4_t (&kf)[D / 16]) {
  constexpr int CH = M % NRTW, ST = M / NRTW;
  const f32x16_t c = ST == 0 ? f32x16_t{} : nxt[CH];
  const uint4 k = __builtin_bit_cast(uint4, kf[ST]);
  nxt[CH] = KROWS ? mfma32x32x16(k, qr[CH][ST], c) : mfma32x32x16(qr[CH][ST], k, c);
}

// Scheduling pattern of a slot's arithmetic: NMF groups of one MFMA followed
// by the VALU and transcendental instructions of its logits, so that the
// matrix pipe and the VALU of one wavefront run side by side. (Without it the
// scheduler issued half of the MFMAs back to back and left a row tile's
// exponentials for after the last one.)
template <int NMF, int NVALU, int NTRANS>
__device__ __forceinline__ void slot_schedule() {
#pragma unroll
  for (int m = 0; m < NMF; ++m) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);       // MFMA
    __builtin_amdgcn_sched_group_barrier(0x400, NTRANS, 0);  // v_exp
    __builtin_amdgcn_sched_group_barrier(0x002, NVALU, 0);   // other VALU
  }
}

template <int... I>
struct Seq {};
template <int N, int... I>
struct MakeSeq : MakeSeq<N - 1, N - 1, I...> {};
template <int... I>
struct MakeSeq<0, I...> {
  using type = Seq<I...>;
};

// One group of a slot's arithmetic, in this order: the MFMA of the next
// slot's contraction (FIRST: its chain starts from zero) and, for two logits
// x0, x1 of the current slot, p = 2^(x * c - b) added to s0 and s1. Inline
// assembly fixes the interleaving (the compiler's scheduler issued the MFMAs
// back to back and the exponentials after them). Every exponential has one
// instruction between it and the add that reads it; the hazards with the
// MFMAs are covered by slot_nops() before the first and after the last group
// of a slot.
template <bool FIRST>
__device__ __forceinline__ void mfma_exp_group(f32x16_t& acc, const uint4& qa, const u32x4_t& kb, bool krows,
                                               float x0, float x1, float b0, float b1, float c, float& s0,
                                               float& s1) {
  float t0, t1;
  const u32x4_t q = __builtin_bit_cast(u32x4_t, qa);
  const u32x4_t A = krows ? kb : q, B = krows ? q : kb;
  if constexpr (FIRST) {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %5, %6, 0\n\t"
        "v_fma_f32 %3, %7, %11, -%9\n\t"
        "v_fma_f32 %4, %8, %11, -%10\n\t"
        "v_exp_f32 %3, %3\n\t"
        "v_exp_f32 %4, %4\n\t"
        "v_add_f32 %1, %1, %3\n\t"
        "v_add_f32 %2, %2, %4"
        : "=&v"(acc), "+v"(s0), "+v"(s1), "=&v"(t0), "=&v"(t1)
        : "v"(A), "v"(B), "v"(x0), "v"(x1), "v"(b0), "v"(b1), "s"(c));
  } else {
    asm volatile(
        "v_mfma_f32_32x32x16_bf16 %0, %5, %6, %0\n\t"
        "v_fma_f32 %3, %7, %11, -%9\n\t"
        "v_fma_f32 %4, %8, %11, -%10\n\t"
        "v_exp_f32 %3, %3\n\t"
        "v_exp_f32 %4, %4\n\t"
        "v_add_f32 %1, %1, %3\n\t"
        "v_add_f32 %2, %2, %4"
        : "+v"(acc), "+v"(s0), "+v"(s1), "=&v"(t0), "=&v"(t1)
        : "v"(A), "v"(B), "v"(x0), "v"(x1), "v"(b0), "v"(b1), "s"(c));
  }
}

// As mfma_exp_group without the MFMA (a slot's first logits in pass 2) or
// without the logits (its last MFMA).
__device__ __forceinline__ void exp_group(float x0, float x1, float b0, float b1, float c, float& s0, float& s1) {
  float t0, t1;
  asm volatile(
      "v_fma_f32 %2, %4, %8, -%6\n\t"
      "v_fma_f32 %3, %5, %8, -%7\n\t"
      "v_exp_f32 %2, %2\n\t"
      "v_exp_f32 %3, %3\n\t"
      "v_add_f32 %0, %0, %2\n\t"
      "v_add_f32 %1, %1, %3"
      : "+v"(s0), "+v"(s1), "=&v"(t0), "=&v"(t1)
      : "v"(x0), "v"(x1), "v"(b0), "v"(b1), "s"(c));
}

__device__ __forceinline__ void mfma_group(f32x16_t& acc, const uint4& qa, const u32x4_t& kb, bool krows) {
  const u32x4_t q = __builtin_bit_cast(u32x4_t, qa);
  const u32x4_t A = krows ? kb : q, B = krows ? q : kb;
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(acc) : "v"(A), "v"(B));
}

// 24 wait states: more than any MFMA-result or MFMA-operand hazard needs, so
// that code the compiler places around a slot's groups never sees one.
__device__ __forceinline__ void slot_nops() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7"); }

// The prologue's contraction of slot 0 in the same alternating order.
template <int D, int NRTW, bool KROWS, int... M>
__device__ __forceinline__ void slot_contract(f32x16_t (&acc)[NRTW], const uint4 (&qr)[NRTW][D / 16],
                                              const u32x4_t (&kf)[D / 16], Seq<M...>) {
  (slot_mfma<D, NRTW, KROWS, M>(acc, qr, kf), ...);
}

// Pass 1, slot n: cur holds its dot products (key rows x query columns); the
// lane's query row of tile i sits at prompt position qpos[i].
template <int D, int NRTW, bool EDGE, int... M>
__device__ __forceinline__ void pass1_slot(const ScoreArgs& a, f32x16_t (&cur)[NRTW], f32x16_t (&nxt)[NRTW],
                                           const uint4 (&qr)[NRTW][D / 16], u32x4_t (&kf)[D / 16],
                                           int kbase, int half, const int (&qpos)[NRTW],
                                           float (&mrun)[NRTW], float (&zrun)[NRTW], Seq<M...>) {
  constexpr int LPM = 16 / (D / 16);  // logits of the tile-major sequence per MFMA
  float mnew[NRTW], mc[NRTW], s0[NRTW], s1[NRTW];
  bool dead[NRTW];
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    if constexpr (EDGE) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kbase + 8 * (e >> 2) + 4 * half + (e & 3);
        if (key >= a.s || key > qpos[i]) cur[i][e] = -INFINITY;
      }
    }
    mnew[i] = fmaxf(mrun[i], max16(cur[i]));
    dead[i] = EDGE && mnew[i] == -INFINITY;  // every key masked: contributes nothing
    mc[i] = dead[i] ? 0.f : mnew[i] * a.c;
    s0[i] = 0.f;
    s1[i] = 0.f;
  }
  slot_nops();
  auto group = [&](auto m_tag) {
    constexpr int MM = decltype(m_tag)::value;
    constexpr int CH = MM % NRTW, ST = MM / NRTW;
#pragma unroll
    for (int j = 0; j < LPM; j += 2) {
      const int L = MM * LPM + j, t = L / 16, e = L % 16;
      if (j == 0)
        mfma_exp_group<ST == 0>(nxt[CH], qr[CH][ST], kf[ST], true, cur[t][e], cur[t][e + 1], mc[t], mc[t], a.c,
                                s0[t], s1[t]);
      else
        exp_group(cur[t][e], cur[t][e + 1], mc[t], mc[t], a.c, s0[t], s1[t]);
    }
  };
  (group(std::integral_constant<int, M>{}), ...);
  slot_nops();
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    if (!dead[i]) {
      zrun[i] = zrun[i] * exp2_raw((mrun[i] - mnew[i]) * a.c) + (s0[i] + s1[i]);
      mrun[i] = mnew[i];
    }
  }
}

// Pass 2, slot n: cur holds its dot products (query rows x key columns); the
// lane's key is `key`; returns the key's weight summed over this wavefront's
// rows (both lane halves).
template <int D, int NRTW, int RS, bool EDGE, int... M>
__device__ __forceinline__ float pass2_slot(const ScoreArgs& a, const f32x16_t (&cur)[NRTW], f32x16_t (&nxt)[NRTW],
                                            const uint4 (&qr)[NRTW][D / 16], u32x4_t (&kf)[D / 16],
                                            const float (&breg)[NRTW][16], const int* qpos,
                                            int rg, int key, int half, Seq<M...>) {
  constexpr int NMF = NRTW * (D / 16);
  constexpr int LPM = 16 / (D / 16);
  float s0 = 0.f, s1 = 0.f;
  if constexpr (!EDGE) {
    slot_nops();
#pragma unroll
    for (int j = 0; j < LPM; j += 2) exp_group(cur[0][j], cur[0][j + 1], breg[0][j], breg[0][j + 1], a.c, s0, s1);
    auto group = [&](auto m_tag) {
      constexpr int MM = decltype(m_tag)::value;
      constexpr int CH = MM % NRTW, ST = MM / NRTW;
      if constexpr (MM + 1 < NMF) {
#pragma unroll
        for (int j = 0; j < LPM; j += 2) {
          const int L = (MM + 1) * LPM + j, t = L / 16, e = L % 16;
          if (j == 0)
            mfma_exp_group<ST == 0>(nxt[CH], qr[CH][ST], kf[ST], false, cur[t][e], cur[t][e + 1], breg[t][e],
                                    breg[t][e + 1], a.c, s0, s1);
          else
            exp_group(cur[t][e], cur[t][e + 1], breg[t][e], breg[t][e + 1], a.c, s0, s1);
        }
      } else {
        mfma_group(nxt[CH], qr[CH][ST], kf[ST], false);
      }
    };
    (group(std::integral_constant<int, M>{}), ...);
    slot_nops();
    return add_other_half(s0 + s1);
  }
  auto logits = [&](int m) {
#pragma unroll
    for (int j = 0; j < LPM; j += 2) {
      const int L = m * LPM + j, t = L / 16, e = L % 16;
      float p0 = exp2_raw(fmaf(cur[t][e], a.c, -breg[t][e]));
      float p1 = exp2_raw(fmaf(cur[t][e + 1], a.c, -breg[t][e + 1]));
      if constexpr (EDGE) {
        // positions of the query rows (e, e + 1 share a group of four), read
        // when needed: edge slots are rare and registers are not
        u32x4_t qq[1] = {lds_read_b128(qpos + (rg + RS * t) * kRowTile + 4 * half + 8 * (e >> 2))};
        lds_settle(qq);
        if (key >= a.s || key > (int)qq[0][e & 3]) p0 = 0.f;
        if (key >= a.s || key > (int)qq[0][(e + 1) & 3]) p1 = 0.f;
      }
      s0 += p0;
      s1 += p1;
    }
  };
  logits(0);
  auto group = [&](auto m_tag) {
    constexpr int MM = decltype(m_tag)::value;
    slot_mfma<D, NRTW, false, MM>(nxt, qr, kf);
    if constexpr (MM + 1 < NMF) logits(MM + 1);
  };
  (group(std::integral_constant<int, M>{}), ...);
  return add_other_half(s0 + s1);
}

struct Range {
  int t0, nst;  // first token, slots
  int toks;     // tokens per slot
  bool rev;     // slots visited from the last one down
  // first token of the n-th slot visited
  __device__ __forceinline__ int tok(int n) const { return t0 + (rev ? nst - 1 - n : n) * toks; }
};

__device__ __forceinline__ Range wg_range(const ScoreArgs& a, int split, int toks, bool rev) {
  Range r;
  r.t0 = split * a.blocks_per_wg * toks;
  int t1 = r.t0 + a.blocks_per_wg * toks;
  t1 = t1 < a.s ? t1 : a.s;
  r.nst = (t1 - r.t0 + toks - 1) / toks;
  r.toks = toks;
  r.rev = rev;
  return r;
}

// Ring prologue: copies of slots n0 .. kRingSlots-2 (slot 0 goes out first,
// before the query loads, so that a workgroup's first data is requested as
// early as possible; slots 1 and 2 follow them).
template <int D, int HG>
__device__ __forceinline__ void ring_fill(const ScoreArgs& a, int h0, const Range& rg, int wave, int lane,
                                          const uint32_t* off, unsigned char* smem, int n0 = 0, int n1 = kRingSlots - 1) {
#pragma unroll
  for (int n = 0; n < kRingSlots - 1; ++n)
    if (n >= n0 && n < n1 && n < rg.nst) slot_issue<D, HG>(a, h0, rg.tok(n), wave, lane, off, smem + n * kSlotBytes);
}

// Slots issued after the query loads by the prologue (slots 1 and 2).
__device__ __forceinline__ int slots_after_queries(const Range& rg) {
  return rg.nst < kRingSlots - 1 ? (rg.nst > 1 ? rg.nst - 1 : 0) : kRingSlots - 2;
}

// Top of ring iteration n: slot n has landed for the whole workgroup, and
// every wavefront is done with slot n-1, whose buffer then takes slot
// n + kRingSlots - 1.
template <int D, int HG>
__device__ __forceinline__ void ring_advance(const ScoreArgs& a, int h0, const Range& rg, int n, int wave,
                                             int lane, const uint32_t* off,
                                             unsigned char* smem) {
  using R = Ring<D, HG>;
  const int later = min(kRingSlots - 2, rg.nst - 1 - n);
  wait_slots<R::NI, kRingSlots - 2>(later);
  lds_barrier();
  const int nn = n + kRingSlots - 1;
  if (nn < rg.nst)
    slot_issue<D, HG>(a, h0, rg.tok(nn), wave, lane, off, smem + (nn % kRingSlots) * kSlotBytes);
}

// ---------------------------------------------------------------------------
// Pass 1
// ---------------------------------------------------------------------------
template <bool EDGE>
__device__ __forceinline__ void lse_update(const ScoreArgs& a, f32x16_t acc, int kbase, int half, int qpos,
                                           float& mrun, float& zrun) {
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

// Pass-1 update of one (slot, row tile) job whose dot products are in acc,
// with the MFMA chain of the next job (keys kf, query rows q) woven in: one
// MFMA, then the exponentials of 16 / (D / 16) logits, so that the matrix
// pipe and the VALU work side by side. Returns the next job's dot products.
template <int D, bool EDGE>
__device__ __forceinline__ f32x16_t lse_update_mfma(const ScoreArgs& a, f32x16_t acc, int kbase, int half,
                                                    int qpos, float& mrun, float& zrun, const uint4 (&kf)[D / 16],
                                                    const uint4 (&q)[D / 16]) {
  constexpr int NST = D / 16, PER = 16 / NST;
  if constexpr (EDGE) {
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int key = kbase + 8 * (e >> 2) + 4 * half + (e & 3);
      if (key >= a.s || key > qpos) acc[e] = -INFINITY;
    }
  }
  const float mnew = fmaxf(mrun, max16(acc));
  const bool dead = EDGE && mnew == -INFINITY;  // every key masked: contributes nothing
  const float mc = dead ? 0.f : mnew * a.c;
  f32x16_t nxt = {};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int st = 0; st < NST; ++st) {
    nxt = mfma32x32x16(kf[st], q[st], nxt);
#pragma unroll
    for (int e = st * PER; e < (st + 1) * PER; e += 2) {
      s0 += exp2_raw(fmaf(acc[e], a.c, -mc));
      s1 += exp2_raw(fmaf(acc[e + 1], a.c, -mc));
    }
    __builtin_amdgcn_sched_barrier(0);
  }
  if (!dead) {
    zrun = zrun * exp2_raw((mrun - mnew) * a.c) + (s0 + s1);
    mrun = mnew;
  }
  return nxt;
}

// ntile: row tiles this wavefront owns (wavefront-uniform, <= NRTW); FULL:
// every wavefront owns NRTW (known at compile time).
template <int D, int NRTW, bool FULL, bool EDGE>
__device__ __forceinline__ void pass1_tile(const ScoreArgs& a, const uint4 (&qr)[NRTW][D / 16],
                                           const uint4 (&kf)[D / 16], int kbase, int half, int ntile,
                                           const int (&qpos)[NRTW], float (&mrun)[NRTW], float (&zrun)[NRTW]) {
  if constexpr (NRTW <= 2) {
    // software-pipelined: the MFMAs of row tile i+1 overlap the VALU of i
    f32x16_t acc[2];
    acc[0] = contract<D, NRTW, true>(qr, kf, 0);
#pragma unroll
    for (int i = 0; i < NRTW; ++i) {
      const bool next = i + 1 < NRTW && (FULL || i + 1 < ntile);
      if (next) acc[(i + 1) & 1] = contract<D, NRTW, true>(qr, kf, i + 1);
      if (FULL || i < ntile) lse_update<EDGE>(a, acc[i & 1], kbase, half, qpos[i], mrun[i], zrun[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
    // register budget: one accumulator; the other wavefront on the SIMD
    // overlaps its MFMAs with this one's VALU
#pragma unroll
    for (int i = 0; i < NRTW; ++i) {
      if (i < ntile) lse_update<EDGE>(a, contract<D, NRTW, true>(qr, kf, i), kbase, half, qpos[i], mrun[i], zrun[i]);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
}

// A streaming-scan workgroup: its head group and token split, and the
// roles of this thread's wavefront.
template <int D, int HG>
struct WgCtx {
  int grp, split, h0, lane, wave, half, l32, head, ntile, first_hidden;
  Role ro;
};

template <int D, int NRT, int HG>
__device__ __forceinline__ WgCtx<D, HG> wg_ctx(const ScoreArgs& a) {
  using R = Ring<D, HG>;
  WgCtx<D, HG> c;
  const int work = xcd_remap(blockIdx.x, gridDim.x);
  c.grp = work / a.n_split;
  c.split = work % a.n_split;
  c.h0 = c.grp * HG;
  c.lane = threadIdx.x & 63;
  c.wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);  // wavefront-uniform: SGPRs
  c.half = c.lane >> 5;
  c.l32 = c.lane & 31;
  c.ro = role_of<D, HG>(c.wave);
  c.head = c.h0 + c.ro.hl;
  c.ntile = (NRT - c.ro.rg + R::RS - 1) / R::RS;  // the last row groups may own one fewer
  c.first_hidden = a.s - a.w + 1;
  return c;
}

// The pass-1 loop over a workgroup's slots: online (max, sum of
// exponentials) of every row the wavefront owns, per lane.
template <int D, int NRT, int HG>
__device__ __forceinline__ void pass1_loops(const ScoreArgs& a, const WgCtx<D, HG>& c, const Range& rg,
                                            const uint32_t* off, unsigned char* smem,
                                            const uint4 (&qr)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS][D / 16],
                                            const int (&qpos)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS],
                                            float (&mrun)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS],
                                            float (&zrun)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS]) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  constexpr bool PIPE = NRT % R::RS == 0;
  constexpr bool SLOT_PIPE = PIPE && NRTW <= 2 && KVC_SLOT_PIPE;
  const int h0 = c.h0, wave = c.wave, lane = c.lane, half = c.half, l32 = c.l32, ntile = c.ntile;
  const int first_hidden = c.first_hidden;
  const Role ro = c.ro;
  if constexpr (SLOT_PIPE) {
    using Ms = typename MakeSeq<NRTW * (D / 16)>::type;
    const int kt_off = ro.kt * kKeyTile;
    u32x4_t kf[D / 16];
    f32x16_t accA[NRTW], accB[NRTW];
    if (rg.nst > 0) {
      ring_advance<D, HG>(a, h0, rg, 0, wave, lane, off, smem);
      key_read<D, HG>(smem, ro.hl, ro.kt, half, l32, kf);
      using M0 = typename MakeSeq<NRTW * (D / 16)>::type;
      slot_contract<D, NRTW, true>(accA, qr, kf, M0{});
    }
    // slot n: its dot products in cur; the MFMAs of slot n+1 go to nxt (on
    // the last slot they redo slot n's keys into accumulators never read)
    auto step = [&](int n, f32x16_t (&cur)[NRTW], f32x16_t (&nxt)[NRTW]) {
      const int kbase = rg.tok(n) + kt_off;
      // the last slot re-reads its own fragments (its buffer is not refilled)
      // so that the fragment registers are redefined in every iteration
      const bool more = n + 1 < rg.nst;
      if (more) ring_advance<D, HG>(a, h0, rg, n + 1, wave, lane, off, smem);
      key_read<D, HG>(smem + ((more ? n + 1 : n) % kRingSlots) * kSlotBytes, ro.hl, ro.kt, half, l32, kf);
      if (kbase + kKeyTile > first_hidden)
        pass1_slot<D, NRTW, true>(a, cur, nxt, qr, kf, kbase, half, qpos, mrun, zrun, Ms{});
      else
        pass1_slot<D, NRTW, false>(a, cur, nxt, qr, kf, kbase, half, qpos, mrun, zrun, Ms{});
    };
    for (int n = 0; n < rg.nst; n += 2) {
      step(n, accA, accB);
      if (n + 1 < rg.nst) step(n + 1, accB, accA);
    }
  } else if constexpr (PIPE) {
    // Jobs (slot n, row tile i) in order; the MFMAs of each job run beside
    // the VALU work of the one before, across slot boundaries too. Jobs past
    // the prompt compute on clamped keys and are masked out.
    constexpr int LAST = NRTW - 1;
    const int kt_off = ro.kt * kKeyTile;
    uint4 kf[D / 16];
    f32x16_t A;
    if (rg.nst > 0) {
      ring_advance<D, HG>(a, h0, rg, 0, wave, lane, off, smem);
      load_key_regs<D, HG>(smem, ro.hl, ro.kt, half, l32, kf);
      A = contract<D, NRTW, true>(qr, kf, 0);
    }
    for (int n = 0; n < rg.nst; ++n) {
      const int kbase = rg.tok(n) + kt_off;
      const bool edge = kbase + kKeyTile > first_hidden;
      const bool more = n + 1 < rg.nst;
      // the next slot's key reads overlap this slot's remaining jobs
      u32x4_t raw[D / 16];
      if (more) {
        ring_advance<D, HG>(a, h0, rg, n + 1, wave, lane, off, smem);
        key_issue<D, HG>(smem + ((n + 1) % kRingSlots) * kSlotBytes, ro.hl, ro.kt, half, l32, raw);
      }
#pragma unroll
      for (int i = 0; i < LAST; ++i)
        A = edge ? lse_update_mfma<D, true>(a, A, kbase, half, qpos[i], mrun[i], zrun[i], kf, qr[i + 1])
                 : lse_update_mfma<D, false>(a, A, kbase, half, qpos[i], mrun[i], zrun[i], kf, qr[i + 1]);
      if (more) {
        key_settle<D>(raw, kf);
        A = edge ? lse_update_mfma<D, true>(a, A, kbase, half, qpos[LAST], mrun[LAST], zrun[LAST], kf, qr[0])
                 : lse_update_mfma<D, false>(a, A, kbase, half, qpos[LAST], mrun[LAST], zrun[LAST], kf, qr[0]);
      } else {
        if (edge) lse_update<true>(a, A, kbase, half, qpos[LAST], mrun[LAST], zrun[LAST]);
        else lse_update<false>(a, A, kbase, half, qpos[LAST], mrun[LAST], zrun[LAST]);
      }
    }
  } else {
    for (int n = 0; n < rg.nst; ++n) {
      ring_advance<D, HG>(a, h0, rg, n, wave, lane, off, smem);
      const unsigned char* slot = smem + (n % kRingSlots) * kSlotBytes;
      const int kbase = rg.tok(n) + ro.kt * kKeyTile;
      if (kbase < a.s) {
        uint4 kf[D / 16];
        load_key_regs<D, HG>(slot, ro.hl, ro.kt, half, l32, kf);
        if (kbase + kKeyTile <= first_hidden)
          pass1_tile<D, NRTW, NRT % R::RS == 0, false>(a, qr, kf, kbase, half, ntile, qpos, mrun, zrun);
        else
          pass1_tile<D, NRTW, NRT % R::RS == 0, true>(a, qr, kf, kbase, half, ntile, qpos, mrun, zrun);
      }
    }
  }

}

// Pass-1 epilogue: merge the lanes and wavefronts that share rows and write
// the workgroup's partial (max, sum) of every row (COHERENT: stores that
// other workgroups of the same launch can read).
template <int D, int NRT, int HG, bool COHERENT>
__device__ __forceinline__ void pass1_finish(const ScoreArgs& a, const WgCtx<D, HG>& c, unsigned char* smem,
                                             float (&mrun)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS],
                                             float (&zrun)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS]) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  constexpr int ROWS_PAD = NRT * kRowTile;
  const int h0 = c.h0, split = c.split, half = c.half, l32 = c.l32, ntile = c.ntile;
  const Role ro = c.ro;
  // lanes l and l+32 share a query row; then the KT wavefronts of a head
  // that own the same rows
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    const float mo = __shfl_xor(mrun[i], 32);
    const float zo = __shfl_xor(zrun[i], 32);
    lse_merge(mrun[i], zrun[i], mo, zo, a.c);
  }
  __syncthreads();  // the ring is idle now: every copy was waited for
  float2* red = reinterpret_cast<float2*>(smem);  // [HG][KT][ROWS_PAD]
  if (half == 0) {
#pragma unroll
    for (int i = 0; i < NRTW; ++i)
      if (i < ntile)
        red[(ro.hl * R::KT + ro.kt) * ROWS_PAD + (ro.rg + R::RS * i) * kRowTile + l32] = make_float2(mrun[i], zrun[i]);
  }
  __syncthreads();
  for (int idx = threadIdx.x; idx < HG * a.rows; idx += blockDim.x) {
    const int h = idx / a.rows, r = idx % a.rows;
    float m = -INFINITY, z = 0.f;
    for (int k = 0; k < R::KT; ++k) {
      const float2 p = red[(h * R::KT + k) * ROWS_PAD + r];
      lse_merge(m, z, p.x, p.y, a.c);
    }
    float2* dst = reinterpret_cast<float2*>(a.part) + ((int64_t)(h0 + h) * a.n_split + split) * ROWS_PAD + r;
    if constexpr (COHERENT)
      __hip_atomic_store(reinterpret_cast<uint64_t*>(dst), __builtin_bit_cast(uint64_t, make_float2(m, z)),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      *dst = make_float2(m, z);
  }
}

template <int D, int NRT, int HG>
__global__ void __launch_bounds__(8 * kWave) pass1_stream_kernel(ScoreArgs a) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  extern __shared__ __align__(16) unsigned char smem[];
  const WgCtx<D, HG> c = wg_ctx<D, NRT, HG>(a);
  const int split = c.split, h0 = c.h0, lane = c.lane, wave = c.wave, half = c.half, l32 = c.l32;
  const Role ro = c.ro;
  const int head = c.head;
  const Range rg = wg_range(a, split, R::TOKS, false);

  if (a.hist != nullptr && split == 0)
    for (int i = threadIdx.x; i < HG * kHistBins; i += blockDim.x) a.hist[(int64_t)h0 * kHistBins + i] = 0u;

  uint32_t off[R::NI];
  copy_offsets<D, HG>(a, wave, lane, off);
  ring_fill<D, HG>(a, h0, rg, wave, lane, off, smem, 0, 1);
  uint4 qr[NRTW][D / 16];
  load_query_regs<D, NRTW, R::RS>(a, head, ro.rg, NRT, half, l32, qr);
  ring_fill<D, HG>(a, h0, rg, wave, lane, off, smem, 1);
  vm_settle_after<R::NI>(qr, slots_after_queries(rg));

  float mrun[NRTW], zrun[NRTW];
  int qpos[NRTW];
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    mrun[i] = -INFINITY;
    zrun[i] = 0.f;
    const int r = (ro.rg + R::RS * i) * kRowTile + l32;
    qpos[i] = r < a.rows ? a.s - a.w + (r % a.w) : -1;
  }

  pass1_loops<D, NRT, HG>(a, c, rg, off, smem, qr, qpos, mrun, zrun);
  pass1_finish<D, NRT, HG, false>(a, c, smem, mrun, zrun);
}

// ---------------------------------------------------------------------------
// Pass 2
// ---------------------------------------------------------------------------
// bias / qpos: per row of the head, log2 of the normaliser and the prompt
// position of its query (-1 for padding rows), read from LDS inside the loop
// (the wide-row path, where registers are short; with up to two row tiles
// per wavefront the biases stay in registers, see weight_sum_r).
template <bool EDGE>
__device__ __forceinline__ void weight_sum(const ScoreArgs& a, const f32x16_t& acc, const float* bias,
                                           const int* qpos, int t, int key, int half, float& s0, float& s1) {
  const int o = t * kRowTile + 4 * half;
  // two rounds of 8 rows keep the register footprint small
#pragma unroll
  for (int q2 = 0; q2 < 4; q2 += 2) {
    u32x4_t bq[2] = {lds_read_b128(bias + o + 8 * q2), lds_read_b128(bias + o + 8 * q2 + 8)};
    lds_settle(bq);
#pragma unroll
    for (int q1 = 0; q1 < 2; ++q1) {
      const int q4 = q2 + q1;
      u32x4_t qv = {0u, 0u, 0u, 0u};
      if constexpr (EDGE) {
        u32x4_t qq[1] = {lds_read_b128(qpos + o + 8 * q4)};
        lds_settle(qq);
        qv = qq[0];
      }
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        float p = exp2_raw(fmaf(acc[4 * q4 + e4], a.c, -__uint_as_float(bq[q1][e4])));
        if constexpr (EDGE) {
          if (key >= a.s || key > (int)qv[e4]) p = 0.f;
        }
        if (e4 & 1) s1 += p; else s0 += p;
      }
    }
  }
}

// As weight_sum, with this lane's 16 row biases of the tile in registers.
template <bool EDGE>
__device__ __forceinline__ void weight_sum_r(const ScoreArgs& a, const f32x16_t& acc, const float (&b)[16],
                                             const int* qpos, int t, int key, int half, float& s0, float& s1) {
  const int o = t * kRowTile + 4 * half;
#pragma unroll
  for (int q4 = 0; q4 < 4; ++q4) {
    u32x4_t qv = {0u, 0u, 0u, 0u};
    if constexpr (EDGE) {
      u32x4_t qq[1] = {lds_read_b128(qpos + o + 8 * q4)};
      lds_settle(qq);
      qv = qq[0];
    }
#pragma unroll
    for (int e4 = 0; e4 < 4; ++e4) {
      float p = exp2_raw(fmaf(acc[4 * q4 + e4], a.c, -b[4 * q4 + e4]));
      if constexpr (EDGE) {
        if (key >= a.s || key > (int)qv[e4]) p = 0.f;
      }
      if (e4 & 1) s1 += p; else s0 += p;
    }
  }
}

template <int D, int NRTW, int RS, bool EDGE>
__device__ __forceinline__ float pass2_tile(const ScoreArgs& a, const uint4 (&qr)[NRTW][D / 16],
                                            const uint4 (&kf)[D / 16], const float* bias, const int* qpos,
                                            int key, int half, int rg, int ntile, const float (&breg)[NRTW][16]) {
  float s0 = 0.f, s1 = 0.f;
  if constexpr (NRTW <= 2) {
    f32x16_t acc[2];
    // the MFMA chains run at raised wave priority, so that the other
    // wavefront on the SIMD fills the matrix pipe's gaps with its VALU work
    // instead of both contending for issue
    __builtin_amdgcn_s_setprio(1);
    acc[0] = contract<D, NRTW, false>(qr, kf, 0);
    __builtin_amdgcn_s_setprio(0);
#pragma unroll
    for (int i = 0; i < NRTW; ++i) {
      __builtin_amdgcn_s_setprio(1);
      if (i + 1 < NRTW && i + 1 < ntile) acc[(i + 1) & 1] = contract<D, NRTW, false>(qr, kf, i + 1);
      __builtin_amdgcn_s_setprio(0);
      if (i < ntile) weight_sum_r<EDGE>(a, acc[i & 1], breg[i], qpos, rg + RS * i, key, half, s0, s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NRTW; ++i) {
      if (i < ntile) weight_sum<EDGE>(a, contract<D, NRTW, false>(qr, kf, i), bias, qpos, rg + RS * i, key, half, s0, s1);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  const float s = s0 + s1;
  return s + __shfl_xor(s, 32);
}

// Store a key's score (to device memory unless the caller asked for none,
// and to the segment's LDS copy when the launch selects) and count it in the
// head's LDS histogram.
__device__ __forceinline__ void emit_score(const ScoreArgs& a, float* out, uint32_t* lh, bool with_hist, int key,
                                           float sum, float* seg_sc = nullptr, int seg0 = 0) {
  if (a.scores != nullptr) out[key] = sum;
  if (seg_sc != nullptr) seg_sc[key - seg0] = sum;
  if (with_hist && key >= a.sink_end && key < a.rec_begin) {
    const uint32_t b = (__float_as_uint(sum) >> 19) & (kHistBins - 1);
    lds_add_u32(&lh[b >> 1], 1u << ((b & 1) * 16));
  }
}

// Where pass 2 leaves the segment's scores in LDS when the launch selects:
// past the ring, the row biases and prompt positions, the histogram halves
// and the row-group partial sums.
template <int NRT, int HG>
__device__ __forceinline__ float* pass2_seg_scores(unsigned char* smem) {
  constexpr int ROWS_PAD = NRT * kRowTile;
  return reinterpret_cast<float*>(smem + kRingBytes + HG * ROWS_PAD * (sizeof(float) + sizeof(int)) +
                                  HG * (kHistBins / 2) * sizeof(uint32_t)) +
         2 * 8 * kKeyTile;
}

// Pass 2 after its prologue: the ring's first slots are requested, qr holds
// the wavefront's query rows and (mv, zv) this thread's row normaliser.
template <int D, int NRT, int HG>
__device__ __forceinline__ void pass2_main(const ScoreArgs& a, const WgCtx<D, HG>& c, const Range& rg,
                                           const uint32_t* off, unsigned char* smem,
                                           const uint4 (&qr)[(NRT + Ring<D, HG>::RS - 1) / Ring<D, HG>::RS][D / 16],
                                           float mv, float zv, bool real_row) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  constexpr int ROWS_PAD = NRT * kRowTile;
  constexpr bool SLOT_PIPE = NRT % R::RS == 0 && NRTW <= 2 && KVC_SLOT_PIPE;
  float* bias_all = reinterpret_cast<float*>(smem + kRingBytes);            // [HG][ROWS_PAD]
  int* qpos_all = reinterpret_cast<int*>(bias_all + HG * ROWS_PAD);         // [HG][ROWS_PAD]
  uint32_t* hist2 = reinterpret_cast<uint32_t*>(qpos_all + HG * ROWS_PAD);  // [HG][kHistBins/2], u16 pairs
  float* psum = reinterpret_cast<float*>(hist2 + HG * (kHistBins / 2));     // [2][HG][KT][RS][32]
  // the segment's scores when the launch selects (one head per workgroup)
  float* seg_sc = a.fsel_kpt ? pass2_seg_scores<NRT, HG>(smem) : nullptr;
  static_assert(R::WAVES == 8, "row-group partial sums: [2][8 wavefronts][32]");
  const int seg0 = rg.t0;
  const int h0 = c.h0, lane = c.lane, wave = c.wave, half = c.half, l32 = c.l32, ntile = c.ntile;
  const int head = c.head, first_hidden = c.first_hidden;
  const Role ro = c.ro;
  const int bidx = threadIdx.x;
  // p = 2^(dot * c - (m * log2 e + log2 Z)); padding rows get +inf (p = 0).
  // One explicit fused multiply-add, so every kernel that runs this pass
  // rounds the bias alike.
  if (bidx < HG * ROWS_PAD) {
    bias_all[bidx] = real_row ? fmaf(mv, kLog2e, __log2f(zv)) : INFINITY;
    qpos_all[bidx] = real_row ? a.s - a.w + (bidx % ROWS_PAD) % a.w : -1;
  }
  const bool with_hist = a.hist != nullptr;
  if (with_hist)
    for (int i = threadIdx.x; i < HG * kHistBins / 2; i += blockDim.x) hist2[i] = 0u;

  const float* bias = bias_all + ro.hl * ROWS_PAD;
  const int* qpos = qpos_all + ro.hl * ROWS_PAD;
  uint32_t* lh = hist2 + ro.hl * (kHistBins / 2);
  float* out = a.scores != nullptr ? a.scores + (int64_t)head * a.s : nullptr;
  // row-group partial sums of slot n: psum[n & 1][hl][kt][rg][key]
  auto psum_at = [&](int n, int g) {
    return psum + ((((n & 1) * HG + ro.hl) * R::KT + ro.kt) * R::RS + g) * kKeyTile + l32;
  };
  // the first row group adds the partials of slot n in a fixed order
  auto finish = [&](int n) {
    const int key = rg.tok(n) + ro.kt * kKeyTile + l32;
    if (ro.rg == 0 && half == 0 && key < a.s) {
      float v[R::RS];
#pragma unroll
      for (int g = 0; g < R::RS; ++g) v[g] = lds_read_f32(psum_at(n, g));
      lds_settle(v);
      float sum = v[0];
#pragma unroll
      for (int g = 1; g < R::RS; ++g) sum += v[g];
      emit_score(a, out, lh, with_hist, key, sum, seg_sc, seg0);
    }
  };

  // this lane's row biases of its row tiles, once, after a barrier that makes
  // every thread's bias entry visible
  float breg[NRTW][16];
  auto load_breg = [&]() {
#pragma unroll
    for (int i = 0; i < NRTW; ++i) {
      const int o = (ro.rg + R::RS * i) * kRowTile + 4 * half;
      u32x4_t bq[4];
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) bq[q4] = lds_read_b128(bias + o + 8 * q4);
      lds_settle(bq);
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4)
#pragma unroll
        for (int e4 = 0; e4 < 4; ++e4) breg[i][4 * q4 + e4] = __uint_as_float(bq[q4][e4]);
    }
  };
  if constexpr (NRTW <= 2 && !SLOT_PIPE) {
    lds_barrier();
    load_breg();
  }
  if constexpr (SLOT_PIPE) {
    using Ms = typename MakeSeq<NRTW * (D / 16)>::type;
    u32x4_t kf[D / 16];
    f32x16_t accA[NRTW], accB[NRTW];
    if (rg.nst > 0) {
      // (the first barrier also publishes the biases)
      ring_advance<D, HG>(a, h0, rg, 0, wave, lane, off, smem);
      load_breg();
      key_read<D, HG>(smem, ro.hl, ro.kt, half, l32, kf);
      slot_contract<D, NRTW, false>(accA, qr, kf, Ms{});
    }
    // With two row groups each wavefront finishes half of its key tile's
    // keys: it keeps its own partial of the previous slot in a register and
    // reads the other group's with this slot's key fragments, so the sum
    // costs no LDS round trip of its own and both groups share the stores.
    float own_prev = 0.f;
    auto other_at = [&](int m) {
      return psum + ((((m & 1) * HG + ro.hl) * R::KT + ro.kt) * R::RS + (R::RS - 1 - ro.rg)) * kKeyTile + l32;
    };
    auto finalize = [&](int m, float own, float other) {
      const int key = rg.tok(m) + ro.kt * kKeyTile + l32;
      // own + other is v[0] + v[1] for either group (addition commutes)
      if (half == 0 && (l32 >> 4) == ro.rg && key < a.s) emit_score(a, out, lh, with_hist, key, own + other, seg_sc, seg0);
    };
    auto step = [&](int n, f32x16_t (&cur)[NRTW], f32x16_t (&nxt)[NRTW]) {
      const int kbase = rg.tok(n) + ro.kt * kKeyTile;
      const int key = kbase + l32;
      // the last slot re-reads its own fragments (its buffer is not refilled)
      // so that the fragment registers are redefined in every iteration
      const bool more = n + 1 < rg.nst;
      if (more) ring_advance<D, HG>(a, h0, rg, n + 1, wave, lane, off, smem);
      else if constexpr (R::RS > 1) lds_barrier();  // the other row groups' partial sums of slot n-1
      float other = 0.f;
      if constexpr (R::RS > 1)  // (for n = 0 the read lands in the idle half of psum and is unused)
        key_read_x<D, HG>(smem + ((more ? n + 1 : n) % kRingSlots) * kSlotBytes, ro.hl, ro.kt, half, l32, kf,
                          other_at(n - 1), other);
      else
        key_read<D, HG>(smem + ((more ? n + 1 : n) % kRingSlots) * kSlotBytes, ro.hl, ro.kt, half, l32, kf);
      const float sum = kbase + kKeyTile > first_hidden
                            ? pass2_slot<D, NRTW, R::RS, true>(a, cur, nxt, qr, kf, breg, qpos, ro.rg, key, half, Ms{})
                            : pass2_slot<D, NRTW, R::RS, false>(a, cur, nxt, qr, kf, breg, qpos, ro.rg, key, half, Ms{});
      if constexpr (R::RS > 1) {
        static_assert(R::RS == 2, "two row groups");
        if (half == 0) lds_write_f32(psum_at(n, ro.rg), sum);
        if (n > 0) finalize(n - 1, own_prev, other);
        own_prev = sum;
      } else {
        if (half == 0 && key < a.s) emit_score(a, out, lh, with_hist, key, sum, seg_sc, seg0);
      }
    };
    for (int n = 0; n < rg.nst; n += 2) {
      step(n, accA, accB);
      if (n + 1 < rg.nst) step(n + 1, accB, accA);
    }
    if constexpr (R::RS > 1) {
      if (rg.nst > 0) {
        lds_barrier();
        float other[1] = {lds_read_f32(other_at(rg.nst - 1))};
        lds_settle(other);
        finalize(rg.nst - 1, own_prev, other[0]);
      }
    }
  } else {
  for (int n = 0; n < rg.nst; ++n) {
    ring_advance<D, HG>(a, h0, rg, n, wave, lane, off, smem);
    if constexpr (R::RS > 1) {
      if (n > 0) finish(n - 1);
    }
    const unsigned char* slot = smem + (n % kRingSlots) * kSlotBytes;
    const int kbase = rg.tok(n) + ro.kt * kKeyTile;
    if (kbase < a.s) {
      uint4 kf[D / 16];
      load_key_regs<D, HG>(slot, ro.hl, ro.kt, half, l32, kf);
      const int key = kbase + l32;
      const float sum = kbase + kKeyTile <= first_hidden
                            ? pass2_tile<D, NRTW, R::RS, false>(a, qr, kf, bias, qpos, key, half, ro.rg, ntile, breg)
                            : pass2_tile<D, NRTW, R::RS, true>(a, qr, kf, bias, qpos, key, half, ro.rg, ntile, breg);
      if constexpr (R::RS > 1) {
        if (half == 0) lds_write_f32(psum_at(n, ro.rg), sum);
      } else {
        if (half == 0 && key < a.s) emit_score(a, out, lh, with_hist, key, sum, seg_sc, seg0);
      }
    }
  }
  }
  if constexpr (R::RS > 1 && !SLOT_PIPE) {
    lds_barrier();
    if (rg.nst > 0) finish(rg.nst - 1);
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

template <int D, int NRT, int HG>
__global__ void __launch_bounds__(8 * kWave) pass2_stream_kernel(ScoreArgs a) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  constexpr int ROWS_PAD = NRT * kRowTile;
  extern __shared__ __align__(16) unsigned char smem[];
  const WgCtx<D, HG> c = wg_ctx<D, NRT, HG>(a);
  const int h0 = c.h0, lane = c.lane, wave = c.wave, half = c.half, l32 = c.l32;
  const Role ro = c.ro;
  // the K that pass 1 read last (still in the memory-side cache) goes first
  const Range rg = wg_range(a, c.split, R::TOKS, true);

  uint32_t off[R::NI];
  copy_offsets<D, HG>(a, wave, lane, off);
  ring_fill<D, HG>(a, h0, rg, wave, lane, off, smem, 0, 1);
  uint4 qr[NRTW][D / 16];
  load_query_regs<D, NRTW, R::RS>(a, c.head, ro.rg, NRT, half, l32, qr);
  // this thread's normaliser (one bias entry per thread)
  static_assert(HG * ROWS_PAD <= R::WAVES * kWave, "one bias entry per thread");
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
  ring_fill<D, HG>(a, h0, rg, wave, lane, off, smem, 1);
  vm_settle_after<R::NI>(qr, slots_after_queries(rg));
  vm_settle(mv);
  vm_settle(zv);

  pass2_main<D, NRT, HG>(a, c, rg, off, smem, qr, mv, zv, real_row);
}

// ---------------------------------------------------------------------------
// Both scans in one launch. Each workgroup runs its pass-1 split, publishes
// its partial (max, sum) rows and requests its first pass-2 slots (the K it
// has just read). When every workgroup of its head group has published, it
// merges a share of the group's rows in the split combine's order (so the
// normalisers are bitwise those of the separate kernels) and publishes them;
// when all have done that, it runs its pass-2 split. Publishing is a flag per
// workgroup set to the launch's epoch after the data stores are acknowledged;
// data and flags go through device-coherent (cross-XCD) loads and stores. The
// host takes this path only when every workgroup of the launch can be
// resident at once, and a wait gives up after kSpinLimit polls (then the
// outputs are not valid) rather than spin for ever.
// ---------------------------------------------------------------------------
constexpr uint32_t kSpinLimit = 1u << 20;

// The XCD (accelerator die, with its own L2) this wavefront runs on.
__device__ __forceinline__ uint32_t xcc_id() {
  uint32_t v;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(v));
  return v & 0xFu;
}

// Whether this workgroup runs on the XCD its head group is meant for: the
// hardware deals workgroups to the eight XCDs in turn (workgroup b to XCD
// b % 8), xcd_remap gives every XCD a contiguous range of the work, and when
// that range holds whole head groups, a group placed as dealt lies on one
// XCD and shares its L2.
__device__ __forceinline__ bool on_group_xcd(const ScoreArgs& a) {
  return a.xcd_local && (gridDim.x & 7u) == 0 && (int)((gridDim.x >> 3) % (unsigned)a.n_split) == 0 &&
         xcc_id() == (blockIdx.x & 7u);
}

// A store that the group's later device-coherent loads observe: device
// coherent (through to memory) in general, or kept in the XCD's L2 when the
// whole group runs on that XCD (a workgroup-scope store is written through
// the CU's cache to the L2, where the other CUs' coherent loads find it).
template <typename T>
__device__ __forceinline__ void group_store(T* p, T v, bool local) {
  if (local) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Publish `value` in flag `flag` once this workgroup's stores are
// acknowledged (vmcnt) and every thread has issued its own (barrier).
__device__ __forceinline__ void group_arrive(uint64_t* flag, uint64_t value, bool local) {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  lds_barrier();
  if (threadIdx.x == 0) group_store(flag, value, local);
}

// Wait until the n_split flags from `flags` hold the epoch (or, with
// `either`, the epoch with its lowest bit flipped too): wavefront 0 polls
// them (a lane per flag), the others wait at an LDS-only barrier, so ring
// copies in flight stay in flight. Returns whether every flag holds exactly
// the epoch (the same answer in every workgroup that reads the same flags).
__device__ __forceinline__ bool group_wait(const ScoreArgs& a, const uint64_t* flags, bool either = false) {
  __shared__ uint32_t s_exact;
  if (threadIdx.x < kWave) {
    bool exact = true;
    for (uint32_t spins = 0; spins < kSpinLimit; ++spins) {
      bool ok = true;
      exact = true;
      for (int i = threadIdx.x; i < a.n_split; i += kWave) {
        const uint64_t f = __hip_atomic_load(flags + i, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ok = ok && (f == a.epoch || (either && f == (a.epoch ^ 1u)));
        exact = exact && f == a.epoch;
      }
      if (__all(ok)) break;
      __builtin_amdgcn_s_sleep(2);
    }
    if (threadIdx.x == 0) s_exact = 1u;
    if (!exact) s_exact = 0u;  // (any lane; the value written is the same)
  }
  lds_barrier();
  return s_exact != 0u;
}

// This workgroup's share of its head group's rows: the partials of every
// split merged as the split combine merges them (eight strided runs, then
// runs 1..7 into run 0), written as the normalisers (m in natural-log units).
template <int NRT, int HG>
__device__ __forceinline__ void group_merge(const ScoreArgs& a, int h0, int split, float2* red, bool local) {
  constexpr int ROWS_PAD = NRT * kRowTile;
  constexpr int RPR = kWave;  // rows per round: eight threads per row
  const int total = HG * a.rows;
  const int per = (total + a.n_split - 1) / a.n_split;
  const int r0 = split * per;
  const int nr = min(per, total - r0);
  const int sl = threadIdx.x & 7, rl = threadIdx.x >> 3;
  for (int base = 0; base < nr; base += RPR) {
    const int lr = base + rl;
    const bool ok = lr < nr;
    const int gr = r0 + (ok ? lr : 0);
    const int h = gr / a.rows, r = gr % a.rows;
    const uint64_t* part = reinterpret_cast<const uint64_t*>(a.part) + (int64_t)(h0 + h) * a.n_split * ROWS_PAD;
    float2 v[kMaxSplit / 8];
#pragma unroll
    for (int u = 0; u < kMaxSplit / 8; ++u) {
      const int sp = sl + 8 * u;
      v[u] = ok && sp < a.n_split
                 ? __builtin_bit_cast(float2, __hip_atomic_load(part + (int64_t)sp * ROWS_PAD + r, __ATOMIC_RELAXED,
                                                                __HIP_MEMORY_SCOPE_AGENT))
                 : make_float2(-INFINITY, 0.f);
    }
    float m = -INFINITY, z = 0.f;
#pragma unroll
    for (int u = 0; u < kMaxSplit / 8; ++u) lse_merge(m, z, v[u].x, v[u].y, a.c);
    red[sl * RPR + rl] = make_float2(m, z);
    __syncthreads();
    if (sl == 0 && ok) {
      for (int k = 1; k < 8; ++k) lse_merge(m, z, red[k * RPR + rl].x, red[k * RPR + rl].y, a.c);
      const int hh = r / a.w, i = r % a.w;
      const int64_t o = (int64_t)((h0 + h) * a.g + hh) * a.w + i;
      group_store(a.m_out + o, m * a.scale, local);
      group_store(a.z_out + o, z, local);
    }
    __syncthreads();
  }
}

template <int D, int NRT, int HG>
__global__ void __launch_bounds__(8 * kWave) scan_fused_kernel(ScoreArgs a, SelectArgs sa) {
  using R = Ring<D, HG>;
  constexpr int NRTW = (NRT + R::RS - 1) / R::RS;
  constexpr int ROWS_PAD = NRT * kRowTile;
  static_assert(NRTW <= 3, "at most three query-row tiles per wavefront");
  extern __shared__ __align__(16) unsigned char smem[];
  const WgCtx<D, HG> c = wg_ctx<D, NRT, HG>(a);
  const Range rg1 = wg_range(a, c.split, R::TOKS, false);
  const Range rg2 = wg_range(a, c.split, R::TOKS, true);  // pass 2 starts on the K read last
  const int wg = c.grp * a.n_split;  // the head group's first flag
  uint64_t* pub1 = a.sync + wg;                 // partials written
  uint64_t* pub2 = a.sync + kMaxFusedWgs + wg;  // normalisers written

  // pass 2 of every workgroup adds to the head group's histogram during this
  // launch, so the clear goes straight to memory
  if (a.hist != nullptr && c.split == 0)
    for (int i = threadIdx.x; i < HG * kHistBins; i += blockDim.x)
      __hip_atomic_store(a.hist + (int64_t)c.h0 * kHistBins + i, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  // the selection's round histograms likewise (written after the first rendezvous)
  if (HG == 1 && a.fsel_kpt && c.split == 0)
    for (int i = threadIdx.x; i < kFselR1Bins + kFselR2Bins; i += blockDim.x)
      __hip_atomic_store(a.ghist + (int64_t)c.h0 * (kFselR1Bins + kFselR2Bins) + i, 0u, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);

  uint32_t off[R::NI];
  copy_offsets<D, HG>(a, c.wave, c.lane, off);
  ring_fill<D, HG>(a, c.h0, rg1, c.wave, c.lane, off, smem, 0, 1);
  uint4 qr[NRTW][D / 16];
  load_query_regs<D, NRTW, R::RS>(a, c.head, c.ro.rg, NRT, c.half, c.l32, qr);
  ring_fill<D, HG>(a, c.h0, rg1, c.wave, c.lane, off, smem, 1);
  vm_settle_after<R::NI>(qr, slots_after_queries(rg1));
  float mrun[NRTW], zrun[NRTW];
  int qpos[NRTW];
#pragma unroll
  for (int i = 0; i < NRTW; ++i) {
    mrun[i] = -INFINITY;
    zrun[i] = 0.f;
    const int r = (c.ro.rg + R::RS * i) * kRowTile + c.l32;
    qpos[i] = r < a.rows ? a.s - a.w + (r % a.w) : -1;
  }
  pass1_loops<D, NRT, HG>(a, c, rg1, off, smem, qr, qpos, mrun, zrun);
  pass1_finish<D, NRT, HG, true>(a, c, smem, mrun, zrun);

  // The first rendezvous is device coherent; its flags also say whether each
  // workgroup runs on its group's XCD. If all do, the group's later stores
  // and flags stay in that XCD's L2.
  group_arrive(pub1 + c.split, on_group_xcd(a) ? a.epoch : a.epoch ^ 1u, false);
  ring_fill<D, HG>(a, c.h0, rg2, c.wave, c.lane, off, smem);  // (the reduction above is done with the ring)
  const bool local = group_wait(a, pub1, true);
  group_merge<NRT, HG>(a, c.h0, c.split, reinterpret_cast<float2*>(smem + kRingBytes), local);
  group_arrive(pub2 + c.split, a.epoch, local);
  group_wait(a, pub2);

  // this thread's normaliser (one bias entry per thread), as pass 2 reads it
  const int bidx = threadIdx.x;
  float mv = 0.f, zv = 1.f;
  bool real_row = false;
  if (bidx < HG * ROWS_PAD) {
    const int h = bidx / ROWS_PAD, r = bidx % ROWS_PAD;
    if (r < a.rows) {
      const int64_t o = (int64_t)((c.h0 + h) * a.g + r / a.w) * a.w + r % a.w;
      mv = __hip_atomic_load(a.m_in + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      zv = __hip_atomic_load(a.z_in + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      real_row = true;
    }
  }
  pass2_main<D, NRT, HG>(a, c, rg2, off, smem, qr, mv, zv, real_row);

  if constexpr (HG == 1) {
    if (a.fsel_kpt == 0) return;
    // selection and gather, once the head's scores and histogram are complete
    static_assert(sizeof(FselLds) <= kRingBytes, "the selection's LDS lives in the idle ring");
    const float* seg_sc = pass2_seg_scores<NRT, HG>(smem);
    uint64_t* pub3 = a.sync + 2 * kMaxFusedWgs + wg;
    group_arrive(pub3 + c.split, a.epoch, local);
    group_wait(a, pub3);
    const int64_t seg0 = rg1.t0;
    const int64_t seg1 = min((int64_t)a.s, seg0 + (int64_t)a.blocks_per_wg * R::TOKS);
    scan_select(a, sa, c.h0, c.split, seg0, seg1, seg_sc, smem, local, [&](int n) {
      uint64_t* pub = a.sync + (2 + n) * kMaxFusedWgs + wg;
      group_arrive(pub + c.split, a.epoch, local);
      group_wait(a, pub);
    });
  }
}

template <int D, int HG>
const void* fused_fn(int nrt) {
  constexpr int RS = Ring<D, HG>::RS;
  switch (nrt) {
    case 1: if constexpr (1 % RS == 0) return reinterpret_cast<const void*>(&scan_fused_kernel<D, 1, HG>); else return nullptr;
    case 2: return reinterpret_cast<const void*>(&scan_fused_kernel<D, 2, HG>);
    case 4: if constexpr ((4 + RS - 1) / RS <= 2) return reinterpret_cast<const void*>(&scan_fused_kernel<D, 4, HG>); else return nullptr;
    // (five and six row tiles: D = 128 with two row groups, as the host takes them)
    case 5: if constexpr (D == 128 && RS == 2) return reinterpret_cast<const void*>(&scan_fused_kernel<D, 5, HG>); else return nullptr;
    case 6: if constexpr (D == 128 && RS == 2) return reinterpret_cast<const void*>(&scan_fused_kernel<D, 6, HG>); else return nullptr;
    default: return nullptr;
  }
}

const void* stream_fused_fn(const Layer& L) {
  if (L.d == 128) return L.stream_hg == 2 ? fused_fn<128, 2>(L.row_tiles) : fused_fn<128, 1>(L.row_tiles);
  return L.stream_hg == 2 ? fused_fn<64, 2>(L.row_tiles) : fused_fn<64, 1>(L.row_tiles);
}

template <int D, int HG>
const void* pass1_stream_fn(int nrt) {
  switch (nrt) {
    case 1: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 1, HG>);
    case 2: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 2, HG>);
    case 3: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 3, HG>);
    case 4: return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 4, HG>);
    // (five and six row tiles: D = 128 only, as the host takes them)
    case 5: if constexpr (D == 128) return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 5, HG>); else return nullptr;
    case 6: if constexpr (D == 128) return reinterpret_cast<const void*>(&pass1_stream_kernel<D, 6, HG>); else return nullptr;
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
    // (five and six row tiles: D = 128 only, as the host takes them)
    case 5: if constexpr (D == 128) return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 5, HG>); else return nullptr;
    case 6: if constexpr (D == 128) return reinterpret_cast<const void*>(&pass2_stream_kernel<D, 6, HG>); else return nullptr;
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

int slot_key_tiles(const Layer& L) {
  if (L.d == 128) return L.stream_hg == 2 ? Ring<128, 2>::KT : Ring<128, 1>::KT;
  return L.stream_hg == 2 ? Ring<64, 2>::KT : Ring<64, 1>::KT;
}

}  // namespace

int stream_tokens(int d, int hg) { return kSlotBytes / (hg * d * 2); }

bool stream_offsets_fit(const Layer& L, int hg) {
  const int64_t toks = stream_tokens(L.d, hg);
  const int64_t span = ((toks - 1) * L.k_tok + (int64_t)(hg - 1) * L.k_head + L.d) * 2;
  return span < (1LL << 32);
}

int stream_row_groups(int d, int hg) {
  if (d == 128) return hg == 2 ? Ring<128, 2>::RS : Ring<128, 1>::RS;
  return hg == 2 ? Ring<64, 2>::RS : Ring<64, 1>::RS;
}

size_t pass1_stream_lds_bytes(const Layer& L) {
  const size_t red = (size_t)L.stream_hg * slot_key_tiles(L) * L.row_tiles * kRowTile * sizeof(float2);
  return red > (size_t)kRingBytes ? red : (size_t)kRingBytes;
}

size_t pass2_stream_lds_bytes(const Layer& L) {
  const size_t rows_pad = (size_t)L.row_tiles * kRowTile;
  const size_t psum = (size_t)2 * 8 * kKeyTile * sizeof(float);  // [2][HG][KT][RS][32]
  return kRingBytes + L.stream_hg * rows_pad * (sizeof(float) + sizeof(int)) +
         (size_t)L.stream_hg * (kHistBins / 2) * sizeof(uint32_t) + psum;
}

bool stream_fused_ok(const Layer& L, int cus) {
  if (L.stream_hg == 0 || stream_fused_fn(L) == nullptr) return false;
  const int64_t wgs = (int64_t)(L.hkv / L.stream_hg) * L.n_split;
  return wgs <= cus && wgs <= kMaxFusedWgs;
}

size_t fused_lds_bytes(const Layer& L) {
  // pass 1's reduction, the merge's (kWave rows x 8 partials past the ring),
  // pass 2's, and the segment's scores after pass 2's when the launch selects
  const size_t merge = (size_t)kRingBytes + (size_t)8 * kWave * sizeof(float2);
  size_t p2 = pass2_stream_lds_bytes(L);
  if (L.fsel) p2 += (size_t)L.blocks_per_wg * stream_tokens(L.d, L.stream_hg) * sizeof(float);
  return std::max({pass1_stream_lds_bytes(L), p2, merge});
}

hipError_t launch_stream_fused(const Layer& L, const ScoreArgs& a, const SelectArgs& sel, hipStream_t st) {
  const void* fn = stream_fused_fn(L);
  if (fn == nullptr) return hipErrorInvalidValue;
  const size_t lds = fused_lds_bytes(L);
  const hipError_t e = ensure_lds(fn, lds);
  if (e != hipSuccess) return e;
  ScoreArgs args = a;
  SelectArgs sargs = sel;
  void* kargs[] = {&args, &sargs};
  const dim3 grid((unsigned)(L.hkv / L.stream_hg * L.n_split));
  return hipLaunchKernel(fn, grid, dim3(8 * kWave), kargs, lds, st);
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
