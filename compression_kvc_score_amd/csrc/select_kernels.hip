// Selection of the retained keys (TideKV, Fig. 3 caption): per KV head, the
// mandatory sink and recent keys plus the top K_h - |mandatory| other keys by
// (score descending, index ascending), written in ascending key order; with
// the gather (TideKV, Fig. 2 caption) the same pass copies their K and V rows.
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
//           holding the k-th best candidate, counts per 1024-key sub-chunk its
//           candidates above b* and inside b*, and lists the patterns of those
//           inside b* in its own slot (no atomics).
//  compact  a small workgroup per sub-chunk reads its head's short lists (a
//           few thousand patterns, from L2), radix-selects in LDS the exact
//           pattern T of the k-th best candidate and how many candidates equal
//           to T are taken (the lowest indices: ties go to the lower index),
//           derives its first output row from the counts of the keys before
//           it, writes its kept indices (and positions) in ascending order and
//           copies the kept keys' K and V rows. If a slot or the lists
//           overflow (heavily tied scores), it selects by a radix over the
//           head's whole score row instead -- same result, slower.
//
// All counts are integers, so the output does not depend on the order in
// which workgroups run.

#include <type_traits>

#include "kvc_internal.h"
#include "select_common.h"
#include "wave_ops.h"

namespace kvc {
namespace {

constexpr int kThreads = kSelectThreads;          // 1024 per filter workgroup
constexpr int kWaves = kThreads / kWave;          // 16
constexpr int kChunk = kSelectChunk;              // 4096 keys per filter workgroup, 4 per thread
constexpr int kWavesPerSub = kWaves / kSubsPerChunk;
constexpr int kCWaves = kCompactThreads / kWave;  // 4 per compaction workgroup
constexpr int kMaxReplicas = 16;                  // compaction workgroups per sub-chunk, at most
constexpr int kCompactTarget = 512;               // compaction workgroups aimed for with the row copy
constexpr int kCopyUnroll = 8;                    // rows in flight per thread in the row copy

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// init: clear the per-head histograms.
// ---------------------------------------------------------------------------
__global__ void __launch_bounds__(256) init_kernel(SelectArgs a, int hkv) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < hkv * kHistBins) a.hist[i] = 0u;
}

// ---------------------------------------------------------------------------
// hist: per-chunk LDS histogram of candidate ranking values, merged into the
// head's global histogram; writes pooled values when pooling.
// ---------------------------------------------------------------------------
template <bool SIGNED>
__global__ void __launch_bounds__(kThreads) hist_kernel(SelectArgs a) {
  using KF = KeyFmt<SIGNED>;
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
    if (is_candidate(h, j)) atomicAdd(&lh[KF::bin(KF::key(v))], 1u);
  }
  __syncthreads();
  uint32_t* gh = a.hist + (int64_t)head * kHistBins;
  for (int i = threadIdx.x; i < kHistBins; i += kThreads)
    if (lh[i]) atomicAdd(&gh[i], lh[i]);
}

// ---------------------------------------------------------------------------
// filter: per chunk, count per sub-chunk the candidates above b* and inside
// it, and list, in key order, the patterns of those inside b* (in the chunk's
// own slot: no atomics).
// ---------------------------------------------------------------------------
template <bool SIGNED>
__global__ void __launch_bounds__(kThreads) filter_kernel(SelectArgs a) {
  using KF = KeyFmt<SIGNED>;
  __shared__ uint32_t scratch[kWaves];
  __shared__ uint32_t w_in[kWaves], w_above[kWaves];
  __shared__ uint32_t s_b;
  const int head = blockIdx.x / a.n_chunks, chunk = blockIdx.x % a.n_chunks;
  const HeadGeom h = head_geom(a, head);
  if (h.keep_all || h.k_sel == 0) return;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  // no bin reached: b* stays this value (a histogram that undercounts), and
  // the chunk then sends the compaction to the exact whole-row radix
  if (threadIdx.x == 0) s_b = 0xFFFFFFFFu;
  // this thread's four values, loaded before the histogram scan so that the
  // two memory round trips overlap
  const float* vals = a.vals + (int64_t)head * h.s;
  const int64_t j0 = (int64_t)chunk * kChunk + 4 * threadIdx.x;
  uint32_t bits[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    bits[e] = (j < h.s && is_candidate(h, j)) ? KF::key(vals[j]) : 0u;
  }
  // b*: the bin holding the k-th best candidate (thread t owns bins
  // 4095-4t .. 4092-4t, descending)
  const uint32_t* hist = a.hist + (int64_t)head * kHistBins;
  // (one 16-byte load per thread: a quarter of the cache-line requests of
  // four 4-byte loads at a 16-byte stride)
  typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));
  const u32x4v c4 = *reinterpret_cast<const u32x4v*>(hist + kHistBins - 4 - 4 * threadIdx.x);
  uint32_t c[4], loc = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    c[q] = c4[3 - q];  // bin 4095-4t-q
    loc += c[q];
  }
  uint32_t total;
  uint32_t before = block_exclusive_scan<kWaves>(loc, scratch, total);
  if (before < h.k_sel && h.k_sel <= before + loc) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (before < h.k_sel && h.k_sel <= before + c[q]) s_b = kHistBins - 1 - 4 * threadIdx.x - q;
      before += c[q];
    }
  }
  __syncthreads();
  const uint32_t bstar = s_b;
  uint32_t* slot = a.slots + ((int64_t)head * a.n_chunks + chunk) * kSlotStride;
  if (bstar == 0xFFFFFFFFu) {
    // an overflowing list count makes every compaction of the head resolve
    // from the scores themselves
    if (threadIdx.x < kSubsPerChunk) {
      slot[threadIdx.x] = threadIdx.x == 0 ? (uint32_t)kSlotCap + 1u : 0u;
      slot[kSubsPerChunk + threadIdx.x] = 0u;
    }
    if (threadIdx.x == 0) slot[2 * kSubsPerChunk] = 0u;
    return;
  }

  uint32_t above = 0, nin = 0;
  bool in[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    in[e] = false;
    if (j < h.s && is_candidate(h, j)) {
      const uint32_t b = KF::bin(bits[e]);
      above += b > bstar;
      in[e] = b == bstar;
      nin += in[e];
    }
  }
  const uint32_t inc_in = wave_inclusive_sum(nin), inc_ab = wave_inclusive_sum(above);
  if (lane == 63) {
    w_in[wave] = inc_in;
    w_above[wave] = inc_ab;
  }
  __syncthreads();
  uint32_t pos = inc_in - nin;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) pos += w < wave ? w_in[w] : 0u;
  // listed entries carry their sub-chunk: the keys inside b* share the bits
  // above LOW, so the low LOW bits identify them
  const uint32_t tag = (uint32_t)(chunk * kSubsPerChunk + (int)threadIdx.x / (kSub / 4)) << KF::LOW;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    if (in[e]) {
      if (pos < (uint32_t)kSlotCap) slot[kSlotHdr + pos] = tag | (bits[e] & KF::LOW_MASK);
      ++pos;
    }
  }
  // header: candidates inside b* and above it per sub-chunk, then b*
  if (threadIdx.x < kSubsPerChunk) {
    uint32_t ni = 0, na = 0;
#pragma unroll
    for (int q = 0; q < kWavesPerSub; ++q) {
      ni += w_in[kWavesPerSub * threadIdx.x + q];
      na += w_above[kWavesPerSub * threadIdx.x + q];
    }
    slot[threadIdx.x] = ni;
    slot[kSubsPerChunk + threadIdx.x] = na;
  }
  if (threadIdx.x == 0) slot[2 * kSubsPerChunk] = bstar;
}

// Shared memory of a compaction workgroup while it resolves its head.
struct ResolveLds {
  uint32_t* cbits;    // kCandCap listed entries (any order)
  uint32_t* hist1;    // 1024 radix bins (pattern bits 18..9)
  uint32_t* hist2;    // 512 radix bins (pattern bits 8..0)
  uint32_t* scratch;  // 2 * kCWaves
  uint32_t* pick;     // 2: digit and rank from pick_digit_wave
};

constexpr int kGroupChunks = 4;             // chunk slots a wavefront reads per round trip
constexpr int kSpecRounds = 4;              // 64-word reads per slot: header + 240 entries
constexpr int kSpecEntries = kSpecRounds * kWave - kSlotHdr;

enum ResolveOutcome { kResolved = 0, kNeedLists = 1, kNeedRow = 2 };

// Heads of at most this many chunks resolve with the chunk lists spread over
// every wavefront slot (two or more 256-word segments per chunk).
constexpr int kSpreadChunks = kCWaves * kGroupChunks / 2;

// As resolve_from_lists, for heads of at most NG x 16 chunks whose lists all
// fit in the first 256 words of their slots: the words stay in registers
// (wavefront w holds chunks 16g + 4w + i, word 64r + lane) and the radix
// histograms are built from them directly. Returns kNeedLists if a list is
// longer (nothing done yet) and kNeedRow if a slot overflowed.
template <bool SIGNED, int NG, typename OnBstar>
__device__ int resolve_in_registers(const SelectArgs& a, const HeadGeom& h, int head, int sub,
                                    const ResolveLds& m, uint32_t& thr, uint32_t& need_eq,
                                    uint32_t& gt_before, uint32_t& eq_before, OnBstar on_bstar) {
  using KF = KeyFmt<SIGNED>;
  constexpr int NW = kCWaves;
  constexpr int GC = NW * kGroupChunks;  // chunks per group
  const int nc = a.n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t* slots = a.slots + (int64_t)head * nc * kSlotStride;
  uint32_t v[NG][kGroupChunks][kSpecRounds];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = g * GC + wave * kGroupChunks + i;
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r)
        v[g][i][r] = c < nc ? slots[(int64_t)c * kSlotStride + r * kWave + lane] : 0u;
    }
  // headers (wavefront-uniform): listed entries per chunk; candidates above b*
  // in all sub-chunks and in those before this one; long lists; b* (chunk 0)
  uint32_t n[NG][kGroupChunks];
  uint32_t sums[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = g * GC + wave * kGroupChunks + i;
      n[g][i] = 0u;
#pragma unroll
      for (int q = 0; q < kSubsPerChunk; ++q) {
        n[g][i] += (uint32_t)__builtin_amdgcn_readlane((int)v[g][i][0], q);
        const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)v[g][i][0], kSubsPerChunk + q);
        sums[0] += ab;
        sums[1] += c * kSubsPerChunk + q < sub ? ab : 0u;
      }
      if (n[g][i] > (uint32_t)kSpecEntries) sums[2] += n[g][i] > (uint32_t)kSlotCap ? 0x10000u : 1u;
    }
  if (wave == 0) sums[3] = (uint32_t)__builtin_amdgcn_readlane((int)v[0][0][0], 2 * kSubsPerChunk);
  if (lane != 0) {  // wavefront-uniform: count once per wavefront
#pragma unroll
    for (int i = 0; i < 4; ++i) sums[i] = 0u;
  }
  block_sums<NW, 4, true>(sums, m.scratch);
  if (sums[2] >= 0x10000u) return kNeedRow;
  if (sums[2] != 0u) return kNeedLists;
  const uint32_t bstar = sums[3];
  on_bstar(bstar);

  // radix over the LOW key bits: the top 10, then the other R2 (the listed
  // keys share the bits above LOW)
  uint32_t rem = h.k_sel - sums[0];  // rank of the threshold inside the lists
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = r * kWave + lane - kSlotHdr;
        if (e >= 0 && (uint32_t)e < n[g][i]) atomicAdd(&m.hist1[(v[g][i][r] >> KF::R2) & 1023u], 1u);
      }
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<1024>(m.hist1, rem, m.pick);
  wg_sync<true>();
  const uint32_t d1 = m.pick[0];
  rem = m.pick[1];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = r * kWave + lane - kSlotHdr;
        if (e >= 0 && (uint32_t)e < n[g][i] && ((v[g][i][r] >> KF::R2) & 1023u) == d1)
          atomicAdd(&m.hist2[v[g][i][r] & (KF::R2_BINS - 1u)], 1u);
      }
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<KF::R2_BINS>(m.hist2, rem, m.pick);
  wg_sync<true>();
  const uint32_t low = (d1 << KF::R2) | m.pick[0];
  need_eq = m.pick[1];
  thr = (bstar << KF::LOW) | low;
  // listed candidates of the sub-chunks before this one
  uint32_t gq[2] = {0u, 0u};
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = r * kWave + lane - kSlotHdr;
        const uint32_t x = v[g][i][r];
        if (e >= 0 && (uint32_t)e < n[g][i] && (int)(x >> KF::LOW) < sub) {
          gq[0] += (x & KF::LOW_MASK) > low;
          gq[1] += (x & KF::LOW_MASK) == low;
        }
      }
  block_sums<NW, 2, true>(gq, m.scratch);
  gt_before = sums[1] + gq[0];
  eq_before = gq[1];
  return kResolved;
}

// As resolve_in_registers, for heads of few chunks (one group): the 16
// wavefront slots spread over the head's chunks, slot u reading 256-word
// segment u / nc of chunk u % nc (up to kMaxSegs per chunk), so that lists
// longer than one segment stay in registers (at 16K keys the threshold bin's
// lists run to about 500 entries per chunk). Returns kNeedLists if a list is
// longer than its chunk's segments (nothing done yet) and kNeedRow if a slot
// overflowed. It runs in a compaction kernel of its own: folded into the one
// of the longer prompts, it made those 1-2 us slower.
template <bool SIGNED, typename OnBstar, int NG = 1, bool SPREAD = true>
__device__ int resolve_spread(const SelectArgs& a, const HeadGeom& h, int head, int sub,
                                    const ResolveLds& m, uint32_t& thr, uint32_t& need_eq,
                                    uint32_t& gt_before, uint32_t& eq_before, OnBstar on_bstar) {
  using KF = KeyFmt<SIGNED>;
  constexpr int NW = kCWaves;
  constexpr int GC = NW * kGroupChunks;  // wavefront slots per group
  constexpr int SEGW = kSpecRounds * kWave;        // words per segment
  constexpr int kMaxSegs = kSlotStride / SEGW;     // whole segments inside a slot
  __shared__ uint32_t s_cn[GC];                    // listed entries per chunk (one group)
  const int nc = a.n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t* slots = a.slots + (int64_t)head * nc * kSlotStride;
  static_assert(!SPREAD || NG == 1, "segments spread over one group");
  // chunk (nc for a slot without one) and segment of slot (g, i)
#define KVC_SLOT_CHUNK(g, i)                                                                        \
  (SPREAD ? ((wave * kGroupChunks + (i)) / nc < kMaxSegs ? (wave * kGroupChunks + (i)) % nc : nc) \
          : ((g) * GC + wave * kGroupChunks + (i) < nc ? (g) * GC + wave * kGroupChunks + (i) : nc))
#define KVC_SLOT_SEG(i) (SPREAD ? (wave * kGroupChunks + (i)) / nc : 0)
  uint32_t v[NG][kGroupChunks][kSpecRounds];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = KVC_SLOT_CHUNK(g, i);
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r)
        v[g][i][r] = c < nc ? slots[(int64_t)c * kSlotStride + KVC_SLOT_SEG(i) * SEGW + r * kWave + lane] : 0u;
    }
  // headers (wavefront-uniform, from each chunk's first segment): listed
  // entries per chunk; candidates above b* in all sub-chunks and in those
  // before this one; long lists; b* (chunk 0)
  uint32_t n[NG][kGroupChunks];
  uint32_t sums[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = KVC_SLOT_CHUNK(g, i);
      n[g][i] = 0u;
      if (c < nc && KVC_SLOT_SEG(i) == 0) {
#pragma unroll
        for (int q = 0; q < kSubsPerChunk; ++q) {
          n[g][i] += (uint32_t)__builtin_amdgcn_readlane((int)v[g][i][0], q);
          const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)v[g][i][0], kSubsPerChunk + q);
          sums[0] += ab;
          sums[1] += c * kSubsPerChunk + q < sub ? ab : 0u;
        }
        // the words this chunk's slots cover
        const int segs = SPREAD ? min(kMaxSegs, (GC - 1 - c) / nc + 1) : 1;
        if (n[g][i] > (uint32_t)(segs * SEGW - kSlotHdr)) sums[2] += n[g][i] > (uint32_t)kSlotCap ? 0x10000u : 1u;
        if (SPREAD && lane == 0) s_cn[c] = n[g][i];
      }
    }
  if (wave == 0) sums[3] = (uint32_t)__builtin_amdgcn_readlane((int)v[0][0][0], 2 * kSubsPerChunk);
  if (lane != 0) {  // wavefront-uniform: count once per wavefront
#pragma unroll
    for (int i = 0; i < 4; ++i) sums[i] = 0u;
  }
  block_sums<NW, 4, true>(sums, m.scratch);  // (its barrier also publishes s_cn)
  if (sums[2] >= 0x10000u) return kNeedRow;
  if (sums[2] != 0u) return kNeedLists;
  const uint32_t bstar = sums[3];
  on_bstar(bstar);
  // every slot's entry count: its chunk's (spread: from LDS)
  if constexpr (SPREAD) {
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = KVC_SLOT_CHUNK(0, i);
      n[0][i] = c < nc ? s_cn[c] : 0u;
    }
  }
  // index of word (g, i, r) of this lane among its chunk's listed entries
#define KVC_SLOT_ENTRY(g, i, r) (KVC_SLOT_SEG(i) * SEGW + (r) * kWave + lane - kSlotHdr)

  // radix over the LOW key bits: the top 10, then the other R2 (the listed
  // keys share the bits above LOW)
  uint32_t rem = h.k_sel - sums[0];  // rank of the threshold inside the lists
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = KVC_SLOT_ENTRY(g, i, r);
        if (e >= 0 && (uint32_t)e < n[g][i]) atomicAdd(&m.hist1[(v[g][i][r] >> KF::R2) & 1023u], 1u);
      }
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<1024>(m.hist1, rem, m.pick);
  wg_sync<true>();
  const uint32_t d1 = m.pick[0];
  rem = m.pick[1];
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = KVC_SLOT_ENTRY(g, i, r);
        if (e >= 0 && (uint32_t)e < n[g][i] && ((v[g][i][r] >> KF::R2) & 1023u) == d1)
          atomicAdd(&m.hist2[v[g][i][r] & (KF::R2_BINS - 1u)], 1u);
      }
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<KF::R2_BINS>(m.hist2, rem, m.pick);
  wg_sync<true>();
  const uint32_t low = (d1 << KF::R2) | m.pick[0];
  need_eq = m.pick[1];
  thr = (bstar << KF::LOW) | low;
  // listed candidates of the sub-chunks before this one
  uint32_t gq[2] = {0u, 0u};
#pragma unroll
  for (int g = 0; g < NG; ++g)
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i)
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r) {
        const int e = KVC_SLOT_ENTRY(g, i, r);
        const uint32_t x = v[g][i][r];
        if (e >= 0 && (uint32_t)e < n[g][i] && (int)(x >> KF::LOW) < sub) {
          gq[0] += (x & KF::LOW_MASK) > low;
          gq[1] += (x & KF::LOW_MASK) == low;
        }
      }
  block_sums<NW, 2, true>(gq, m.scratch);
  gt_before = sums[1] + gq[0];
  eq_before = gq[1];
  return kResolved;
#undef KVC_SLOT_ENTRY
#undef KVC_SLOT_SEG
#undef KVC_SLOT_CHUNK
}

// Threshold of one head, resolved from the chunk lists: the pattern T of the
// k-th best candidate, the number need_eq of candidates equal to T that are
// kept, and, for the keys before sub-chunk `sub`, the candidates above T and
// equal to T. One speculative read per slot brings its header and most of its
// list; once b* is known, on_bstar(b*) runs (before the radix rounds).
// Returns false (nothing resolved) if a chunk's slot or the gathered list
// overflowed.
template <bool SIGNED, typename OnBstar>
__device__ bool resolve_from_lists(const SelectArgs& a, const HeadGeom& h, int head, int sub,
                                   const ResolveLds& m, uint32_t& thr, uint32_t& need_eq,
                                   uint32_t& gt_before, uint32_t& eq_before, OnBstar on_bstar) {
  using KF = KeyFmt<SIGNED>;
  constexpr int NW = kCWaves;
  __shared__ uint32_t s_count, s_flag, s_bstar;
  const int nc = a.n_chunks;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t* slots = a.slots + (int64_t)head * nc * kSlotStride;
  if (threadIdx.x == 0) {
    s_count = 0u;
    s_flag = 0u;
  }
  uint32_t ab_all = 0, ab_before = 0;  // wavefront-uniform partial sums
  for (int c0 = 0; c0 < nc; c0 += NW * kGroupChunks) {
    // this wavefront's chunks of the group: c0 + wave * kGroupChunks + i
    uint32_t v[kGroupChunks][kSpecRounds];
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = c0 + wave * kGroupChunks + i;
#pragma unroll
      for (int r = 0; r < kSpecRounds; ++r)
        v[i][r] = c < nc ? slots[(int64_t)c * kSlotStride + r * kWave + lane] : 0u;
    }
    if (c0 == 0) wg_sync<true>();  // s_count and the radix bins are cleared
    uint32_t n[kGroupChunks], tot = 0;
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      n[i] = 0u;
#pragma unroll
      for (int q = 0; q < kSubsPerChunk; ++q) {
        const int c = c0 + wave * kGroupChunks + i;
        n[i] += (uint32_t)__builtin_amdgcn_readlane((int)v[i][0], q);
        const uint32_t ab = (uint32_t)__builtin_amdgcn_readlane((int)v[i][0], kSubsPerChunk + q);
        ab_all += ab;
        ab_before += c * kSubsPerChunk + q < sub ? ab : 0u;
      }
      tot += n[i];
    }
    if (c0 == 0 && wave == 0 && lane == 2 * kSubsPerChunk) s_bstar = v[0][0];
    // space in the LDS list for this wavefront's chunks
    uint32_t base = 0;
    if (lane == 0) base = atomicAdd(&s_count, tot);
    base = (uint32_t)__builtin_amdgcn_readfirstlane((int)base);
#pragma unroll
    for (int i = 0; i < kGroupChunks; ++i) {
      const int c = c0 + wave * kGroupChunks + i;
      if (n[i] > (uint32_t)kSlotCap || base + n[i] > (uint32_t)kCandCap) {
        if (lane == 0) s_flag = 1u;
      } else {
#pragma unroll
        for (int r = 0; r < kSpecRounds; ++r) {
          const int e = r * kWave + lane - kSlotHdr;  // entry index of this word
          if (e >= 0 && (uint32_t)e < n[i]) m.cbits[base + e] = v[i][r];
        }
        // rest of a long list
        for (uint32_t e = kSpecEntries + lane; e < n[i]; e += kWave)
          m.cbits[base + e] = slots[(int64_t)c * kSlotStride + kSlotHdr + e];
      }
      base += n[i];
    }
  }
  if (lane != 0) {  // wavefront-uniform: count once per wavefront
    ab_all = 0u;
    ab_before = 0u;
  }
  block_sum2<NW, true>(ab_all, ab_before, m.scratch);
  if (s_flag != 0u) return false;
  on_bstar(s_bstar);

  // radix over pattern bits 18..9, then 8..0 (the listed patterns share the rest)
  const uint32_t n_total = s_count;
  uint32_t rem = h.k_sel - ab_all;  // rank of the threshold inside the list
  for (uint32_t i = threadIdx.x; i < n_total; i += kCompactThreads)
    atomicAdd(&m.hist1[(m.cbits[i] >> KF::R2) & 1023u], 1u);
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<1024>(m.hist1, rem, m.pick);
  wg_sync<true>();
  const uint32_t d1 = m.pick[0];
  rem = m.pick[1];
  for (uint32_t i = threadIdx.x; i < n_total; i += kCompactThreads) {
    const uint32_t e = m.cbits[i];
    if (((e >> KF::R2) & 1023u) == d1) atomicAdd(&m.hist2[e & (KF::R2_BINS - 1u)], 1u);
  }
  wg_sync<true>();
  if (threadIdx.x < kWave) pick_digit_wave<KF::R2_BINS>(m.hist2, rem, m.pick);
  wg_sync<true>();
  const uint32_t low = (d1 << KF::R2) | m.pick[0];
  need_eq = m.pick[1];
  thr = (s_bstar << KF::LOW) | low;
  // listed candidates of the sub-chunks before this one
  uint32_t g = 0, q = 0;
  for (uint32_t i = threadIdx.x; i < n_total; i += kCompactThreads) {
    const uint32_t e = m.cbits[i];
    if ((int)(e >> KF::LOW) < sub) {
      g += (e & KF::LOW_MASK) > low;
      q += (e & KF::LOW_MASK) == low;
    }
  }
  block_sum2<NW, true>(g, q, m.scratch);
  gt_before = ab_before + g;
  eq_before = q;
  return true;
}

// Slow path: the same quantities by radix passes over the head's whole
// score row (8 bits per round from the top).
template <bool SIGNED>
__device__ void resolve_from_row(const SelectArgs& a, const HeadGeom& h, int head, int sub,
                                 const ResolveLds& m, uint32_t& thr, uint32_t& need_eq,
                                 uint32_t& gt_before, uint32_t& eq_before) {
  using KF = KeyFmt<SIGNED>;
  constexpr int NT = kCompactThreads, NW = kCWaves;
  const float* row = a.vals + (int64_t)head * h.s;
  uint32_t prefix = 0u, mask = 0u, rem = h.k_sel;
  for (int shift = 24; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += NT) m.hist1[i] = 0u;
    wg_sync<true>();
    for (int64_t j = h.sink_end + threadIdx.x; j < h.rec_begin; j += NT) {
      const uint32_t u = KF::key(row[j]);
      if ((u & mask) == prefix) atomicAdd(&m.hist1[(u >> shift) & 255u], 1u);
    }
    wg_sync<true>();
    if (threadIdx.x < kWave) pick_digit_wave<256>(m.hist1, rem, m.pick);
    wg_sync<true>();
    prefix |= m.pick[0] << shift;
    rem = m.pick[1];
    mask |= 255u << shift;
    wg_sync<true>();
  }
  thr = prefix;
  need_eq = rem;
  const int64_t s0 = (int64_t)sub * kSub;
  const int64_t lim = s0 < h.rec_begin ? s0 : h.rec_begin;
  uint32_t g = 0, q = 0;
  for (int64_t j = h.sink_end + threadIdx.x; j < lim; j += NT) {
    const uint32_t u = KF::key(row[j]);
    g += u > thr;
    q += u == thr;
  }
  block_sum2<NW, true>(g, q, m.scratch);
  gt_before = g;
  eq_before = q;
}

// ---------------------------------------------------------------------------
// compact: per sub-chunk, resolve the head's threshold, then write the kept
// indices (and positions) in ascending order from the sub-chunk's first
// output row; with GATHER also copy their K and V rows. SPREAD: the heads
// have at most kSpreadChunks chunks, resolved by resolve_spread.
// ---------------------------------------------------------------------------
template <bool GATHER, bool SIGNED, bool SPREAD>
__global__ void __launch_bounds__(kCompactThreads) compact_kernel(SelectArgs a) {
  using KF = KeyFmt<SIGNED>;
  extern __shared__ __align__(16) unsigned char smem[];
  __shared__ uint32_t hist1[1024], hist2[1024];
  __shared__ uint32_t scratch[4 * kCWaves], pick[2];
  __shared__ int32_t kept_keys[GATHER ? kSub : 1];
  // replicas of a sub-chunk resolve it alike; replica 0 writes the indices
  // and each copies every replicas-th group of kept rows
  const int rep = blockIdx.x % a.replicas, blk = blockIdx.x / a.replicas;
  const int head = blk / a.n_subs, sub = blk % a.n_subs;
  const HeadGeom h = head_geom(a, head);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t s0 = (int64_t)sub * kSub;
  const int64_t j0 = s0 + 4 * threadIdx.x;
  const bool ranked = !h.keep_all && h.k_sel > 0;
  uint32_t vb[4] = {0u, 0u, 0u, 0u};
  uint32_t thr = 0xFFFFFFFFu, quota = 0u, first;
  uint32_t touched[4][4] = {};  // words of prefetched rows (consumed at the end)
  if (ranked) {
    const float* vals = a.vals + (int64_t)head * h.s;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int64_t j = j0 + e;
      if (j < h.s && is_candidate(h, j)) vb[e] = KF::key(vals[j]);
    }
    for (int i = threadIdx.x; i < 1024; i += kCompactThreads) hist1[i] = 0u;
    for (int i = threadIdx.x; i < 1024; i += kCompactThreads) hist2[i] = 0u;
    ResolveLds m;
    m.cbits = reinterpret_cast<uint32_t*>(smem);
    m.hist1 = hist1;
    m.hist2 = hist2;
    m.scratch = scratch;
    m.pick = pick;
    // with the copy: once b* is known, touch the rows of the keys that are
    // kept for sure (mandatory, or above b*) or may be (inside b*), so that
    // they are in L2 when the copy runs after the resolve
    auto prefetch = [&](uint32_t bstar) {
      if constexpr (GATHER) {
        if (a.replicas > 1) return;  // the copy is spread thin enough
        // decide for all four keys first: a decision after a prefetch would
        // wait for it
        bool want[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int64_t j = j0 + e;
          want[e] = j < h.s && (!is_candidate(h, j) || KF::bin(vb[e]) >= bstar);
        }
        // every address first, outside the conditional loads, so that the
        // layout fields are read once rather than inside each branch
        const uint16_t* kr0 = a.k + j0 * a.k_tok + (int64_t)head * a.k_head;
        const uint16_t* vr0 = a.v + j0 * a.v_tok + (int64_t)head * a.v_head;
        const int64_t kt = a.k_tok, vt = a.v_tok;
        const bool wide = a.d > 64;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          if (want[e]) {
            // one word per 128-byte line; the words are only consumed at the
            // end of the kernel, so nothing waits for them before then
            const uint16_t* kr = kr0 + e * kt;
            const uint16_t* vr = vr0 + e * vt;
            touched[e][0] = *reinterpret_cast<const uint32_t*>(kr);
            touched[e][1] = *reinterpret_cast<const uint32_t*>(vr);
            if (wide) {
              touched[e][2] = *reinterpret_cast<const uint32_t*>(kr + 64);
              touched[e][3] = *reinterpret_cast<const uint32_t*>(vr + 64);
            }
          }
        }
      }
    };
    uint32_t need_eq, gt_before, eq_before;
    constexpr int GC = kCWaves * kGroupChunks;
    int outcome = kNeedLists;
    if constexpr (SPREAD) {
      outcome = resolve_spread<SIGNED>(a, h, head, sub, m, thr, need_eq, gt_before, eq_before, prefetch);
    } else {
      if (a.n_chunks <= GC)
        outcome = resolve_in_registers<SIGNED, 1>(a, h, head, sub, m, thr, need_eq, gt_before, eq_before, prefetch);
      else if (a.n_chunks <= 2 * GC)
        outcome = resolve_in_registers<SIGNED, 2>(a, h, head, sub, m, thr, need_eq, gt_before, eq_before, prefetch);
    }
    if (outcome == kNeedLists)
      outcome = resolve_from_lists<SIGNED>(a, h, head, sub, m, thr, need_eq, gt_before, eq_before, prefetch)
                    ? kResolved
                    : kNeedRow;
    if (outcome == kNeedRow) resolve_from_row<SIGNED>(a, h, head, sub, m, thr, need_eq, gt_before, eq_before);
    quota = need_eq > eq_before ? need_eq - eq_before : 0u;  // equal candidates this sub-chunk may take
    first = mandatory_in(h, 0, s0) + gt_before + (need_eq < eq_before ? need_eq : eq_before);
  } else {
    first = h.keep_all ? (uint32_t)s0 : mandatory_in(h, 0, s0);
  }
  // 1: kept; 2: equal to T (taken in key order while the quota lasts)
  uint32_t flag[4], n_kept = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int64_t j = j0 + e;
    flag[e] = 0u;
    if (j >= h.s) continue;
    if (h.keep_all || !is_candidate(h, j)) flag[e] = 1u;
    else if (ranked) flag[e] = vb[e] > thr ? 1u : (vb[e] == thr ? 2u : 0u);
    n_kept += flag[e] == 1u;
    n_eq += flag[e] == 2u;
  }
  // one scan of (kept << 16 | equal); both halves stay below 2^16
  const uint32_t packed = (n_kept << 16) | n_eq;
  const uint32_t incl = wave_inclusive_sum(packed);
  if (lane == 63) scratch[wave] = incl;
  wg_sync<true>();  // (LDS only: the prefetched rows stay in flight)
  uint32_t before = incl - packed, total = 0;
#pragma unroll
  for (int w = 0; w < kCWaves; ++w) {
    const uint32_t t = scratch[w];
    before += w < wave ? t : 0u;
    total += t;
  }
  uint32_t eq_seen = before & 0xFFFFu;
  uint32_t p = (before >> 16) + (eq_seen < quota ? eq_seen : quota);
  const int64_t row0 = a.heads.offset[head];
  int32_t* out = a.idx_out + row0;
  // Index stores, and the positions when they follow from the index; looked
  // up positions are written after the copy from the kept keys in LDS. (A
  // load feeding these stores would make each of them wait for every earlier
  // memory operation, the rows prefetched during the resolve among them.)
  const bool lookup = GATHER && a.pos_in != nullptr;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    bool keep = flag[e] == 1u;
    if (flag[e] == 2u) {
      keep = eq_seen < quota;
      ++eq_seen;
    }
    if (keep) {
      const int64_t o = (int64_t)first + p;
      const int32_t j = (int32_t)(j0 + e);
      if (o < h.budget && rep == 0) {
        out[o] = j;
        if (GATHER && !lookup) a.pos_out[row0 + o] = (int32_t)(a.pos_offset + j);
      }
      if (GATHER) kept_keys[p] = j;
      ++p;
    }
  }
  if constexpr (GATHER) {
    const uint32_t eq_all = total & 0xFFFFu;
    int64_t n = (int64_t)(total >> 16) + (eq_all < quota ? eq_all : quota);
    if (n > h.budget - (int64_t)first) n = h.budget - (int64_t)first;  // never past this head's rows
    // (LDS only: the index stores and the prefetched rows stay in flight)
    wg_sync<true>();
    // a row is d/8 16-byte units of K then d/8 of V; consecutive threads take
    // consecutive units, so each row is one contiguous read and write
    const int cpr = a.d >> 3;
    const int units = 2 * cpr;
    const int rpp = kCompactThreads / units;  // rows per pass
    const int u = threadIdx.x % units, r0 = threadIdx.x / units;
    const bool is_k = u < cpr;
    const int cu = is_k ? u : u - cpr;
    const uint16_t* src = (is_k ? a.k + (int64_t)head * a.k_head : a.v + (int64_t)head * a.v_head) + cu * 8;
    const int64_t tok = is_k ? a.k_tok : a.v_tok;
    uint16_t* dst = (is_k ? a.k_out : a.v_out) + (row0 + first) * a.d + cu * 8;
    const int nr = (int)n;
    for (int r = r0 + rep * kCopyUnroll * rpp; r < nr; r += kCopyUnroll * rpp * a.replicas) {
      u32x4 buf[kCopyUnroll];
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) {
        const int rr = r + i * rpp;
        const int key = kept_keys[rr < nr ? rr : r];
        if (rr < nr) buf[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)key * tok);
      }
#pragma unroll
      for (int i = 0; i < kCopyUnroll; ++i) {
        const int rr = r + i * rpp;
        if (rr < nr) __builtin_nontemporal_store(buf[i], reinterpret_cast<u32x4*>(dst + (int64_t)rr * a.d));
      }
    }
    if (lookup && rep == 0)
      for (int r = threadIdx.x; r < nr; r += kCompactThreads)
        a.pos_out[row0 + first + r] = a.pos_in[head * a.pos_in_head + kept_keys[r]];
#pragma unroll
    for (int e = 0; e < 4; ++e)
#pragma unroll
      for (int q = 0; q < 4; ++q) asm volatile("" : : "v"(touched[e][q]));
  }
}

}  // namespace

size_t select_lds_bytes(int n_chunks, int n_subs) {
  (void)n_chunks;
  (void)n_subs;
  return (size_t)kCandCap * 4;
}

template <bool SIGNED>
hipError_t launch_select_keys(const Layer& L, const SelectArgs& a, bool need_hist, hipStream_t st) {
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
    e = hipLaunchKernel(reinterpret_cast<const void*>(&hist_kernel<SIGNED>), chunks, dim3(kThreads), kargs, 0, st);
    if (e != hipSuccess) return e;
  }
  e = hipLaunchKernel(reinterpret_cast<const void*>(&filter_kernel<SIGNED>), chunks, dim3(kThreads), kargs, 0, st);
  if (e != hipSuccess) return e;
  // short rows (few sub-chunks) spread their row copy over more workgroups
  const int subs = L.hkv * a.n_subs;
  const int want = kCompactTarget / subs;
  args.replicas = a.k == nullptr || want < 1 ? 1 : (want > kMaxReplicas ? kMaxReplicas : want);
  const size_t lds = select_lds_bytes(a.n_chunks, a.n_subs);
  const bool spread = a.n_chunks <= kSpreadChunks;
  const void* compact =
      a.k != nullptr ? (spread ? reinterpret_cast<const void*>(&compact_kernel<true, SIGNED, true>)
                               : reinterpret_cast<const void*>(&compact_kernel<true, SIGNED, false>))
                     : (spread ? reinterpret_cast<const void*>(&compact_kernel<false, SIGNED, true>)
                               : reinterpret_cast<const void*>(&compact_kernel<false, SIGNED, false>));
  e = ensure_lds(compact, lds);
  if (e != hipSuccess) return e;
  return hipLaunchKernel(compact, dim3((unsigned)(subs * args.replicas)), dim3(kCompactThreads), kargs, lds, st);
}

hipError_t launch_select(const Layer& L, const SelectArgs& a, bool need_hist, hipStream_t st) {
  return a.signed_keys ? launch_select_keys<true>(L, a, need_hist, st) : launch_select_keys<false>(L, a, need_hist, st);
}

hipError_t launch_hist_clear(const Layer& L, const SelectArgs& a, hipStream_t st) {
  SelectArgs args = a;
  int hkv = L.hkv;
  void* iargs[] = {&args, &hkv};
  return hipLaunchKernel(reinterpret_cast<const void*>(&init_kernel),
                         dim3((unsigned)((L.hkv * kHistBins + 255) / 256)), dim3(256), iargs, 0, st);
}

}  // namespace kvc
