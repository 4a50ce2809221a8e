// Selection and gather inside the fused scan launch, with each workgroup's
// scores kept on chip (TideKV, Fig. 3 caption: per KV head the mandatory sink
// and recent keys plus the top K_h - |R_mand| other keys by (score
// descending, index ascending), in ascending key order, with a scoring
// footprint that does not grow with S; Fig. 2 caption: their K and V rows and
// absolute positions).
//
// A workgroup owns one KV head's key segment (its token range). Pass 2 leaves
// the segment's scores in LDS and adds the segment's top-bit histogram to the
// head's. Then, with a rendezvous of the head's workgroups before each step
// that needs all of them:
//
//  1. b* = the histogram bin holding the head's k-th best candidate (every
//     workgroup reads the head's histogram);
//  2. each workgroup lists, in key order, the LOW pattern bits of its
//     segment's candidates inside b* (tagged with the segment) in the
//     segment's slot, with its count above b*; after the rendezvous every
//     workgroup reads all of the head's slots (the headers and the first
//     entries in one round trip) and radix-selects in LDS the exact pattern T
//     of the k-th best candidate, how many candidates equal to T are taken
//     (the lowest indices), and how many kept candidates the earlier
//     segments hold;
//  3. where a list does not fit its slot (heavy ties), the workgroups instead
//     run two radix rounds over the candidates inside b* (the top 10 LOW
//     bits, then the other 9): each adds its segment's LDS histogram of the
//     round's digit to the head's round histogram in device memory and,
//     after a rendezvous, picks the same digit from it; then each publishes
//     its segment's counts above and equal to T and reads the earlier ones.
//     Exact whatever the ties;
//  4. each workgroup writes its kept indices and positions in ascending order
//     from there (the rows it keeps were requested into the caches while it
//     resolved) and copies the kept K and V rows.
//
// Device memory holds only the histograms, the per-segment lists (bounded
// by the number of segments, not by S) and counts. Every decision a barrier
// depends on is the same for all threads of the workgroup, and the same for
// every workgroup of a head.

#pragma once

#include "select_common.h"

namespace kvc {
namespace {

constexpr int kFselThreads = 8 * kWave;  // the scan workgroup
constexpr int kFselWaves = kFselThreads / kWave;
constexpr int kFselMaxKpt = kFselMaxSegKeys / kFselThreads;  // segment keys per thread
constexpr int kFselCopyUnroll = 4;       // row pieces in flight per thread
constexpr int kFSlotHdr = 4;             // a list's header words: entries, count above b*, -, -
constexpr int kFSlotCap = kFSlotWords - kFSlotHdr;
constexpr int kFselCand = 8192;          // listed entries of a head gathered in LDS
constexpr int kFselSpecPerThread = 16;   // list words per thread read in the first round trip
static_assert(kFselSpecPerThread * kFselThreads == kMaxSplit * 64 && kFselSpecPerThread * kFselThreads == 32 * kFSlotWords,
              "the first round trip covers 64 words of 128 lists, or 32 whole lists");
static_assert(kFselThreads == kFselThreadsHost && kFselMaxKpt * kFselThreads == kFselMaxSegKeys, "host sizes");
static_assert(kFselR1Bins == 1024 && kFselR2Bins == (int)KeyFmt<false>::R2_BINS, "radix round widths");

typedef uint32_t fsel_u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint32_t ld_coh(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A store the head's other workgroups read with ld_coh: device coherent, or
// kept in the XCD's L2 when all of them run on that XCD (`local`).
__device__ __forceinline__ void st_coh(uint32_t* p, uint32_t v, bool local) {
  if (local) __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  else __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// LDS of the selection (inside the scan's ring, idle by then).
struct FselLds {
  uint32_t hist[kFselR1Bins];      // a radix round's histogram (this segment's, or of the lists)
  uint32_t ghist[kFselR1Bins];     // the head's, as read back (or the lists' second round)
  int32_t kept[kFselMaxSegKeys];   // kept keys of the segment, in order
  uint32_t cand[kFselCand];        // the head's listed entries
  uint32_t n_in[kMaxSplit];        // listed entries per segment
  uint32_t off[kMaxSplit];         // their exclusive prefix
  uint32_t scratch[4 * kFselWaves];
  uint32_t pick[2];
  uint32_t bstar;
};

// This segment's histogram of `digit(u)` over its candidates u with
// (u & mask) == prefix into the head's round histogram `g` (nb bins), then
// publish and wait; returns with m.ghist holding the head's bins.
template <int NB, typename Digit, typename Meet>
__device__ __forceinline__ void fsel_round(const uint32_t (&bits)[kFselMaxKpt], const bool (&cand)[kFselMaxKpt],
                                           uint32_t mask, uint32_t prefix, Digit digit, uint32_t* g, FselLds& m,
                                           Meet meet) {
  for (int i = threadIdx.x; i < NB; i += kFselThreads) m.hist[i] = 0u;
  wg_sync<true>();
#pragma unroll
  for (int e = 0; e < kFselMaxKpt; ++e)
    if (cand[e] && (bits[e] & mask) == prefix) atomicAdd(&m.hist[digit(bits[e])], 1u);
  wg_sync<true>();
  for (int i = threadIdx.x; i < NB; i += kFselThreads) {
    const uint32_t c = m.hist[i];
    if (c != 0u) atomicAdd(g + i, c);  // device scope: performed where every XCD sees it
  }
  meet();
  for (int i = threadIdx.x; i < NB; i += kFselThreads) m.ghist[i] = ld_coh(g + i);
  wg_sync<true>();
}

// Steps 1-4 for KV head `head`, segment [seg0, seg1) of split `split`; the
// segment's scores are in LDS at `sc` (key seg0 + i at sc[i]). meet(n):
// publish this workgroup's n-th selection flag and wait for the head's.
template <typename Meet>
__device__ __forceinline__ void scan_select(const ScoreArgs& a, const SelectArgs& sa, int head, int split,
                                            int64_t seg0, int64_t seg1, const float* sc, unsigned char* smem,
                                            bool local, Meet meet) {
  using KF = KeyFmt<false>;
  FselLds& m = *reinterpret_cast<FselLds*>(smem);
  const int t = threadIdx.x;
  const int kpt = a.fsel_kpt;
  const HeadGeom h = head_geom(sa, head);
  const bool ranked = !h.keep_all && h.k_sel > 0;  // the same in every workgroup of the head
  const int64_t k0 = seg0 + (int64_t)t * kpt;

  // this thread's keys: contiguous, kpt of them
  uint32_t bits[kFselMaxKpt];
  bool cand[kFselMaxKpt];
#pragma unroll
  for (int e = 0; e < kFselMaxKpt; ++e) {
    const int64_t j = k0 + e;
    cand[e] = e < kpt && j < seg1 && is_candidate(h, j);
    bits[e] = cand[e] ? KF::key(sc[j - seg0]) : 0u;
  }
  uint32_t* g1 = a.ghist + (int64_t)head * (kFselR1Bins + kFselR2Bins);
  uint32_t* g2 = g1 + kFselR1Bins;
  uint32_t* cnt = a.segcnt + (int64_t)head * kMaxSplit * 2;

  uint32_t thr = 0xFFFFFFFFu, need_eq = 0u, gt_before = 0u, eq_before = 0u;
  uint32_t touched[kFselMaxKpt][4] = {};  // words of prefetched rows (consumed at the end)
  if (ranked) {
    // ---- 1. b*: thread t owns bins 4095-8t .. 4088-8t (descending)
    const uint32_t* hist = a.hist + (int64_t)head * kHistBins;
    uint32_t c[8], loc = 0;
    {
      // bins 4088-8t .. 4095-8t as two 16-byte device-coherent loads
      fsel_u32x4 lo, hi;
      const uint32_t* b0 = hist + kHistBins - 8 - 8 * t;
      asm volatile(
          "global_load_dwordx4 %0, %2, off sc1\n\tglobal_load_dwordx4 %1, %3, off sc1\n\ts_waitcnt vmcnt(0)"
          : "=&v"(lo), "=&v"(hi)
          : "v"(b0), "v"(b0 + 4)
          : "memory");
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        c[q] = hi[3 - q];  // bin 4095-8t-q
        c[4 + q] = lo[3 - q];
      }
    }
#pragma unroll
    for (int q = 0; q < 8; ++q) loc += c[q];
    if (t == 0) m.bstar = 0u;
    uint32_t total;
    uint32_t before = block_exclusive_scan<kFselWaves, true>(loc, m.scratch, total);
    if (before < h.k_sel && h.k_sel <= before + loc) {
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        if (before < h.k_sel && h.k_sel <= before + c[q]) {
          m.bstar = (uint32_t)(kHistBins - 1 - 8 * t - q);
          m.pick[1] = h.k_sel - before;  // rank inside b*
        }
        before += c[q];
      }
    }
    wg_sync<true>();
    // (a histogram that missed keys cannot hold the k-th: b* would stay 0 and
    // the rounds below pick from what is there; pass 2 counts every candidate)
    const uint32_t bstar = m.bstar;
    uint32_t rem = m.pick[1];
    wg_sync<true>();
    // ---- 2. this segment's list of its candidates inside b*
    uint32_t above = 0, nin = 0;
#pragma unroll
    for (int e = 0; e < kFselMaxKpt; ++e) {
      if (cand[e]) {
        const uint32_t bin = bits[e] >> KF::LOW;
        above += bin > bstar;
        nin += bin == bstar;
      }
    }
    uint32_t tot_in;
    uint32_t pos = block_exclusive_scan<kFselWaves, true>(nin, m.scratch, tot_in);
    uint32_t ab[1] = {above};
    block_sums<kFselWaves, 1, true>(ab, m.scratch);
    uint32_t* slot = a.fslots + ((int64_t)head * kMaxSplit + split) * kFSlotWords;
    const uint32_t tag = (uint32_t)split << KF::LOW;
#pragma unroll
    for (int e = 0; e < kFselMaxKpt; ++e) {
      if (cand[e] && (bits[e] >> KF::LOW) == bstar) {
        if (pos < (uint32_t)kFSlotCap) st_coh(slot + kFSlotHdr + pos, tag | (bits[e] & KF::LOW_MASK), local);
        ++pos;
      }
    }
    if (t == 0) {
      st_coh(slot, tot_in, local);
      st_coh(slot + 1, ab[0], local);
    }
    meet(1);
    // every list of the head, the first spw words of each in one round trip
    // (whole lists for up to 32 segments): word i*512 + t of the lists laid
    // end to end is this thread's w[i]
    const int n_split = a.n_split;
    const uint32_t* slots = a.fslots + (int64_t)head * kMaxSplit * kFSlotWords;
    const int lg = n_split <= 32 ? 8 : (n_split <= 64 ? 7 : 6);
    const int spw = 1 << lg;
    uint32_t w[kFselSpecPerThread];
#pragma unroll
    for (int i = 0; i < kFselSpecPerThread; ++i) {
      const int L = i * kFselThreads + t;
      const int sl = L >> lg;
      w[i] = sl < n_split ? ld_coh(slots + (int64_t)sl * kFSlotWords + (L & (spw - 1))) : 0u;
    }
    uint32_t sums[3] = {0u, 0u, 0u};  // above b* in all lists, in the earlier ones; lists that overflow
#pragma unroll
    for (int i = 0; i < kFselSpecPerThread; ++i) {
      const int L = i * kFselThreads + t;
      const int sl = L >> lg, wd = L & (spw - 1);
      if (sl < n_split && wd == 0) {
        m.n_in[sl] = w[i];
        sums[2] += w[i] > (uint32_t)kFSlotCap;
      }
      if (sl < n_split && wd == 1) {
        sums[0] += w[i];
        sums[1] += sl < split ? w[i] : 0u;
      }
    }
    block_sums<kFselWaves, 3, true>(sums, m.scratch);  // (its barrier also publishes n_in)
    uint32_t listed;
    const uint32_t o = block_exclusive_scan<kFselWaves, true>(t < n_split ? m.n_in[t] : 0u, m.scratch, listed);
    if (t < n_split) m.off[t] = o;
    if (sums[2] == 0u && listed <= (uint32_t)kFselCand) {
      wg_sync<true>();
      // gather the entries: the speculative words, then the rest of the long
      // lists (the eight threads of a list read eight entries at a time)
#pragma unroll
      for (int i = 0; i < kFselSpecPerThread; ++i) {
        const int L = i * kFselThreads + t;
        const int sl = L >> lg;
        const int e = (L & (spw - 1)) - kFSlotHdr;
        if (sl < n_split && e >= 0 && (uint32_t)e < m.n_in[sl]) m.cand[m.off[sl] + e] = w[i];
      }
      // (more than 64 lists: the eight threads t/8 of a list read the rest of
      // it eight entries at a time)
#pragma unroll
      for (int g = 0; g < kMaxSplit / (kFselThreads / 8); ++g) {
        const int sl = (t >> 3) + g * (kFselThreads / 8);
        const uint32_t nl = sl < n_split ? m.n_in[sl] : 0u;
        for (uint32_t e0 = (uint32_t)(spw - kFSlotHdr) + (t & 7); e0 < nl; e0 += 64) {
          uint32_t tmp[8];
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t e = e0 + 8 * q;
            tmp[q] = e < nl ? ld_coh(slots + (int64_t)sl * kFSlotWords + kFSlotHdr + e) : 0u;
          }
#pragma unroll
          for (int q = 0; q < 8; ++q) {
            const uint32_t e = e0 + 8 * q;
            if (e < nl) m.cand[m.off[sl] + e] = tmp[q];
          }
        }
      }
      for (int i = t; i < kFselR1Bins; i += kFselThreads) {
        m.hist[i] = 0u;
        m.ghist[i] = 0u;
      }
      // the rows this segment keeps for sure or may keep, into the caches
      // while the threshold is resolved (consumed at the end)
      // (every address first, outside the conditional loads, so that the
      // layout fields are read once rather than inside each branch)
      const uint16_t* kr0 = sa.k + k0 * sa.k_tok + (int64_t)head * sa.k_head;
      const uint16_t* vr0 = sa.v + k0 * sa.v_tok + (int64_t)head * sa.v_head;
      const int64_t ktk = sa.k_tok, vtk = sa.v_tok;
      const bool wide = sa.d > 64;
#pragma unroll
      for (int e = 0; e < kFselMaxKpt; ++e) {
        const int64_t j = k0 + e;
        const bool want = e < kpt && j < seg1 && (!cand[e] || (bits[e] >> KF::LOW) >= bstar);
        if (want) {
          const uint16_t* kr = kr0 + e * ktk;
          const uint16_t* vr = vr0 + e * vtk;
          touched[e][0] = *reinterpret_cast<const uint32_t*>(kr);
          touched[e][1] = *reinterpret_cast<const uint32_t*>(vr);
          if (wide) {
            touched[e][2] = *reinterpret_cast<const uint32_t*>(kr + 64);
            touched[e][3] = *reinterpret_cast<const uint32_t*>(vr + 64);
          }
        }
      }
      wg_sync<true>();
      // radix over the LOW bits: the top 10, then the other 9
      for (uint32_t x = t; x < listed; x += kFselThreads) atomicAdd(&m.hist[(m.cand[x] >> KF::R2) & 1023u], 1u);
      wg_sync<true>();
      if (t < kWave) pick_digit_wave<kFselR1Bins>(m.hist, rem, m.pick);
      wg_sync<true>();
      const uint32_t d1 = m.pick[0];
      rem = m.pick[1];
      for (uint32_t x = t; x < listed; x += kFselThreads) {
        const uint32_t u = m.cand[x];
        if (((u >> KF::R2) & 1023u) == d1) atomicAdd(&m.ghist[u & (KF::R2_BINS - 1u)], 1u);
      }
      wg_sync<true>();
      if (t < kWave) pick_digit_wave<kFselR2Bins>(m.ghist, rem, m.pick);
      wg_sync<true>();
      const uint32_t low = (d1 << KF::R2) | m.pick[0];
      need_eq = m.pick[1];
      thr = (bstar << KF::LOW) | low;
      // listed candidates of the earlier segments
      uint32_t gq[2] = {0u, 0u};
      for (uint32_t x = t; x < listed; x += kFselThreads) {
        const uint32_t u = m.cand[x];
        if ((int)(u >> KF::LOW) < split) {
          gq[0] += (u & KF::LOW_MASK) > low;
          gq[1] += (u & KF::LOW_MASK) == low;
        }
      }
      block_sums<kFselWaves, 2, true>(gq, m.scratch);
      gt_before = sums[1] + gq[0];
      eq_before = gq[1];
    } else {
      // ---- 3. a list overflowed: radix rounds over the device-memory histograms
      wg_sync<true>();
      const uint32_t top = bstar << KF::LOW;
      fsel_round<kFselR1Bins>(bits, cand, ~KF::LOW_MASK, top, [](uint32_t u) { return (u >> KF::R2) & 1023u; },
                              g1, m, [&]() { meet(2); });
      if (t < kWave) pick_digit_wave<kFselR1Bins>(m.ghist, rem, m.pick);
      wg_sync<true>();
      const uint32_t d1 = m.pick[0];
      rem = m.pick[1];
      wg_sync<true>();
      const uint32_t pre2 = top | (d1 << KF::R2);
      fsel_round<kFselR2Bins>(bits, cand, ~(KF::R2_BINS - 1u), pre2,
                              [](uint32_t u) { return u & (KF::R2_BINS - 1u); }, g2, m, [&]() { meet(3); });
      if (t < kWave) pick_digit_wave<kFselR2Bins>(m.ghist, rem, m.pick);
      wg_sync<true>();
      thr = pre2 | m.pick[0];
      need_eq = m.pick[1];
      wg_sync<true>();
      uint32_t q2[2] = {0u, 0u};
#pragma unroll
      for (int e = 0; e < kFselMaxKpt; ++e) {
        q2[0] += cand[e] && bits[e] > thr;
        q2[1] += cand[e] && bits[e] == thr;
      }
      block_sums<kFselWaves, 2, true>(q2, m.scratch);
      if (t == 0) {
        st_coh(cnt + 2 * split, q2[0], local);
        st_coh(cnt + 2 * split + 1, q2[1], local);
      }
      meet(4);
      uint32_t b2[2] = {0u, 0u};
      for (int s = t; s < split; s += kFselThreads) {
        b2[0] += ld_coh(cnt + 2 * s);
        b2[1] += ld_coh(cnt + 2 * s + 1);
      }
      block_sums<kFselWaves, 2, true>(b2, m.scratch);
      gt_before = b2[0];
      eq_before = b2[1];
    }
  }

  // ---- 4. kept indices and positions of this segment, then the row copy
  uint32_t first, quota = 0u;
  if (ranked) {
    quota = need_eq > eq_before ? need_eq - eq_before : 0u;
    first = mandatory_in(h, 0, seg0) + gt_before + (need_eq < eq_before ? need_eq : eq_before);
  } else {
    first = h.keep_all ? (uint32_t)seg0 : mandatory_in(h, 0, seg0);
  }
  // 1: kept; 2: equal to T (taken in key order while the quota lasts)
  uint32_t flag[kFselMaxKpt], n_kept = 0, n_eq = 0;
#pragma unroll
  for (int e = 0; e < kFselMaxKpt; ++e) {
    const int64_t j = k0 + e;
    flag[e] = 0u;
    if (e >= kpt || j >= seg1) continue;
    if (h.keep_all || !is_candidate(h, j)) flag[e] = 1u;
    else if (ranked) flag[e] = bits[e] > thr ? 1u : (bits[e] == thr ? 2u : 0u);
    n_kept += flag[e] == 1u;
    n_eq += flag[e] == 2u;
  }
  uint32_t total;
  const uint32_t before = block_exclusive_scan<kFselWaves, true>((n_kept << 16) | n_eq, m.scratch, total);
  uint32_t eq_seen = before & 0xFFFFu;
  uint32_t p = (before >> 16) + (eq_seen < quota ? eq_seen : quota);
  const int64_t row0 = sa.heads.offset[head];
  // Index stores, and the positions when they follow from the index; looked
  // up positions are written after the copy from the kept keys in LDS. (A
  // load feeding these stores would make each of them wait for every earlier
  // memory operation, the rows prefetched above among them.)
  const bool lookup = sa.pos_in != nullptr;
#pragma unroll
  for (int e = 0; e < kFselMaxKpt; ++e) {
    bool keep = flag[e] == 1u;
    if (flag[e] == 2u) {
      keep = eq_seen < quota;
      ++eq_seen;
    }
    if (keep) {
      const int64_t o = (int64_t)first + p;
      const int32_t j = (int32_t)(k0 + e);
      if (o < h.budget) {
        sa.idx_out[row0 + o] = j;
        if (!lookup) sa.pos_out[row0 + o] = (int32_t)(sa.pos_offset + j);
      }
      m.kept[p] = j;
      ++p;
    }
  }
  const uint32_t eq_all = total & 0xFFFFu;
  int64_t n = (int64_t)(total >> 16) + (eq_all < quota ? eq_all : quota);
  if (n > h.budget - (int64_t)first) n = h.budget - (int64_t)first;  // never past this head's rows
  wg_sync<true>();
  // a row is d/8 16-byte pieces of K then d/8 of V; consecutive threads take
  // consecutive pieces, so each row is one contiguous read and write
  typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
  const int cpr = sa.d >> 3;
  const int units = 2 * cpr;
  const int rpp = kFselThreads / units;  // rows per pass
  const int u = t % units, r0 = t / units;
  const bool is_k = u < cpr;
  const int cu = is_k ? u : u - cpr;
  const uint16_t* src = (is_k ? sa.k + (int64_t)head * sa.k_head : sa.v + (int64_t)head * sa.v_head) + cu * 8;
  const int64_t tok = is_k ? sa.k_tok : sa.v_tok;
  uint16_t* dst = (is_k ? sa.k_out : sa.v_out) + (row0 + first) * sa.d + cu * 8;
  for (int64_t rb = r0; rb < n; rb += (int64_t)kFselCopyUnroll * rpp) {
    u32x4 buf[kFselCopyUnroll];
#pragma unroll
    for (int i = 0; i < kFselCopyUnroll; ++i) {
      const int64_t rr = rb + (int64_t)i * rpp;
      if (rr < n) buf[i] = *reinterpret_cast<const u32x4*>(src + (int64_t)m.kept[rr] * tok);
    }
#pragma unroll
    for (int i = 0; i < kFselCopyUnroll; ++i) {
      const int64_t rr = rb + (int64_t)i * rpp;
      if (rr < n) __builtin_nontemporal_store(buf[i], reinterpret_cast<u32x4*>(dst + rr * sa.d));
    }
  }
  if (lookup)
    for (int64_t r = t; r < n; r += kFselThreads)
      sa.pos_out[row0 + first + r] = sa.pos_in[head * sa.pos_in_head + m.kept[r]];
#pragma unroll
  for (int e = 0; e < kFselMaxKpt; ++e)
#pragma unroll
    for (int q = 0; q < 4; ++q) asm volatile("" : : "v"(touched[e][q]));
}

}  // namespace
}  // namespace kvc
