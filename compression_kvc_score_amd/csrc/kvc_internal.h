// Internal types shared by the host API and the gfx950 kernels of libkvc.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc.h"

namespace kvc {

constexpr int kWave = 64;        // CDNA wavefront width
constexpr int kKeyTile = 32;     // keys per wave per block (one 32x32 MFMA tile)
constexpr int kRowTile = 32;     // query rows per MFMA tile
constexpr int kMaxSplit = 128;   // max workgroups per KV head in the scans
constexpr int kMaxRowTiles = KVC_MAX_ROWS / kRowTile;
constexpr int kSelectThreads = 1024;
constexpr int kSelectChunk = 4 * kSelectThreads;  // keys per filter workgroup
constexpr int kCompactThreads = 256;
constexpr int kSub = 4 * kCompactThreads;         // keys per compaction workgroup (a sub-chunk)
constexpr int kSubsPerChunk = kSelectChunk / kSub;
constexpr int kHistBins = 4096;   // top-bits histogram of candidate scores (bits 30..19)
constexpr int kCandCap = 16384;   // listed candidates per head inside the threshold bin
constexpr int kSlotCap = 1024;    // listed candidates per 4096-key chunk
constexpr int kSlotHdr = 16;      // header words of a chunk's slot (counts, b*)
constexpr int kSlotStride = kSlotHdr + kSlotCap;
constexpr int kMaxSubs = 8192;    // sub-chunk tags of listed candidates take 13 bits

// Descriptor after validation, with defaults resolved.
struct Layer {
  int64_t s;
  int w, hq, hkv, d, g, block;
  int rows;        // g * w query rows per KV head, ordered (head-in-group, window index)
  int row_tiles;   // ceil(rows / 32)
  float scale;
  int n_sink, n_recent, pool;
  int64_t pos_offset;
  int64_t q_tok, q_head, k_tok, k_head, v_tok, v_head;
  int n_blocks;       // ceil(s / block), or stages of the streaming scans
  int blocks_per_wg;  // consecutive key blocks (stages) scanned by one workgroup
  int n_split;        // workgroups per KV head (per head group when streaming)
  int stream_hg;      // 0: per-head scans; 1 or 2: streaming scans with this many heads per workgroup
  int score_mode;     // KVC_SCORE_*
  bool fsel;          // KVC_FLAG_FUSED_SELECT: select inside the fused scan launch, scores on chip
};

// Arguments of the two scans and the split combine (passed by value).
struct ScoreArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_tok, q_head, k_tok, k_head;
  int s, w, g, rows;
  int block;        // keys per block (a multiple of 32 * wavefronts per workgroup)
  int n_blocks, blocks_per_wg, n_split;
  float c;          // scale * log2(e): raw dot products to base-2 logits
  float scale;
  float* part;      // [hkv][n_split][row_tiles * 32] x (m_raw, z) split partials
  const float* m_in;  // [hq][w] natural-log row max (pass 2 input)
  const float* z_in;  // [hq][w]
  float* m_out;     // [hq][w]
  float* z_out;     // [hq][w]
  float* scores;    // [hkv][s]
  uint32_t* hist;   // [hkv][kHistBins]: pass 1 clears it, pass 2 fills it (null: skip)
  int sink_end, rec_begin;  // candidate keys [sink_end, rec_begin) for the histogram
  // fused scans only: arrival flags [2][workgroups], stamped with the launch's
  // epoch (a value no earlier launch used), so they need no clearing
  uint64_t* sync;
  uint64_t epoch;
  // selection inside the fused launch (0: none): segment keys per thread;
  // the heads' radix round histograms [hkv][kFselR1Bins + kFselR2Bins] and
  // per-segment counts [hkv][kMaxSplit][2]
  int fsel_kpt;
  uint32_t* ghist;
  uint32_t* segcnt;
  uint32_t* fslots;  // per (head, segment) a list of the candidates inside b*: [hkv][kMaxSplit][kFSlotWords]
  // 1: head groups whose workgroups all run on one XCD may meet through that
  // XCD's L2 after their first (device-coherent) rendezvous
  int xcd_local;
};

// static LDS the scan kernels declare beside their dynamic LDS (a rendezvous
// result word), rounded up
constexpr size_t kFusedStaticLds = 16;
// Query-row tiles of a KV head the streaming scans take with D = 128: past
// four, a wavefront keeps three tiles of queries in registers with one
// accumulator (the Qwen-shaped 160 rows: 99 against 111 us per 64K layer for
// the per-head scans); with four tiles per wavefront (seven or eight row
// tiles) pass 1 spills and the per-head scans are faster.
constexpr int kStreamMaxRowTiles = 6;
constexpr int kMaxFusedWgs = 1024;  // workgroups of one fused scan launch (one per compute unit)
constexpr int kFusedFlagSets = 7;   // partials, normalisers, scores + histogram, lists, two radix rounds, counts
constexpr size_t kSyncBytes = (size_t)kFusedFlagSets * kMaxFusedWgs * sizeof(uint64_t);
constexpr int kFselMaxSegKeys = 4096;  // selection in the fused launch: keys of a segment, at most
constexpr int kFselThreadsHost = 512;  // its threads per workgroup
constexpr int kFselR1Bins = 1024;      // its radix rounds: 10 bits, then 9
constexpr int kFselR2Bins = 512;
constexpr int kFSlotWords = 256;       // a segment's list: 4 header words, then up to 252 entries

// Arguments of the raw inner-product scan (score modes other than softmax).
struct LogitArgs {
  const uint16_t* q;
  const uint16_t* k;
  int64_t q_tok, q_head, k_tok, k_head;
  int s, w, g, hkv;
  int n_split;      // prefix-key workgroups per KV head (plus one for the window keys)
  int keys_per_wg;  // prefix keys per workgroup
  float* scores;    // [hkv][s]
  uint32_t* hist;   // [hkv][kHistBins] signed-key bins (null: skip)
  int sink_end, rec_begin;
};

struct HeadTable {
  int32_t budget[KVC_MAX_KV_HEADS];
  int64_t offset[KVC_MAX_KV_HEADS + 1];  // packed row offsets of the retained outputs
};

struct SelectArgs {
  const float* scores;   // [hkv][s] pass-2 scores
  const float* vals;     // [hkv][s] ranking values (scores, or pooled scores)
  float* pooled;         // pooled values written by the histogram pass (null: no pool)
  int pool_radius;
  int32_t* idx_out;
  int64_t s;
  int n_sink, n_recent;
  int n_chunks;          // ceil(s / kSelectChunk)
  int n_subs;            // ceil(s / kSub)
  uint32_t* hist;        // [hkv][kHistBins]
  uint32_t* slots;       // [hkv][n_chunks][kSlotStride]: per chunk, the candidates inside and
                         // above the threshold bin b* of each sub-chunk, b*, and the list of
                         // those inside b* (sub-chunk << 19 | low 19 pattern bits, key order)
  HeadTable heads;
  bool signed_keys;      // scores may be negative (raw inner-product modes)
  int replicas;          // compaction workgroups per sub-chunk (set by the launcher): each
                         // resolves the sub-chunk and copies its share of the kept rows
  // retained rows copied by the compaction (k == nullptr: indices only)
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_tok, k_head, v_tok, v_head;
  uint16_t* k_out;
  uint16_t* v_out;
  int32_t* pos_out;
  int64_t pos_offset;
  const int32_t* pos_in;  // non-null: position of key j of head g is pos_in[g * pos_in_head + j]
  int64_t pos_in_head;
  int d;
};

struct GatherArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_tok, k_head, v_tok, v_head;
  const int32_t* idx;
  uint16_t* k_out;
  uint16_t* v_out;
  int32_t* pos_out;
  int64_t total_rows;
  int64_t s;
  int64_t pos_offset;
  int hkv, d;
  HeadTable heads;
};

// Raise a kernel's dynamic-LDS limit to at least `bytes` (once per kernel).
hipError_t ensure_lds(const void* fn, size_t bytes);

// Launchers (kernels in the .hip files). Each returns the launch status.
hipError_t launch_pass1(const Layer& L, const ScoreArgs& a, hipStream_t st);
// Workgroups of the per-head scans (the smaller of the two passes) that one
// compute unit of the current device holds at once; 0 if it cannot be read.
int per_head_wgs_per_cu(const Layer& L);
hipError_t launch_combine(const Layer& L, const ScoreArgs& a, hipStream_t st);
hipError_t launch_pass2(const Layer& L, const ScoreArgs& a, hipStream_t st);
// need_hist: clear and build the histogram (and pooled values) first;
// otherwise pass 2 has built it. a.k != nullptr: the compaction also copies
// the retained K/V rows and positions.
hipError_t launch_select(const Layer& L, const SelectArgs& a, bool need_hist, hipStream_t st);
// Clear the selection histograms (before a scan that fills them).
hipError_t launch_hist_clear(const Layer& L, const SelectArgs& a, hipStream_t st);
size_t select_lds_bytes(int n_chunks, int n_subs);
hipError_t launch_gather(const GatherArgs& a, hipStream_t st);

// Append of a prompt chunk to a head-major arena (immediate eviction): chunk
// token t of head g goes to arena row g * cap + row0 + t, with position pos0 + t.
struct AppendArgs {
  const uint16_t* k;
  const uint16_t* v;
  int64_t k_tok, k_head, v_tok, v_head;
  uint16_t* k_arena;
  uint16_t* v_arena;
  int32_t* pos_arena;
  int64_t cap, row0, n;  // arena rows per head, first row written, chunk tokens
  int64_t pos0;
  int hkv, d;
};
struct AppendJobs {
  AppendArgs job[2];
};
// Appends up to two chunks (n_jobs of them; jobs with n == 0 are skipped) in
// one launch; the chunks must not write the same arena rows.
hipError_t launch_append(const AppendArgs* jobs, int n_jobs, hipStream_t st);
struct OverlapArgs {
  const int32_t* idx_a;
  const int32_t* idx_b;
  float* out;
  HeadTable heads;
};
hipError_t launch_overlap(const OverlapArgs& a, int hkv, hipStream_t st);

// Raw inner-product scores (int8: their INT8 form) of all keys; with a.hist
// also the signed-key histogram of the candidates (cleared beforehand).
hipError_t launch_logit_scan(const Layer& L, const LogitArgs& a, bool int8, hipStream_t st);

// Wavefronts per scan workgroup: the largest count up to 8 that divides the
// block's 32-key tiles, so that every wavefront visits the same number of
// tiles per block and together they cover all of them (a block of 11 tiles
// runs on one wavefront, 12 on six, 16 on eight).
constexpr int kMaxScanWaves = 8;
inline int scan_waves(const Layer& L) {
  const int t = L.block / kKeyTile;
  for (int w = t < kMaxScanWaves ? t : kMaxScanWaves; w > 1; --w)
    if (t % w == 0) return w;
  return 1;
}

// Streaming scans (G*W <= 128, or 192 at D = 128): head-group workgroups
// with K staged in LDS.
int stream_tokens(int d, int hg);                  // tokens per ring slot of the streaming scans
int stream_row_groups(int d, int hg);              // row groups sharing a key tile (RS)
bool stream_offsets_fit(const Layer& L, int hg);  // a slot's copy offsets fit in 32 bits
size_t pass1_stream_lds_bytes(const Layer& L);
size_t pass2_stream_lds_bytes(const Layer& L);
hipError_t launch_stream(bool pass1, const Layer& L, const ScoreArgs& a, hipStream_t st);
// Both streaming scans and the split combine in one launch (a.sync, a.epoch
// set): true when the layer's shape has a fused kernel and its workgroups
// can all be resident at once on a device of `cus` compute units.
bool stream_fused_ok(const Layer& L, int cus);
// sel: the selection's arguments when a.fsel_kpt != 0 (else unused).
hipError_t launch_stream_fused(const Layer& L, const ScoreArgs& a, const SelectArgs& sel, hipStream_t st);
// Dynamic LDS of the fused launch (with the segment's scores when the layer selects in it).
size_t fused_lds_bytes(const Layer& L);

// Dynamic LDS bytes of the scans.
size_t pass1_lds_bytes(const Layer& L);
size_t pass2_lds_bytes(const Layer& L);

}  // namespace kvc
