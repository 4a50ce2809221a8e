// Host side of the C ABI: argument validation, workspace layout, launch
// sequencing and error reporting. Nothing here touches device memory; every
// check runs before the first launch of a call.

#include <algorithm>
#include <atomic>
#include <chrono>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <random>
#include <string>
#include <vector>

#include "kvc_internal.h"
#include "prefill_internal.h"

using namespace kvc;

// Workspace of kvc_compress_layer_noalloc: one copy per device, held until the
// process ends. Host code must not pass this name to a kernel or a copy (on
// the host it is a stand-in, not a device address); it uses the address that
// hipGetSymbolAddress returns on each device.
static __device__ __align__(256) unsigned char scratch[KVC_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local std::string g_last_error;

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = std::string(kvc_strerror(status)) + ": " + buf;
  return status;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(KVC_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

constexpr int64_t kInt32Max = 2147483647LL;
constexpr int64_t kMaxPrompt = (int64_t)kMaxSubs * kSub;  // 2^23: sub-chunk tags fit in 13 bits

size_t align_up(size_t x, size_t a) { return (x + a - 1) / a * a; }

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

int device_cus();

// Workgroups the per-head softmax scans aim for across all KV heads: as many
// as the device holds at once (one round; on the 128K-key layer with 256 query
// rows per KV head, one per CU took 206.8 against 220.8 us per layer for two
// per CU in two rounds), or 512 where the device cannot be asked; 512 for the
// raw inner-product scan. Overridable for tuning sweeps (KVC_SCORE_WGS).
int score_wg_target(const Layer& L) {
  static const int env = [] {
    const char* e = std::getenv("KVC_SCORE_WGS");
    const int x = e ? std::atoi(e) : 0;
    return x > 0 ? x : 0;
  }();
  if (env > 0) return env;
  if (L.score_mode != KVC_SCORE_SOFTMAX) return 512;
  const int cus = device_cus();
  const int per = cus > 0 ? per_head_wgs_per_cu(L) : 0;
  return per > 0 ? cus * per : 512;
}

// Workgroups the streaming scans aim for: one per CU of the current device
// (each uses most of the LDS), 256 where the device cannot be asked.
// Overridable for tuning sweeps (KVC_STREAM_WGS).
int stream_wg_target() {
  static const int env = [] {
    const char* e = std::getenv("KVC_STREAM_WGS");
    const int x = e ? std::atoi(e) : 0;
    return x > 0 ? x : 0;
  }();
  if (env > 0) return env;
  const int cus = device_cus();
  return cus > 0 ? cus : 256;
}

// KVC_STREAM=0 selects the per-head scans everywhere (for comparisons).
bool stream_scans_enabled() {
  static const bool v = [] {
    const char* e = std::getenv("KVC_STREAM");
    return !(e && e[0] == '0');
  }();
  return v;
}

// KVC_FUSED=0 keeps the streaming scans as separate launches (pass 1, the
// split combine, pass 2) even where one fused launch would do.
bool fused_scans_enabled() {
  static const bool v = [] {
    const char* e = std::getenv("KVC_FUSED");
    return !(e && e[0] == '0');
  }();
  return v;
}

// Head groups that run on one XCD meet through its L2 after their first
// rendezvous (KVC_XCD_LOCAL=0: always through device-coherent memory).
bool xcd_local_enabled() {
  static const bool v = [] {
    const char* e = std::getenv("KVC_XCD_LOCAL");
    return !(e && e[0] == '0');
  }();
  return v;
}

// Compute units of the current device (0 if it cannot be read), cached per device.
int device_cus() {
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  int n = __atomic_load_n(&cache[dev], __ATOMIC_RELAXED);
  if (n == 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    __atomic_store_n(&cache[dev], n, __ATOMIC_RELAXED);
  }
  return n;
}

// A fresh 64-bit stamp per fused launch: successive values of the SplitMix64
// sequence (Steele, Lea, Flood, "Fast splittable pseudorandom number
// generators", OOPSLA 2014) from a seed drawn once per process, so that no
// flag left in a workspace by an earlier launch, or by other data, matches.
uint64_t next_epoch() {
  static std::atomic<uint64_t> ctr{[] {
    std::random_device rd;
    return ((uint64_t)rd() << 32) ^ rd() ^ (uint64_t)std::chrono::steady_clock::now().time_since_epoch().count();
  }()};
  uint64_t x = ctr.fetch_add(0x9E3779B97F4A7C15ull, std::memory_order_relaxed) + 0x9E3779B97F4A7C15ull;
  x = (x ^ (x >> 30)) * 0xBF58476D1CE4E5B9ull;
  x = (x ^ (x >> 27)) * 0x94D049BB133111EBull;
  return x ^ (x >> 31);
}

// The layer's scans run as one launch (softmax scores, streaming scans,
// every workgroup resident at once).
bool use_fused_scans(const Layer& L) {
  if (L.score_mode != KVC_SCORE_SOFTMAX || L.stream_hg == 0 || !fused_scans_enabled()) return false;
  const int cus = device_cus();
  return cus > 0 && stream_fused_ok(L, std::min(cus, kMaxFusedWgs));
}

int normalize(const kvc_layer_desc* d, Layer& L) {
  if (d == nullptr) return fail(KVC_ERR_INVALID_ARG, "desc is NULL");
  if (d->s < 1) return fail(KVC_ERR_INVALID_ARG, "s=%lld must be >= 1", (long long)d->s);
  if (d->s > kMaxPrompt) return fail(KVC_ERR_UNSUPPORTED, "s=%lld > 2^23", (long long)d->s);
  if (d->w < 1 || d->w > d->s) return fail(KVC_ERR_INVALID_ARG, "w=%d outside [1, s]", d->w);
  if (d->hq < 1 || d->hkv < 1) return fail(KVC_ERR_INVALID_ARG, "hq=%d hkv=%d must be >= 1", d->hq, d->hkv);
  if (d->hkv > KVC_MAX_KV_HEADS) return fail(KVC_ERR_UNSUPPORTED, "hkv=%d > %d", d->hkv, KVC_MAX_KV_HEADS);
  if (d->hq % d->hkv != 0) return fail(KVC_ERR_INVALID_ARG, "hq=%d not a multiple of hkv=%d", d->hq, d->hkv);
  if (d->d < 1) return fail(KVC_ERR_INVALID_ARG, "d=%d must be >= 1", d->d);
  if (d->d != 64 && d->d != 128) return fail(KVC_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d->d);
  if (d->block < 1) return fail(KVC_ERR_INVALID_ARG, "block=%d must be >= 1", d->block);
  if (d->block % kKeyTile != 0 || d->block > 512)
    return fail(KVC_ERR_UNSUPPORTED, "block=%d (supported: multiples of 32 up to 512)", d->block);
  const int64_t g = d->hq / d->hkv;
  if (g * d->w > KVC_MAX_ROWS)
    return fail(KVC_ERR_UNSUPPORTED, "(hq/hkv)*w=%lld > %d query rows per KV head", (long long)(g * d->w), KVC_MAX_ROWS);
  if (std::isnan(d->scale) || std::isinf(d->scale)) return fail(KVC_ERR_INVALID_ARG, "scale is not finite");
  if (d->n_sink < 0 || d->n_recent < 0) return fail(KVC_ERR_INVALID_ARG, "n_sink/n_recent must be >= 0");
  if (d->pool < 1 || d->pool % 2 == 0) return fail(KVC_ERR_INVALID_ARG, "pool=%d must be odd and >= 1", d->pool);
  if (d->pool > KVC_MAX_POOL) return fail(KVC_ERR_UNSUPPORTED, "pool=%d > %d", d->pool, KVC_MAX_POOL);
  if (d->score_mode < KVC_SCORE_SOFTMAX || d->score_mode > KVC_SCORE_LOGIT_INT8)
    return fail(KVC_ERR_INVALID_ARG, "score_mode=%d is not a kvc_score_mode", d->score_mode);
  if (d->score_mode != KVC_SCORE_SOFTMAX && d->s > kMaxPrompt / 2)
    return fail(KVC_ERR_UNSUPPORTED, "s=%lld > 2^22 with signed (raw inner-product) scores", (long long)d->s);
  if (d->pos_offset < 0 || d->pos_offset + d->s > kInt32Max)
    return fail(KVC_ERR_INVALID_ARG, "pos_offset=%lld: positions must fit in int32", (long long)d->pos_offset);
  if ((d->flags & ~KVC_FLAG_FUSED_SELECT) != 0)
    return fail(KVC_ERR_INVALID_ARG, "flags=0x%x has unknown bits", (unsigned)d->flags);
  if (d->reserved != 0) return fail(KVC_ERR_INVALID_ARG, "reserved=%d must be 0", d->reserved);

  const int64_t strides[6] = {d->q_tok_stride, d->q_head_stride, d->k_tok_stride,
                              d->k_head_stride, d->v_tok_stride, d->v_head_stride};
  for (int i = 0; i < 6; ++i) {
    if (strides[i] < 0) return fail(KVC_ERR_INVALID_ARG, "negative stride");
    if (strides[i] % 8 != 0) return fail(KVC_ERR_ALIGN, "stride %lld is not a multiple of 8 elements", (long long)strides[i]);
  }

  L.s = d->s;
  L.w = d->w;
  L.hq = d->hq;
  L.hkv = d->hkv;
  L.d = d->d;
  L.g = (int)g;
  L.block = d->block;
  L.rows = (int)(g * d->w);
  L.row_tiles = (L.rows + kRowTile - 1) / kRowTile;
  L.scale = d->scale > 0.f ? d->scale : (float)(1.0 / std::sqrt((double)d->d));
  L.n_sink = d->n_sink;
  L.n_recent = d->n_recent;
  L.pool = d->pool;
  L.pos_offset = d->pos_offset;
  L.score_mode = d->score_mode;
  L.q_tok = d->q_tok_stride ? d->q_tok_stride : (int64_t)d->hq * d->d;
  L.q_head = d->q_head_stride ? d->q_head_stride : d->d;
  L.k_tok = d->k_tok_stride ? d->k_tok_stride : (int64_t)d->hkv * d->d;
  L.k_head = d->k_head_stride ? d->k_head_stride : d->d;
  L.v_tok = d->v_tok_stride ? d->v_tok_stride : (int64_t)d->hkv * d->d;
  L.v_head = d->v_head_stride ? d->v_head_stride : d->d;

  // Streaming scans for up to four query-row tiles per KV head (six at
  // D = 128); head pairs or one head per workgroup as chosen below, where a
  // slot's copy offsets stay in 32 bits. The selection inside the scan launch
  // takes one head per workgroup.
  L.fsel = (d->flags & KVC_FLAG_FUSED_SELECT) != 0;
  L.stream_hg = 0;
  if (L.fsel) {
    if (L.score_mode != KVC_SCORE_SOFTMAX || L.pool != 1)
      return fail(KVC_ERR_UNSUPPORTED, "KVC_FLAG_FUSED_SELECT needs softmax scores and pool 1");
    const bool wide = L.d == 128 && L.row_tiles <= kStreamMaxRowTiles;
    if ((L.row_tiles > 4 && !wide) || !stream_offsets_fit(L, 1))
      return fail(KVC_ERR_UNSUPPORTED,
                  "KVC_FLAG_FUSED_SELECT needs G*W <= 128 (192 with d=128) and the streaming scans");
    // up to four tiles, the fused kernel's wavefronts split a head's row
    // tiles into row groups of equal size, at most two tiles each: pad to
    // that (padding rows are masked like the ones past G*W in the last
    // tile); five and six take the three-tile loops as they are
    const int rs = stream_row_groups(L.d, 1);
    if (L.row_tiles <= 4) {
      L.row_tiles = (L.row_tiles + rs - 1) / rs * rs;
      if (L.row_tiles / rs > 2)
        return fail(KVC_ERR_UNSUPPORTED, "KVC_FLAG_FUSED_SELECT: %d query rows per KV head > %d with d=%d",
                    L.rows, 64 * rs, L.d);
    }
    L.stream_hg = 1;
  } else if ((L.row_tiles <= 4 || (L.d == 128 && L.row_tiles <= kStreamMaxRowTiles)) && stream_scans_enabled()) {
    // Head pairs (512-byte K segments per token) unless, at D = 128, one head
    // per workgroup measured faster: five or six row tiles, or a short scan
    // (at most 8 slots per workgroup), where the rendezvous inside the fused
    // launch weighs more and a head's workgroups meet within one XCD.
    const int64_t slots1 = (L.s + stream_tokens(L.d, 1) - 1) / stream_tokens(L.d, 1);
    const bool short_scan = slots1 * L.hkv <= 8LL * stream_wg_target();
    const bool prefer_one = L.d == 128 && (L.row_tiles > 4 || short_scan);
    if (L.hkv % 2 == 0 && !prefer_one && stream_offsets_fit(L, 2)) L.stream_hg = 2;
    else if (stream_offsets_fit(L, 1)) L.stream_hg = 1;
  }

  // Partition the key blocks (streaming: stages) of each head (group) over at
  // most kMaxSplit workgroups.
  const int unit = L.stream_hg ? stream_tokens(L.d, L.stream_hg) : L.block;
  const int groups = L.stream_hg ? L.hkv / L.stream_hg : L.hkv;
  const int target = L.stream_hg ? stream_wg_target() : score_wg_target(L);
  L.n_blocks = (int)((L.s + unit - 1) / unit);
  const int64_t min_bpw = (L.n_blocks + kMaxSplit - 1) / kMaxSplit;
  const int64_t want_bpw = ((int64_t)L.n_blocks * groups + target - 1) / target;
  L.blocks_per_wg = (int)std::max<int64_t>(1, std::max(min_bpw, want_bpw));
  L.n_split = (L.n_blocks + L.blocks_per_wg - 1) / L.blocks_per_wg;
  if (L.fsel && (int64_t)L.blocks_per_wg * unit > kFselMaxSegKeys)
    return fail(KVC_ERR_UNSUPPORTED, "KVC_FLAG_FUSED_SELECT: %lld keys per workgroup > %d (s too long for the grid)",
                (long long)L.blocks_per_wg * unit, kFselMaxSegKeys);
  return KVC_OK;
}

// The streaming pass 2 counts its histogram in 16-bit LDS halves: it may
// build the selection histogram only while one workgroup sees fewer than 2^16
// keys of a head (identical scores all land in one bin). Otherwise the
// selection's own histogram kernel (32-bit counters) runs instead.
int64_t stream_keys_per_wg(const Layer& L) {
  return L.stream_hg ? (int64_t)L.blocks_per_wg * stream_tokens(L.d, L.stream_hg) : 0;
}

bool hist_fits_scan(const Layer& L) { return L.stream_hg == 0 || stream_keys_per_wg(L) < 65536; }

int64_t mandatory_count(int64_t s, int n_sink, int n_recent) {
  const int64_t sink_end = std::min<int64_t>(n_sink, s);
  const int64_t rec_begin = std::max<int64_t>(s - n_recent, sink_end);
  return sink_end + (s - rec_begin);
}

int head_table(const Layer& L, const int32_t* budgets, HeadTable& t) {
  if (budgets == nullptr) return fail(KVC_ERR_INVALID_ARG, "budgets is NULL");
  const int64_t n_mand = mandatory_count(L.s, L.n_sink, L.n_recent);
  std::memset(&t, 0, sizeof t);
  int64_t off = 0;
  for (int g = 0; g < L.hkv; ++g) {
    const int64_t b = budgets[g];
    if (b < 0) return fail(KVC_ERR_INVALID_ARG, "budgets[%d]=%lld < 0", g, (long long)b);
    if (b < L.s && b < n_mand)
      return fail(KVC_ERR_INVALID_ARG, "budgets[%d]=%lld below the %lld mandatory keys", g, (long long)b, (long long)n_mand);
    t.budget[g] = (int32_t)b;
    t.offset[g] = off;
    off += std::min<int64_t>(b, L.s);
  }
  t.offset[L.hkv] = off;
  return KVC_OK;
}

int n_chunks(const Layer& L) { return (int)((L.s + kSelectChunk - 1) / kSelectChunk); }
int n_subs(const Layer& L) { return (int)((L.s + kSub - 1) / kSub); }

struct WsLayout {
  size_t sync, part, m, z, scores, pooled;
  size_t hist, slots;
  size_t ghist, segcnt, fslots;  // the selection inside the scan launch
  size_t total;
};

WsLayout ws_layout(const Layer& L) {
  WsLayout w{};
  size_t off = 0;
  const size_t nc = (size_t)n_chunks(L);
  w.sync = off;  // arrival flags of the fused scans (stamped per launch: never cleared)
  off += align_up(kSyncBytes, 256);
  w.hist = off;
  off += align_up((size_t)L.hkv * kHistBins * 4, 256);
  w.part = off;
  off += align_up((size_t)L.hkv * kMaxSplit * L.row_tiles * kRowTile * sizeof(float2), 256);
  w.m = off;
  off += align_up((size_t)L.hq * L.w * sizeof(float), 256);
  w.z = off;
  off += align_up((size_t)L.hq * L.w * sizeof(float), 256);
  if (L.fsel) {
    // scores stay on chip: only the radix round histograms, the segments'
    // counts and lists, none of it growing with s
    w.ghist = off;
    off += align_up((size_t)L.hkv * (kFselR1Bins + kFselR2Bins) * 4, 256);
    w.segcnt = off;
    off += align_up((size_t)L.hkv * kMaxSplit * 2 * 4, 256);
    w.fslots = off;
    off += align_up((size_t)L.hkv * kMaxSplit * kFSlotWords * 4, 256);
    w.slots = w.scores = w.pooled = off;  // (none)
    w.total = off;
    return w;
  }
  w.slots = off;
  off += align_up((size_t)L.hkv * nc * kSlotStride * 4, 256);
  w.scores = off;
  off += align_up((size_t)L.hkv * L.s * sizeof(float), 256);
  w.pooled = off;
  if (L.pool > 1) off += align_up((size_t)L.hkv * L.s * sizeof(float), 256);
  w.total = off;
  return w;
}

// Entry points whose contract involves the s-length score vector or the
// staged selection's bookkeeping reject KVC_FLAG_FUSED_SELECT.
int reject_fsel(const Layer& L, const char* what) {
  if (!L.fsel) return KVC_OK;
  return fail(KVC_ERR_INVALID_ARG, "%s does not take KVC_FLAG_FUSED_SELECT (kvc_compress_layer does)", what);
}

// With KVC_FLAG_FUSED_SELECT a layer runs as one launch whose workgroups must
// all be resident at once: checked before anything is enqueued.
int check_fused_fits(const Layer& L) {
  if (!L.fsel || use_fused_scans(L)) return KVC_OK;
  return fail(KVC_ERR_UNSUPPORTED, "KVC_FLAG_FUSED_SELECT: the %d workgroups of the fused launch do not fit "
              "the device at once", L.hkv * L.n_split);
}

int check_ws(const Layer& L, const void* ws, size_t ws_bytes) {
  const size_t need = ws_layout(L).total;
  if (ws == nullptr) return fail(KVC_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
  if (ws_bytes < need) return fail(KVC_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
  if (!aligned(ws, 256)) return fail(KVC_ERR_ALIGN, "workspace not 256-byte aligned");
  return KVC_OK;
}

int check_ptr(const void* p, size_t align, const char* name) {
  if (p == nullptr) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned(p, align)) return fail(KVC_ERR_ALIGN, "%s is not %zu-byte aligned", name, align);
  return KVC_OK;
}

#define KVC_TRY(x)                 \
  do {                             \
    const int _st = (x);           \
    if (_st != KVC_OK) return _st; \
  } while (0)

// Device LDS limit per workgroup, cached per device.
int check_lds(const Layer& L) {
  static int cache[64] = {0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  int lim = (dev >= 0 && dev < 64) ? __atomic_load_n(&cache[dev], __ATOMIC_RELAXED) : 0;
  if (lim == 0) {
    e = hipDeviceGetAttribute(&lim, hipDeviceAttributeMaxSharedMemoryPerBlock, dev);
    if (e != hipSuccess) return hip_fail(e, "hipDeviceGetAttribute");
    if (dev >= 0 && dev < 64) __atomic_store_n(&cache[dev], lim, __ATOMIC_RELAXED);
  }
  const size_t scan = L.stream_hg ? std::max({pass1_stream_lds_bytes(L), pass2_stream_lds_bytes(L), fused_lds_bytes(L)})
                                  : std::max(pass1_lds_bytes(L), pass2_lds_bytes(L));
  const size_t need = std::max(scan + kFusedStaticLds, select_lds_bytes(n_chunks(L), n_subs(L)) + 16384);
  if (need > (size_t)lim)
    return fail(KVC_ERR_UNSUPPORTED, "kernels need %zu bytes of LDS, device allows %d", need, lim);
  return KVC_OK;
}

ScoreArgs score_args(const Layer& L, const void* q, const void* k) {
  ScoreArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.q_tok = L.q_tok;
  a.q_head = L.q_head;
  a.k_tok = L.k_tok;
  a.k_head = L.k_head;
  a.s = (int)L.s;
  a.w = L.w;
  a.g = L.g;
  a.rows = L.rows;
  a.block = L.block;
  a.n_blocks = L.n_blocks;
  a.blocks_per_wg = L.blocks_per_wg;
  a.n_split = L.n_split;
  a.scale = L.scale;
  a.c = (float)((double)L.scale * 1.4426950408889634);
  const int64_t sink_end = std::min<int64_t>(L.n_sink, L.s);
  a.sink_end = (int)sink_end;
  a.rec_begin = (int)std::max<int64_t>(L.s - L.n_recent, sink_end);
  return a;
}

// with_hist: also clear the selection histogram that pass 2 will fill.
int run_pass1(const Layer& L, const void* q, const void* k, float* m_out, float* z_out,
              void* ws, bool with_hist, hipStream_t st) {
  ScoreArgs a = score_args(L, q, k);
  const WsLayout lay = ws_layout(L);
  char* wsb = static_cast<char*>(ws);
  a.part = reinterpret_cast<float*>(wsb + lay.part);
  if (with_hist) a.hist = reinterpret_cast<uint32_t*>(wsb + lay.hist);
  a.m_out = m_out;
  a.z_out = z_out;
  hipError_t e = L.stream_hg ? launch_stream(true, L, a, st) : launch_pass1(L, a, st);
  if (e != hipSuccess) return hip_fail(e, "pass-1 launch");
  e = launch_combine(L, a, st);
  if (e != hipSuccess) return hip_fail(e, "combine launch");
  return KVC_OK;
}

// ws != nullptr: also build the selection histogram (cleared by pass 1).
int run_pass2(const Layer& L, const void* q, const void* k, const float* m, const float* z,
              float* scores, void* ws, hipStream_t st) {
  ScoreArgs a = score_args(L, q, k);
  if (ws != nullptr) a.hist = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + ws_layout(L).hist);
  a.m_in = m;
  a.z_in = z;
  a.scores = scores;
  const hipError_t e = L.stream_hg ? launch_stream(false, L, a, st) : launch_pass2(L, a, st);
  if (e != hipSuccess) return hip_fail(e, "pass-2 launch");
  return KVC_OK;
}

// Arguments of the selection; k != nullptr: the retained K/V rows are copied
// and their positions written too.
SelectArgs select_args(const Layer& L, const float* scores, const HeadTable& ht, int32_t* idx_out, void* ws,
                       const void* k, const void* v, void* k_out, void* v_out, int32_t* pos_out,
                       const int32_t* pos_in, int64_t pos_in_head) {
  const WsLayout lay = ws_layout(L);
  char* wsb = static_cast<char*>(ws);
  SelectArgs a{};
  a.scores = scores;
  a.pooled = L.pool > 1 ? reinterpret_cast<float*>(wsb + lay.pooled) : nullptr;
  a.vals = L.pool > 1 ? a.pooled : scores;
  a.pool_radius = L.pool / 2;
  a.idx_out = idx_out;
  a.s = L.s;
  a.n_sink = L.n_sink;
  a.n_recent = L.n_recent;
  a.n_chunks = n_chunks(L);
  a.n_subs = n_subs(L);
  a.hist = reinterpret_cast<uint32_t*>(wsb + lay.hist);
  a.slots = reinterpret_cast<uint32_t*>(wsb + lay.slots);
  a.heads = ht;
  a.signed_keys = L.score_mode != KVC_SCORE_SOFTMAX;
  if (k != nullptr) {
    a.k = static_cast<const uint16_t*>(k);
    a.v = static_cast<const uint16_t*>(v);
    a.k_tok = L.k_tok;
    a.k_head = L.k_head;
    a.v_tok = L.v_tok;
    a.v_head = L.v_head;
    a.k_out = static_cast<uint16_t*>(k_out);
    a.v_out = static_cast<uint16_t*>(v_out);
    a.pos_out = pos_out;
    a.pos_offset = L.pos_offset;
    a.pos_in = pos_in;
    a.pos_in_head = pos_in_head;
    a.d = L.d;
  }
  return a;
}

// need_hist: the selection clears and builds its own histogram (and pooled
// values); otherwise pass 1 cleared it and pass 2 built it. k != nullptr: the
// compaction also copies the retained K/V rows and writes their positions.
int run_select(const Layer& L, const float* scores, const HeadTable& ht, int32_t* idx_out,
               void* ws, bool need_hist, hipStream_t st, const void* k = nullptr,
               const void* v = nullptr, void* k_out = nullptr, void* v_out = nullptr,
               int32_t* pos_out = nullptr, const int32_t* pos_in = nullptr, int64_t pos_in_head = 0) {
  const SelectArgs a = select_args(L, scores, ht, idx_out, ws, k, v, k_out, v_out, pos_out, pos_in, pos_in_head);
  const hipError_t e = launch_select(L, a, need_hist || L.pool > 1, st);
  if (e != hipSuccess) return hip_fail(e, "select launch");
  return KVC_OK;
}

// Raw inner-product scores (the non-softmax score modes) into `scores`; with
// hist (cleared beforehand) also the selection histogram.
LogitArgs logit_args(const Layer& L, const void* q, const void* k) {
  LogitArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.q_tok = L.q_tok;
  a.q_head = L.q_head;
  a.k_tok = L.k_tok;
  a.k_head = L.k_head;
  a.s = (int)L.s;
  a.w = L.w;
  a.g = L.g;
  a.hkv = L.hkv;
  const int64_t prefix = L.s - L.w + 1;  // keys seen by every window row
  a.n_split = (int)std::max<int64_t>(1, std::min<int64_t>(stream_wg_target() / L.hkv, (prefix + 255) / 256));
  a.keys_per_wg = (int)((prefix + a.n_split - 1) / a.n_split);
  const int64_t sink_end = std::min<int64_t>(L.n_sink, L.s);
  a.sink_end = (int)sink_end;
  a.rec_begin = (int)std::max<int64_t>(L.s - L.n_recent, sink_end);
  return a;
}

int run_logit(const Layer& L, const void* q, const void* k, float* scores, uint32_t* hist, hipStream_t st) {
  LogitArgs a = logit_args(L, q, k);
  a.scores = scores;
  a.hist = hist;
  const hipError_t e = launch_logit_scan(L, a, L.score_mode == KVC_SCORE_LOGIT_INT8, st);
  if (e != hipSuccess) return hip_fail(e, "raw inner-product scan launch");
  return KVC_OK;
}

int run_gather(const Layer& L, const void* k, const void* v, const int32_t* idx,
               const HeadTable& ht, void* k_out, void* v_out, int32_t* pos_out, hipStream_t st) {
  GatherArgs a{};
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.k_tok = L.k_tok;
  a.k_head = L.k_head;
  a.v_tok = L.v_tok;
  a.v_head = L.v_head;
  a.idx = idx;
  a.k_out = static_cast<uint16_t*>(k_out);
  a.v_out = static_cast<uint16_t*>(v_out);
  a.pos_out = pos_out;
  a.total_rows = ht.offset[L.hkv];
  a.s = L.s;
  a.pos_offset = L.pos_offset;
  a.hkv = L.hkv;
  a.d = L.d;
  a.heads = ht;
  const hipError_t e = launch_gather(a, st);
  if (e != hipSuccess) return hip_fail(e, "gather launch");
  return KVC_OK;
}

// Pointers every whole-layer call needs.
int check_layer_ptrs(const void* q_win, const void* k, const void* v, const int32_t* idx_out,
                     const void* k_out, const void* v_out, const int32_t* pos_out) {
  KVC_TRY(check_ptr(q_win, 16, "q_win"));
  KVC_TRY(check_ptr(k, 16, "k"));
  KVC_TRY(check_ptr(v, 16, "v"));
  KVC_TRY(check_ptr(idx_out, 4, "idx_out"));
  KVC_TRY(check_ptr(k_out, 16, "k_out"));
  KVC_TRY(check_ptr(v_out, 16, "v_out"));
  KVC_TRY(check_ptr(pos_out, 4, "pos_out"));
  return KVC_OK;
}

// The scans of one validated layer onto one stream, exactly as the whole-layer
// call runs them (so they also build the selection histogram where that call
// counts it in the last scan); m, z, scores NULL: in the workspace. Sets
// *hist_built. allow_fused false: three launches even where one would do (for
// callers that overlap layers on several streams: a fused launch needs the
// whole device resident).
int enqueue_scans(const Layer& L, const void* q_win, const void* k, float* m, float* z, float* sc, void* ws,
                  hipStream_t st, bool* hist_built, bool allow_fused = true) {
  const WsLayout lay = ws_layout(L);
  char* wsb = static_cast<char*>(ws);
  // the last scan builds the selection histogram unless ranking uses pooled
  // values or its 16-bit workgroup counters could wrap
  const bool hist_in_pass2 = L.pool == 1 && hist_fits_scan(L);
  *hist_built = hist_in_pass2;
  if (L.score_mode != KVC_SCORE_SOFTMAX) {
    uint32_t* hist = nullptr;
    if (hist_in_pass2) {
      SelectArgs sa{};
      sa.hist = reinterpret_cast<uint32_t*>(wsb + lay.hist);
      const hipError_t e = launch_hist_clear(L, sa, st);
      if (e != hipSuccess) return hip_fail(e, "histogram clear launch");
      hist = sa.hist;
    }
    return run_logit(L, q_win, k, sc, hist, st);
  }
  if (allow_fused && use_fused_scans(L)) {
    ScoreArgs a = score_args(L, q_win, k);
    a.part = reinterpret_cast<float*>(wsb + lay.part);
    if (hist_in_pass2) a.hist = reinterpret_cast<uint32_t*>(wsb + lay.hist);
    a.m_out = m;
    a.z_out = z;
    a.m_in = m;
    a.z_in = z;
    a.scores = sc;
    a.sync = reinterpret_cast<uint64_t*>(wsb + lay.sync);
    a.epoch = next_epoch();
    a.xcd_local = xcd_local_enabled() ? 1 : 0;
    const hipError_t e = launch_stream_fused(L, a, SelectArgs{}, st);
    if (e != hipSuccess) return hip_fail(e, "fused scan launch");
    return KVC_OK;
  }
  KVC_TRY(run_pass1(L, q_win, k, m, z, ws, hist_in_pass2, st));
  return run_pass2(L, q_win, k, m, z, sc, hist_in_pass2 ? ws : nullptr, st);
}

// One validated layer onto one stream; m, z, scores NULL: in the workspace.
// pos_in non-null: retained positions are looked up there (per head, stride
// pos_in_head) instead of pos_offset + index. allow_fused: as enqueue_scans.
int enqueue_layer(const Layer& L, const void* q_win, const void* k, const void* v, const HeadTable& ht,
                  float* m_out, float* z_out, float* scores_out, int32_t* idx_out, void* k_out,
                  void* v_out, int32_t* pos_out, void* ws, hipStream_t st,
                  const int32_t* pos_in = nullptr, int64_t pos_in_head = 0, bool allow_fused = true) {
  const WsLayout lay = ws_layout(L);
  char* wsb = static_cast<char*>(ws);
  float* m = m_out ? m_out : reinterpret_cast<float*>(wsb + lay.m);
  float* z = z_out ? z_out : reinterpret_cast<float*>(wsb + lay.z);
  if (L.fsel) {
    // one launch: both scans, the selection and the gather; the scores stay
    // on chip (written out only when the caller asks for them)
    if (!use_fused_scans(L))
      return fail(KVC_ERR_UNSUPPORTED, "KVC_FLAG_FUSED_SELECT: the %d workgroups of the fused launch do not fit "
                  "the device at once", L.hkv * L.n_split);
    ScoreArgs a = score_args(L, q_win, k);
    a.part = reinterpret_cast<float*>(wsb + lay.part);
    a.hist = reinterpret_cast<uint32_t*>(wsb + lay.hist);
    a.m_out = m;
    a.m_in = m;
    a.z_out = z;
    a.z_in = z;
    a.scores = scores_out;
    a.sync = reinterpret_cast<uint64_t*>(wsb + lay.sync);
    a.epoch = next_epoch();
    a.xcd_local = xcd_local_enabled() ? 1 : 0;
    a.fsel_kpt = (int)((stream_keys_per_wg(L) + kFselThreadsHost - 1) / kFselThreadsHost);
    a.ghist = reinterpret_cast<uint32_t*>(wsb + lay.ghist);
    a.segcnt = reinterpret_cast<uint32_t*>(wsb + lay.segcnt);
    a.fslots = reinterpret_cast<uint32_t*>(wsb + lay.fslots);
    const SelectArgs sa =
        select_args(L, scores_out, ht, idx_out, ws, k, v, k_out, v_out, pos_out, pos_in, pos_in_head);
    const hipError_t e = launch_stream_fused(L, a, sa, st);
    if (e != hipSuccess) return hip_fail(e, "fused scan and selection launch");
    return KVC_OK;
  }
  float* sc = scores_out ? scores_out : reinterpret_cast<float*>(wsb + lay.scores);
  bool hist_built = false;
  KVC_TRY(enqueue_scans(L, q_win, k, m, z, sc, ws, st, &hist_built, allow_fused));
  // the compaction of the selection copies the retained rows as it goes
  return run_select(L, sc, ht, idx_out, ws, !hist_built, st, k, v, k_out, v_out, pos_out, pos_in,
                    pos_in_head);
}

// ---- immediate (chunk-boundary) eviction (TideKV, Fig. 1 caption, schedule
// (c); Table 8, Block-SnapKV). A boundary's accumulated keys -- the retained
// ones, then the new chunk -- live in a head-major arena of `cap` rows per
// head (K, V bf16 [hkv][cap][D], positions int32 [hkv][cap]), so the scans
// and the selection see one ordinary layer of n_kept + c keys.

struct Arena {
  uint16_t* k;
  uint16_t* v;
  int32_t* pos;
};

// The accumulated keys of a boundary as a layer: the chunk's shape and
// options, s_acc keys read from an arena of `cap` rows per head.
int arena_layer(const kvc_layer_desc* chunk, int64_t s_acc, int64_t cap, Layer& La) {
  kvc_layer_desc a = *chunk;
  a.s = s_acc;
  a.pos_offset = 0;
  a.k_tok_stride = a.v_tok_stride = chunk->d;
  a.k_head_stride = a.v_head_stride = cap * chunk->d;
  return normalize(&a, La);
}

// One budget for every head; head g's retained rows start at g * row_stride.
HeadTable arena_table(const Layer& La, int32_t budget, int64_t row_stride) {
  HeadTable t;
  std::memset(&t, 0, sizeof t);
  for (int g = 0; g < La.hkv; ++g) {
    t.budget[g] = budget;
    t.offset[g] = (int64_t)g * row_stride;
  }
  t.offset[La.hkv] = (int64_t)(La.hkv - 1) * row_stride + std::min<int64_t>(budget, La.s);
  return t;
}

// Workspace of one boundary: the layer's, then its retained indices [hkv][cap].
size_t boundary_ws_bytes(const Layer& La, int64_t cap) {
  return ws_layout(La).total + align_up((size_t)La.hkv * cap * 4, 256);
}

int check_boundary(const Layer& La, int32_t budget, int64_t cap) {
  if (budget < La.s && budget < mandatory_count(La.s, La.n_sink, La.n_recent))
    return fail(KVC_ERR_INVALID_ARG, "budget=%d below the %lld mandatory keys of %lld accumulated keys", budget,
                (long long)mandatory_count(La.s, La.n_sink, La.n_recent), (long long)La.s);
  if (cap < La.s) return fail(KVC_ERR_INVALID_ARG, "arena of %lld rows cannot hold %lld keys", (long long)cap, (long long)La.s);
  return KVC_OK;
}

// The append of a chunk (token-major rows of the prompt) to `cur` at row
// n_kept of every head.
AppendArgs append_args(const Layer& Lc, const void* k_chunk, const void* v_chunk, int64_t n_kept, int64_t cap,
                       const Arena& cur) {
  AppendArgs ap{};
  ap.k = static_cast<const uint16_t*>(k_chunk);
  ap.v = static_cast<const uint16_t*>(v_chunk);
  ap.k_tok = Lc.k_tok;
  ap.k_head = Lc.k_head;
  ap.v_tok = Lc.v_tok;
  ap.v_head = Lc.v_head;
  ap.k_arena = cur.k;
  ap.v_arena = cur.v;
  ap.pos_arena = cur.pos;
  ap.cap = cap;
  ap.row0 = n_kept;
  ap.n = Lc.s;
  ap.pos0 = Lc.pos_offset;
  ap.hkv = Lc.hkv;
  ap.d = Lc.d;
  return ap;
}

// With `append`, append the chunk to `cur` at row n_kept (otherwise the
// caller has); with `compress`, score and select the n_kept + c accumulated
// keys and write the retained rows (positions carried from `cur`) to `out`,
// head g at row g * out_stride.
int enqueue_boundary(const Layer& Lc, const kvc_layer_desc* chunk_desc, const void* q_win, const void* k_chunk,
                     const void* v_chunk, int32_t budget, int64_t n_kept, int64_t cap, const Arena& cur,
                     bool append, bool compress, const Arena& out, int64_t out_stride, void* ws, hipStream_t st) {
  if (append) {
    const AppendArgs ap = append_args(Lc, k_chunk, v_chunk, n_kept, cap, cur);
    const hipError_t e = launch_append(&ap, 1, st);
    if (e != hipSuccess) return hip_fail(e, "append launch");
  }
  if (!compress) return KVC_OK;
  Layer La;
  KVC_TRY(arena_layer(chunk_desc, n_kept + Lc.s, cap, La));
  const HeadTable ht = arena_table(La, budget, out_stride);
  int32_t* idx = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + ws_layout(La).total);
  return enqueue_layer(La, q_win, cur.k, cur.v, ht, nullptr, nullptr, nullptr, idx, out.k, out.v, out.pos, ws, st,
                       cur.pos, cap);
}

int check_arena(const Arena& a, const char* which) {
  char name[32];
  std::snprintf(name, sizeof name, "k_%s", which);
  KVC_TRY(check_ptr(a.k, 16, name));
  std::snprintf(name, sizeof name, "v_%s", which);
  KVC_TRY(check_ptr(a.v, 16, name));
  std::snprintf(name, sizeof name, "pos_%s", which);
  return check_ptr(a.pos, 4, name);
}

constexpr int kSweepStreams = 2;  // layers in flight in a sweep with a second stream

// Device address of this device's scratch array, looked up on the first call
// on each device (with that device current) and kept.
int noalloc_scratch(void** out) {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= 64) return fail(KVC_ERR_UNSUPPORTED, "device %d", dev);
  std::lock_guard<std::mutex> lock(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned(p, 256)) return fail(KVC_ERR_HIP, "scratch address %p not usable", p);
    ptrs[dev] = p;
  }
  *out = ptrs[dev];
  return KVC_OK;
}

}  // namespace

namespace kvc {

int record_error(int status, const char* msg) { return fail(status, "%s", msg); }

// Raise a kernel's dynamic LDS limit on the current device (the attribute
// is set per device), once per (device, kernel) and size.
hipError_t ensure_lds(const void* fn, size_t bytes) {
  if (bytes <= 65536) return hipSuccess;
  int dev = 0;
  const hipError_t de = hipGetDevice(&dev);
  if (de != hipSuccess) return de;
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, size_t> done;
  std::lock_guard<std::mutex> lock(mu);
  const std::pair<int, const void*> key(dev, fn);
  auto it = done.find(key);
  if (it != done.end() && it->second >= bytes) return hipSuccess;
  const hipError_t e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
  if (e == hipSuccess) done[key] = bytes;
  return e;
}

}  // namespace kvc

extern "C" {

int kvc_version(void) { return KVC_ABI_VERSION; }

const char* kvc_strerror(int status) {
  switch (status) {
    case KVC_OK: return "KVC_OK";
    case KVC_ERR_INVALID_ARG: return "KVC_ERR_INVALID_ARG";
    case KVC_ERR_UNSUPPORTED: return "KVC_ERR_UNSUPPORTED";
    case KVC_ERR_WORKSPACE: return "KVC_ERR_WORKSPACE";
    case KVC_ERR_ALIGN: return "KVC_ERR_ALIGN";
    case KVC_ERR_HIP: return "KVC_ERR_HIP";
    default: return "KVC_ERR_UNKNOWN";
  }
}

const char* kvc_last_error(void) { return g_last_error.c_str(); }

size_t kvc_workspace_size(const kvc_layer_desc* desc) {
  Layer L;
  if (normalize(desc, L) != KVC_OK) return 0;
  return ws_layout(L).total;
}

int kvc_plan_layer(const kvc_layer_desc* desc, kvc_layer_plan* plan) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  if (plan == nullptr) return fail(KVC_ERR_INVALID_ARG, "plan is NULL");
  kvc_layer_plan p{};
  if (L.score_mode != KVC_SCORE_SOFTMAX) {
    LogitArgs a = logit_args(L, nullptr, nullptr);
    p.scan = KVC_SCAN_LOGIT;
    p.heads_per_wg = 1;
    p.splits = a.n_split;
    p.keys_per_wg = a.keys_per_wg;
    p.hist_in_scan = L.pool == 1;
  } else {
    p.scan = L.stream_hg ? KVC_SCAN_STREAM : KVC_SCAN_PER_HEAD;
    p.heads_per_wg = L.stream_hg ? L.stream_hg : 1;
    p.splits = L.n_split;
    p.keys_per_wg = L.stream_hg ? stream_keys_per_wg(L) : (int64_t)L.blocks_per_wg * L.block;
    p.hist_in_scan = L.pool == 1 && hist_fits_scan(L);
    p.fused_scans = use_fused_scans(L);
    p.fused_select = L.fsel && p.fused_scans;
  }
  p.workspace_bytes = ws_layout(L).total;
  *plan = p;
  return KVC_OK;
}

int kvc_retained_offsets(const kvc_layer_desc* desc, const int32_t* budgets, int64_t* offsets) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  if (offsets == nullptr) return fail(KVC_ERR_INVALID_ARG, "offsets is NULL");
  HeadTable t;
  KVC_TRY(head_table(L, budgets, t));
  for (int g = 0; g <= L.hkv; ++g) offsets[g] = t.offset[g];
  return KVC_OK;
}

int kvc_budgets_inverse_stability(const double* s_stable, int32_t hkv, int64_t total,
                                  int32_t* budgets) {
  if (s_stable == nullptr || budgets == nullptr) return fail(KVC_ERR_INVALID_ARG, "NULL array");
  if (hkv < 1) return fail(KVC_ERR_INVALID_ARG, "hkv=%d must be >= 1", hkv);
  if (total < 0 || total > kInt32Max) return fail(KVC_ERR_INVALID_ARG, "total=%lld outside [0, 2^31-1]", (long long)total);
  std::vector<double> w(hkv), frac(hkv);
  std::vector<int64_t> base(hkv);
  for (int h = 0; h < hkv; ++h) {
    const double x = s_stable[h];
    if (!(x > 0.0) || std::isinf(x)) return fail(KVC_ERR_INVALID_ARG, "s_stable[%d] must be finite and > 0", h);
    w[h] = 1.0 / x;
  }
  double wsum = 0.0;
  for (int h = 0; h < hkv; ++h) wsum += w[h];
  // stabilities so spread (or so small) that the double arithmetic overflows
  // cannot be turned into exact budgets: refuse rather than return a wrong sum
  if (!std::isfinite(wsum))
    return fail(KVC_ERR_INVALID_ARG, "s_stable too small: the inverse weights overflow");
  int64_t used = 0;
  for (int h = 0; h < hkv; ++h) {
    const double exact = (double)total * w[h] / wsum;
    if (!std::isfinite(exact))
      return fail(KVC_ERR_INVALID_ARG, "s_stable[%d] too small for total=%lld: the product overflows", h,
                  (long long)total);
    base[h] = (int64_t)std::floor(exact);
    frac[h] = exact - (double)base[h];
    used += base[h];
  }
  std::vector<int> order(hkv);
  for (int h = 0; h < hkv; ++h) order[h] = h;
  std::stable_sort(order.begin(), order.end(), [&](int a, int b) { return frac[a] > frac[b]; });
  const int64_t rem = total - used;
  if (rem < 0 || rem > hkv)
    return fail(KVC_ERR_INVALID_ARG, "s_stable values too extreme: the budgets would not sum to total=%lld",
                (long long)total);
  for (int64_t r = 0; r < rem && r < hkv; ++r) base[order[r]] += 1;
  for (int h = 0; h < hkv; ++h) budgets[h] = (int32_t)base[h];
  return KVC_OK;
}

int kvc_score_pass1(const kvc_layer_desc* desc, const void* q_win, const void* k, float* m_out,
                    float* z_out, void* ws, size_t ws_bytes, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(reject_fsel(L, "kvc_score_pass1"));
  KVC_TRY(check_ptr(q_win, 16, "q_win"));
  KVC_TRY(check_ptr(k, 16, "k"));
  KVC_TRY(check_ptr(m_out, 4, "m_out"));
  KVC_TRY(check_ptr(z_out, 4, "z_out"));
  KVC_TRY(check_ws(L, ws, ws_bytes));
  if (L.score_mode != KVC_SCORE_SOFTMAX)
    return fail(KVC_ERR_UNSUPPORTED, "score_mode=%d has no softmax normalisers (pass 1)", L.score_mode);
  KVC_TRY(check_lds(L));
  return run_pass1(L, q_win, k, m_out, z_out, ws, false, static_cast<hipStream_t>(stream));
}

int kvc_score_pass2(const kvc_layer_desc* desc, const void* q_win, const void* k, const float* m,
                    const float* z, float* scores, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(reject_fsel(L, "kvc_score_pass2"));
  KVC_TRY(check_ptr(q_win, 16, "q_win"));
  KVC_TRY(check_ptr(k, 16, "k"));
  KVC_TRY(check_ptr(scores, 4, "scores"));
  if (L.score_mode != KVC_SCORE_SOFTMAX)
    return run_logit(L, q_win, k, scores, nullptr, static_cast<hipStream_t>(stream));
  KVC_TRY(check_ptr(m, 4, "m"));
  KVC_TRY(check_ptr(z, 4, "z"));
  KVC_TRY(check_lds(L));
  return run_pass2(L, q_win, k, m, z, scores, nullptr, static_cast<hipStream_t>(stream));
}

int kvc_select_topk(const kvc_layer_desc* desc, const float* scores, const int32_t* budgets,
                    int32_t* idx_out, void* ws, size_t ws_bytes, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(reject_fsel(L, "kvc_select_topk"));
  KVC_TRY(check_ptr(scores, 4, "scores"));
  KVC_TRY(check_ptr(idx_out, 4, "idx_out"));
  HeadTable ht;
  KVC_TRY(head_table(L, budgets, ht));
  KVC_TRY(check_ws(L, ws, ws_bytes));
  KVC_TRY(check_lds(L));
  return run_select(L, scores, ht, idx_out, ws, true, static_cast<hipStream_t>(stream));
}

int kvc_gather_retained(const kvc_layer_desc* desc, const void* k, const void* v,
                        const int32_t* idx, const int32_t* budgets, void* k_out, void* v_out,
                        int32_t* pos_out, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(check_ptr(k, 16, "k"));
  KVC_TRY(check_ptr(v, 16, "v"));
  KVC_TRY(check_ptr(idx, 4, "idx"));
  KVC_TRY(check_ptr(k_out, 16, "k_out"));
  KVC_TRY(check_ptr(v_out, 16, "v_out"));
  KVC_TRY(check_ptr(pos_out, 4, "pos_out"));
  HeadTable ht;
  KVC_TRY(head_table(L, budgets, ht));
  return run_gather(L, k, v, idx, ht, k_out, v_out, pos_out, static_cast<hipStream_t>(stream));
}

int kvc_compress_layer(const kvc_layer_desc* desc, const void* q_win, const void* k, const void* v,
                       const int32_t* budgets, float* m_out, float* z_out, float* scores_out,
                       int32_t* idx_out, void* k_out, void* v_out, int32_t* pos_out, void* ws,
                       size_t ws_bytes, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(check_layer_ptrs(q_win, k, v, idx_out, k_out, v_out, pos_out));
  if (m_out) KVC_TRY(check_ptr(m_out, 4, "m_out"));
  if (z_out) KVC_TRY(check_ptr(z_out, 4, "z_out"));
  if (scores_out) KVC_TRY(check_ptr(scores_out, 4, "scores_out"));
  HeadTable ht;
  KVC_TRY(head_table(L, budgets, ht));
  KVC_TRY(check_ws(L, ws, ws_bytes));
  KVC_TRY(check_lds(L));
  return enqueue_layer(L, q_win, k, v, ht, m_out, z_out, scores_out, idx_out, k_out, v_out, pos_out, ws,
                       static_cast<hipStream_t>(stream));
}

int kvc_score_layer(const kvc_layer_desc* desc, const void* q_win, const void* k, float* m_out, float* z_out,
                    float* scores_out, void* ws, size_t ws_bytes, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(reject_fsel(L, "kvc_score_layer"));
  KVC_TRY(check_ptr(q_win, 16, "q_win"));
  KVC_TRY(check_ptr(k, 16, "k"));
  if (m_out) KVC_TRY(check_ptr(m_out, 4, "m_out"));
  if (z_out) KVC_TRY(check_ptr(z_out, 4, "z_out"));
  if (scores_out) KVC_TRY(check_ptr(scores_out, 4, "scores_out"));
  KVC_TRY(check_ws(L, ws, ws_bytes));
  KVC_TRY(check_lds(L));
  const WsLayout lay = ws_layout(L);
  char* wsb = static_cast<char*>(ws);
  float* m = m_out ? m_out : reinterpret_cast<float*>(wsb + lay.m);
  float* z = z_out ? z_out : reinterpret_cast<float*>(wsb + lay.z);
  float* sc = scores_out ? scores_out : reinterpret_cast<float*>(wsb + lay.scores);
  bool hist_built = false;
  return enqueue_scans(L, q_win, k, m, z, sc, ws, static_cast<hipStream_t>(stream), &hist_built);
}

int kvc_compress_layer_noalloc(const kvc_layer_desc* desc, const void* q_win, const void* k, const void* v,
                               const int32_t* budgets, float* m_out, float* z_out, float* scores_out,
                               int32_t* idx_out, void* k_out, void* v_out, int32_t* pos_out,
                               kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(check_layer_ptrs(q_win, k, v, idx_out, k_out, v_out, pos_out));
  if (m_out) KVC_TRY(check_ptr(m_out, 4, "m_out"));
  if (z_out) KVC_TRY(check_ptr(z_out, 4, "z_out"));
  if (scores_out) KVC_TRY(check_ptr(scores_out, 4, "scores_out"));
  HeadTable ht;
  KVC_TRY(head_table(L, budgets, ht));
  const size_t need = ws_layout(L).total;
  if (need > (size_t)KVC_NOALLOC_SCRATCH_BYTES)
    return fail(KVC_ERR_WORKSPACE, "layer needs %zu bytes of workspace; the fixed scratch holds %zu "
                "(call kvc_compress_layer with a workspace)", need, (size_t)KVC_NOALLOC_SCRATCH_BYTES);
  KVC_TRY(check_lds(L));
  void* ws = nullptr;
  KVC_TRY(noalloc_scratch(&ws));
  return enqueue_layer(L, q_win, k, v, ht, m_out, z_out, scores_out, idx_out, k_out, v_out, pos_out, ws,
                       static_cast<hipStream_t>(stream));
}

int kvc_overlap_coefficient(const kvc_layer_desc* desc, const int32_t* idx_a, const int32_t* idx_b,
                            const int32_t* budgets, float* out, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  KVC_TRY(check_ptr(idx_a, 4, "idx_a"));
  KVC_TRY(check_ptr(idx_b, 4, "idx_b"));
  KVC_TRY(check_ptr(out, 4, "out"));
  HeadTable ht;
  KVC_TRY(head_table(L, budgets, ht));
  OverlapArgs a{};
  a.idx_a = idx_a;
  a.idx_b = idx_b;
  a.out = out;
  a.heads = ht;
  const hipError_t e = launch_overlap(a, L.hkv, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "overlap launch");
  return KVC_OK;
}

int kvc_compress_layers(const kvc_layer_desc* desc, int32_t n_layers, const void* const* q_win,
                        const void* const* k, const void* const* v, const int32_t* budgets,
                        int32_t* const* idx_out, void* const* k_out, void* const* v_out,
                        int32_t* const* pos_out, void* ws, size_t ws_bytes, kvc_stream_t stream,
                        kvc_stream_t aux_stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  if (n_layers < 0) return fail(KVC_ERR_INVALID_ARG, "n_layers=%d < 0", n_layers);
  if (n_layers == 0) return KVC_OK;
  if (!q_win || !k || !v || !budgets || !idx_out || !k_out || !v_out || !pos_out)
    return fail(KVC_ERR_INVALID_ARG, "a per-layer pointer array is NULL");
  // the selection in the scan launch needs the whole device: one lane then
  const int n_lanes = aux_stream != nullptr && aux_stream != stream && !L.fsel ? kSweepStreams : 1;
  const size_t one = ws_layout(L).total;  // a multiple of 256
  if (ws == nullptr) return fail(KVC_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", n_lanes * one);
  if (ws_bytes < n_lanes * one)
    return fail(KVC_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, n_lanes * one);
  if (!aligned(ws, 256)) return fail(KVC_ERR_ALIGN, "workspace not 256-byte aligned");
  std::vector<HeadTable> hts((size_t)n_layers);
  for (int32_t i = 0; i < n_layers; ++i) {
    const int st = check_layer_ptrs(q_win[i], k[i], v[i], idx_out[i], k_out[i], v_out[i], pos_out[i]);
    if (st != KVC_OK) return fail(st, "layer %d: %s", i, g_last_error.c_str());
    const int bt = head_table(L, budgets + (size_t)i * L.hkv, hts[(size_t)i]);
    if (bt != KVC_OK) return fail(bt, "layer %d: %s", i, g_last_error.c_str());
  }
  KVC_TRY(check_lds(L));
  hipStream_t lanes[kSweepStreams] = {static_cast<hipStream_t>(stream), static_cast<hipStream_t>(aux_stream)};
  hipError_t e = hipSuccess;
  if (n_lanes > 1) {
    // fork: the second lane starts after the caller's earlier work
    hipEvent_t ev;
    e = hipEventCreateWithFlags(&ev, hipEventDisableTiming);
    if (e != hipSuccess) return hip_fail(e, "hipEventCreateWithFlags");
    e = hipEventRecord(ev, lanes[0]);
    if (e == hipSuccess) e = hipStreamWaitEvent(lanes[1], ev, 0);
    (void)hipEventDestroy(ev);
    if (e != hipSuccess) return hip_fail(e, "sweep fork");
  }
  // with two lanes the scans stay three launches: a fused scan needs the
  // whole device resident, so two of them must not overlap (and fusing
  // gained nothing there: 77.8-78.8 against 78.3 us per 64K layer)
  int status = KVC_OK;
  for (int32_t i = 0; i < n_layers && status == KVC_OK; ++i) {
    const int j = i % n_lanes;
    status = enqueue_layer(L, q_win[i], k[i], v[i], hts[(size_t)i], nullptr, nullptr, nullptr, idx_out[i],
                           k_out[i], v_out[i], pos_out[i], static_cast<char*>(ws) + j * one, lanes[j], nullptr, 0,
                           n_lanes == 1);
  }
  if (n_lanes > 1) {
    // join: later work on the caller's stream waits for the second lane (also
    // after a failed launch, so that nothing of this call outlives the
    // caller's order)
    hipEvent_t jv;
    e = hipEventCreateWithFlags(&jv, hipEventDisableTiming);
    if (e == hipSuccess) {
      e = hipEventRecord(jv, lanes[1]);
      if (e == hipSuccess) e = hipStreamWaitEvent(lanes[0], jv, 0);
      (void)hipEventDestroy(jv);
    }
    if (e != hipSuccess && status == KVC_OK) status = hip_fail(e, "sweep join");
  }
  return status;
}

size_t kvc_chunk_workspace_size(const kvc_layer_desc* desc, int64_t cap) {
  Layer Lc, La;
  if (normalize(desc, Lc) != KVC_OK || cap < desc->s || cap > kMaxPrompt) return 0;
  if (arena_layer(desc, cap, cap, La) != KVC_OK) return 0;
  return boundary_ws_bytes(La, cap);
}

int kvc_evict_chunk(const kvc_layer_desc* desc, const void* q_win, const void* k_chunk, const void* v_chunk,
                    int32_t budget, int64_t n_kept, int64_t cap, void* k_cur, void* v_cur, int32_t* pos_cur,
                    void* k_next, void* v_next, int32_t* pos_next, void* ws, size_t ws_bytes,
                    kvc_stream_t stream) {
  Layer Lc;
  KVC_TRY(normalize(desc, Lc));
  if (budget < 0) return fail(KVC_ERR_INVALID_ARG, "budget=%d < 0", budget);
  if (n_kept < 0) return fail(KVC_ERR_INVALID_ARG, "n_kept=%lld < 0", (long long)n_kept);
  if (cap < n_kept + Lc.s || cap > kMaxPrompt)
    return fail(KVC_ERR_INVALID_ARG, "cap=%lld outside [n_kept + s, 2^23]", (long long)cap);
  KVC_TRY(check_ptr(q_win, 16, "q_win"));
  KVC_TRY(check_ptr(k_chunk, 16, "k_chunk"));
  KVC_TRY(check_ptr(v_chunk, 16, "v_chunk"));
  const Arena cur{static_cast<uint16_t*>(k_cur), static_cast<uint16_t*>(v_cur), pos_cur};
  KVC_TRY(check_arena(cur, "cur"));
  const bool compress = n_kept + Lc.s > budget;
  const Arena next{static_cast<uint16_t*>(k_next), static_cast<uint16_t*>(v_next), pos_next};
  if (compress) {
    Layer La;
    KVC_TRY(arena_layer(desc, n_kept + Lc.s, cap, La));
    KVC_TRY(check_boundary(La, budget, cap));
    KVC_TRY(check_fused_fits(La));
    KVC_TRY(check_arena(next, "next"));
    if (next.k == cur.k || next.v == cur.v || next.pos == cur.pos)
      return fail(KVC_ERR_INVALID_ARG, "the next arena must not be the current one");
    const size_t need = boundary_ws_bytes(La, cap);
    if (ws == nullptr) return fail(KVC_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", need);
    if (ws_bytes < need) return fail(KVC_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, need);
    if (!aligned(ws, 256)) return fail(KVC_ERR_ALIGN, "workspace not 256-byte aligned");
    KVC_TRY(check_lds(La));
  }
  return enqueue_boundary(Lc, desc, q_win, k_chunk, v_chunk, budget, n_kept, cap, cur, true, compress, next, cap, ws,
                          static_cast<hipStream_t>(stream));
}

namespace {

// Sizes of the whole-prompt immediate-eviction driver.
struct ChunkedPlan {
  int64_t n_chunks, cap, rows;
  size_t arena_k, arena_pos, arena, total;
};

int chunked_plan(const kvc_layer_desc* desc, int64_t chunk, int32_t budget, ChunkedPlan& p) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  if (chunk < L.w) return fail(KVC_ERR_INVALID_ARG, "chunk=%lld shorter than the window w=%d", (long long)chunk, L.w);
  if (budget < 0) return fail(KVC_ERR_INVALID_ARG, "budget=%d < 0", budget);
  p.n_chunks = (L.s + chunk - 1) / chunk;
  const int64_t last = L.s - (p.n_chunks - 1) * chunk;
  if (last < L.w)
    return fail(KVC_ERR_INVALID_ARG, "last chunk of %lld tokens shorter than the window w=%d", (long long)last, L.w);
  p.cap = std::min<int64_t>((int64_t)budget + chunk, L.s);
  p.rows = std::min<int64_t>(budget, L.s);
  p.arena_k = align_up((size_t)L.hkv * p.cap * L.d * 2, 256);
  p.arena_pos = align_up((size_t)L.hkv * p.cap * 4, 256);
  p.arena = 2 * p.arena_k + p.arena_pos;
  Layer La;
  KVC_TRY(arena_layer(desc, p.cap, p.cap, La));
  p.total = 2 * p.arena + boundary_ws_bytes(La, p.cap);
  return KVC_OK;
}

}  // namespace

size_t kvc_chunked_workspace_size(const kvc_layer_desc* desc, int64_t chunk, int32_t budget) {
  ChunkedPlan p;
  if (chunked_plan(desc, chunk, budget, p) != KVC_OK) return 0;
  return p.total;
}

int kvc_compress_chunked(const kvc_layer_desc* desc, int64_t chunk, const void* q_windows, const void* k,
                         const void* v, int32_t budget, void* k_out, void* v_out, int32_t* pos_out, void* ws,
                         size_t ws_bytes, kvc_stream_t stream) {
  Layer L;
  KVC_TRY(normalize(desc, L));
  ChunkedPlan p;
  KVC_TRY(chunked_plan(desc, chunk, budget, p));
  KVC_TRY(check_ptr(q_windows, 16, "q_windows"));
  KVC_TRY(check_ptr(k, 16, "k"));
  KVC_TRY(check_ptr(v, 16, "v"));
  KVC_TRY(check_ptr(k_out, 16, "k_out"));
  KVC_TRY(check_ptr(v_out, 16, "v_out"));
  KVC_TRY(check_ptr(pos_out, 4, "pos_out"));
  if (ws == nullptr) return fail(KVC_ERR_WORKSPACE, "workspace is NULL (need %zu bytes)", p.total);
  if (ws_bytes < p.total) return fail(KVC_ERR_WORKSPACE, "workspace has %zu bytes, need %zu", ws_bytes, p.total);
  if (!aligned(ws, 256)) return fail(KVC_ERR_ALIGN, "workspace not 256-byte aligned");

  // one chunk descriptor per boundary, all validated before the first launch
  std::vector<kvc_layer_desc> cds((size_t)p.n_chunks);
  std::vector<Layer> lcs((size_t)p.n_chunks);
  std::vector<char> squeeze((size_t)p.n_chunks);
  std::vector<Layer> las;
  int64_t n_kept = 0;
  for (int64_t b = 0; b < p.n_chunks; ++b) {
    const int64_t c0 = b * chunk, c = std::min(chunk, L.s - c0);
    kvc_layer_desc& cd = cds[(size_t)b];
    cd = *desc;
    cd.s = c;
    cd.pos_offset = desc->pos_offset + c0;
    cd.q_tok_stride = L.q_tok;
    cd.q_head_stride = L.q_head;
    cd.k_tok_stride = L.k_tok;
    cd.k_head_stride = L.k_head;
    cd.v_tok_stride = L.v_tok;
    cd.v_head_stride = L.v_head;
    KVC_TRY(normalize(&cd, lcs[(size_t)b]));
    const int64_t s_acc = n_kept + c;
    const bool last = b + 1 == p.n_chunks;
    squeeze[(size_t)b] = last || s_acc > budget;
    if (squeeze[(size_t)b]) {
      Layer La;
      KVC_TRY(arena_layer(&cd, s_acc, p.cap, La));
      int st = check_boundary(La, budget, p.cap);
      if (st == KVC_OK) st = check_fused_fits(La);
      if (st != KVC_OK) return fail(st, "chunk %lld: %s", (long long)b, g_last_error.c_str());
      las.push_back(La);
    }
    n_kept = std::min<int64_t>(s_acc, budget);
  }
  for (const Layer& La : las) KVC_TRY(check_lds(La));

  char* wsb = static_cast<char*>(ws);
  Arena arenas[2];
  for (int i = 0; i < 2; ++i) {
    char* base = wsb + i * p.arena;
    arenas[i] = Arena{reinterpret_cast<uint16_t*>(base), reinterpret_cast<uint16_t*>(base + p.arena_k),
                      reinterpret_cast<int32_t*>(base + 2 * p.arena_k)};
  }
  void* bws = wsb + 2 * p.arena;
  const Arena final_out{static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out), pos_out};
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char* qb = static_cast<const char*>(q_windows);
  const char* kb = static_cast<const char*>(k);
  const char* vb = static_cast<const char*>(v);
  // Where each chunk is appended: the arena that holds the keys retained
  // before it, behind them.
  std::vector<int> tgt((size_t)p.n_chunks);
  std::vector<int64_t> row((size_t)p.n_chunks);
  {
    int cur = 0;
    int64_t kept = 0;
    for (int64_t b = 0; b < p.n_chunks; ++b) {
      tgt[(size_t)b] = cur;
      row[(size_t)b] = kept;
      if (squeeze[(size_t)b] && b + 1 < p.n_chunks) cur = 1 - cur;
      kept = std::min<int64_t>(kept + lcs[(size_t)b].s, budget);
    }
  }
  // Chunks 2i and 2i + 1 are appended by one launch before boundary 2i.
  // Chunk 2i + 1's rows are neither read nor written by boundary 2i: when
  // that boundary evicts, it reads the other arena and writes only rows
  // [0, row of chunk 2i + 1) of this one; when it does not, it launches
  // nothing. Every earlier boundary that read those rows precedes the launch.
  for (int64_t b = 0; b < p.n_chunks; ++b) {
    const Layer& Lc = lcs[(size_t)b];
    const int64_t c0 = b * chunk;
    const bool last = b + 1 == p.n_chunks;
    if (b % 2 == 0) {
      AppendArgs jobs[2];
      int n_jobs = 0;
      for (int64_t j = b; j < std::min<int64_t>(b + 2, p.n_chunks); ++j)
        jobs[n_jobs++] = append_args(lcs[(size_t)j], kb + (size_t)(j * chunk * L.k_tok) * 2,
                                     vb + (size_t)(j * chunk * L.v_tok) * 2, row[(size_t)j], p.cap,
                                     arenas[tgt[(size_t)j]]);
      const hipError_t e = launch_append(jobs, n_jobs, st);
      if (e != hipSuccess) return hip_fail(e, "append launch");
    }
    const int cur = tgt[(size_t)b];
    const Arena& out = last ? final_out : arenas[1 - cur];
    KVC_TRY(enqueue_boundary(Lc, &cds[(size_t)b], qb + (size_t)(b * L.w * L.q_tok) * 2, kb + (size_t)(c0 * L.k_tok) * 2,
                             vb + (size_t)(c0 * L.v_tok) * 2, budget, row[(size_t)b], p.cap, arenas[cur], false,
                             squeeze[(size_t)b], out, last ? p.rows : p.cap, bws, st));
  }
  return KVC_OK;
}

}  // extern "C"
