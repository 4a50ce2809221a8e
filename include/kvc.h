/*
 * kvc.h -- C ABI of the layer-end KV-eviction compressor for AMD MI355X (gfx950).
 *
 * One call compresses one Transformer layer's full-prompt KV cache into a
 * retained cache, as TideKV does at each layer boundary (TideKV, Fig. 2
 * caption: layer-major delayed eviction; Fig. 3 caption: memory-controlled
 * two-pass blockwise scoring). With grouped-query attention (G = hq / hkv
 * query heads per KV head, query head h reads KV head h / G):
 *
 *   pass 1  the last W prompt queries (positions S-W .. S-1, causal) scan the
 *           S prefix keys block by block and build per-query log-sum-exp
 *           normalisers (m, Z): m = max_j l_j, Z = sum_j exp(l_j - m), with
 *           logits l_j = scale * <q, k_j> (natural-log units);
 *   pass 2  a second scan forms the normalised weights exp(l_j - m) / Z and
 *           sums them over the W window queries and the G query heads of each
 *           KV head into one score per (KV head, key);
 *   select  per KV head, the mandatory keys -- the first n_sink and the last
 *           n_recent -- plus the K_h - |mandatory| best other keys by
 *           (score descending, index ascending), listed in ascending order;
 *           an optional centred max-pool of odd width over the scores is
 *           applied before ranking;
 *   gather  the retained K and V rows, copied bit for bit, and their absolute
 *           positions pos_offset + index.
 *
 * Per-head budgets K_h may differ (HeteroCache summary, Methodology, Phase 2:
 * budgets weighted by inverse head stability); kvc_budgets_inverse_stability
 * computes them.
 *
 * Conventions shared by every entry point
 *  - Tensors are bf16 (passed as pointers to 16-bit patterns) or fp32/int32.
 *    Default layouts: Q_win [W][hq][D], K and V [S][hkv][D]; D is contiguous
 *    and other strides are given in elements in kvc_layer_desc.
 *  - Device pointers must point to memory on the current HIP device; all work
 *    is enqueued asynchronously on `stream` (a hipStream_t, 0 = null stream).
 *    No entry point synchronises the host or allocates device memory; the
 *    caller owns every buffer, including the workspace `ws`.
 *  - Every argument is validated on the host before anything is enqueued: a
 *    call that fails validation has enqueued nothing and written nothing. A
 *    KVC_ERR_HIP failure of a later launch may leave earlier launches of the
 *    same call enqueued.
 *  - Inputs must be finite. Results are deterministic: the same inputs and
 *    descriptor give bitwise-identical outputs.
 *  - Functions are thread-safe; calls that share output or workspace buffers
 *    must be ordered by the caller (same stream or events).
 *  - Status codes are the kvc_status values; kvc_strerror names them and
 *    kvc_last_error returns a message about the calling thread's last failure.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVC_ABI_VERSION 2
#define KVC_MAX_KV_HEADS 64    /* hkv limit */
#define KVC_MAX_ROWS 256       /* limit on G * W (query rows per KV head) */
#define KVC_MAX_POOL 31        /* largest max-pool width */
#define KVC_NOALLOC_SCRATCH_BYTES (16u << 20) /* scratch of kvc_compress_layer_noalloc per device */

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_ERR_INVALID_ARG = -1,  /* null pointer, bad size, budget below the mandatory set, ... */
  KVC_ERR_UNSUPPORTED = -2,  /* valid but outside what the kernels implement (D, block, G*W) */
  KVC_ERR_WORKSPACE = -3,    /* workspace null or smaller than kvc_workspace_size() */
  KVC_ERR_ALIGN = -4,        /* pointer or stride not 16-byte aligned */
  KVC_ERR_HIP = -5           /* the HIP runtime reported an error (message in kvc_last_error) */
} kvc_status;

/* How keys are scored (kvc_layer_desc.score_mode). */
typedef enum kvc_score_mode {
  /* softmax weights exp(l - m) / Z summed over the window rows (TideKV,
     Fig. 3 caption): two K passes, pass 1 for the normalisers */
  KVC_SCORE_SOFTMAX = 0,
  /* raw inner products <q, k> summed over the rows that see the key, no
     scale, no softmax (HillInfer, Algorithmic Simplification): one K pass;
     scores may be negative */
  KVC_SCORE_LOGIT = 1,
  /* as KVC_SCORE_LOGIT with the pooled query and every key row quantised to
     symmetric per-vector INT8 on the fly and an exact integer dot product
     (HillInfer, Streaming Execution and Asymmetric Precision); the gather
     still copies the original bf16 rows */
  KVC_SCORE_LOGIT_INT8 = 2
} kvc_score_mode;

/* hipStream_t, passed as an opaque pointer so this header needs no HIP headers. */
typedef void* kvc_stream_t;

/*
 * Shape and options of one layer's compression.
 *  s            prompt length = number of keys scored, 1 <= s <= 2^23
 *               (2^22 in the raw inner-product score modes)
 *  w            observation window: the last w prompt queries, 1 <= w <= s
 *  hq, hkv      query and KV heads, hq % hkv == 0, 1 <= hkv <= KVC_MAX_KV_HEADS,
 *               (hq / hkv) * w <= KVC_MAX_ROWS
 *  d            head dimension: 64 or 128
 *  block        key block size b_s of the blockwise scan: a multiple of 32 in
 *               [32, 512]; results do not depend on it beyond fp32 rounding
 *  scale        logit scale; a value <= 0 selects 1 / sqrt(d)
 *  n_sink       mandatory leading keys, >= 0
 *  n_recent     mandatory trailing keys, >= 0
 *  pool         odd max-pool width over scores before selection, 1 = none,
 *               <= KVC_MAX_POOL; the window is truncated at both ends
 *  pos_offset   added to retained key indices to form positions;
 *               0 <= pos_offset and pos_offset + s <= 2^31 - 1
 *  score_mode   a kvc_score_mode; 0 (the default layout of this field) is
 *               the softmax score. In the raw inner-product modes
 *               kvc_score_pass1 is not available (no normalisers exist),
 *               kvc_score_pass2 writes those scores (m and z are ignored and
 *               may be NULL), kvc_select_topk ranks signed scores, and the
 *               whole-layer calls leave m_out and z_out unwritten. For
 *               KVC_SCORE_LOGIT_INT8 the pooled query is the exact sum of the
 *               bf16 window queries rounded once to fp32 (exact when their
 *               magnitudes span less than 2^45). `scale` is not used.
 *  *_tok_stride, *_head_stride
 *               element strides between tokens and between heads of Q_win, K
 *               and V; 0 selects the default dense layout; non-zero strides
 *               must be multiples of 8 elements (16 bytes)
 */
typedef struct kvc_layer_desc {
  int64_t s;
  int32_t w;
  int32_t hq;
  int32_t hkv;
  int32_t d;
  int32_t block;
  float scale;
  int32_t n_sink;
  int32_t n_recent;
  int32_t pool;
  int32_t score_mode;
  int64_t pos_offset;
  int64_t q_tok_stride, q_head_stride;
  int64_t k_tok_stride, k_head_stride;
  int64_t v_tok_stride, v_head_stride;
  int32_t flags;     /* KVC_FLAG_* bits, 0 for none */
  int32_t reserved;  /* 0 */
} kvc_layer_desc;

/*
 * KVC_FLAG_FUSED_SELECT: kvc_compress_layer (and its _noalloc variant and
 * kvc_compress_layers), and every evicting boundary of kvc_evict_chunk and
 * kvc_compress_chunked, run both scans, the selection and the gather as ONE
 * launch in which every workgroup keeps its key segment's scores on chip, so
 * the workspace does not grow with s at all and no fp32 score vector goes to
 * device memory unless scores_out asks for it (TideKV, Fig. 3 caption:
 * scoring temporaries O(W * b_s + K_l), independent of S). The retained
 * indices, rows and positions equal, bit for bit, what kvc_select_topk and
 * kvc_gather_retained make of the same call's scores; a workgroup scans one
 * KV head, so pass 1's partials merge in another order than the unflagged
 * path's when hkv is even and m, Z and the scores then differ from its in the
 * last bits. Needs softmax scores, pool 1, G * W <= 128 (192 with D = 128),
 * at most 4096 keys of a head per workgroup (s up to about 128K with 8 KV
 * heads on a 256-CU device) and a device whose compute units hold the whole
 * launch at once; else KVC_ERR_UNSUPPORTED (the chunk-boundary calls check
 * every boundary before they enqueue anything). The staged entry points
 * reject the flag (KVC_ERR_INVALID_ARG).
 */
#define KVC_FLAG_FUSED_SELECT 1

/* KVC_ABI_VERSION of the built library. */
int kvc_version(void);

/* Static name of a status code ("KVC_OK", ...); never NULL. */
const char* kvc_strerror(int status);

/* Message about the calling thread's most recent failed call ("" if none).
 * The pointer stays valid until the thread's next failing call. */
const char* kvc_last_error(void);

/*
 * Workspace bytes that every entry point below accepts for this descriptor
 * (the largest need, reached by kvc_compress_layer with all optional outputs
 * NULL). Pure host function. Apart from the fp32 score and pooled-score
 * vectors (4 * hkv * s bytes each) and about 1 byte per key and KV head of
 * selection bookkeeping (4104 bytes per 4096 keys), it does not grow with s, following the
 * S-independent temporary bound of TideKV's Fig. 3 caption; with
 * KVC_FLAG_FUSED_SELECT none of it grows with s.
 * Returns 0 if the descriptor is invalid.
 */
size_t kvc_workspace_size(const kvc_layer_desc* desc);

/* Scan designs reported by kvc_plan_layer. */
typedef enum kvc_scan_kind {
  KVC_SCAN_STREAM = 1,    /* head-group workgroups, K streamed through LDS rings (G * W <= 128; 192 at D = 128) */
  KVC_SCAN_PER_HEAD = 2,  /* one KV head per workgroup, K tiles in registers (G * W <= 256) */
  KVC_SCAN_LOGIT = 3      /* the one-pass raw inner-product scan of the non-softmax score modes */
} kvc_scan_kind;

/* How a descriptor is executed, for tuning and tests (kvc_plan_layer). */
typedef struct kvc_layer_plan {
  int32_t scan;            /* a kvc_scan_kind */
  int32_t heads_per_wg;    /* KV heads one scan workgroup covers */
  int32_t splits;          /* scan workgroups per KV head (per head group when streaming) */
  int32_t hist_in_scan;    /* 1: kvc_compress_layer counts the selection histogram inside
                              the last scan; 0: a separate histogram kernel does */
  int32_t fused_scans;     /* 1: kvc_compress_layer runs pass 1, the split merge and
                              pass 2 as one launch on the current device */
  int32_t fused_select;    /* 1: that launch also selects and gathers, scores on chip
                              (KVC_FLAG_FUSED_SELECT) */
  int64_t keys_per_wg;     /* keys of one KV head that one scan workgroup covers (at most) */
  size_t workspace_bytes;  /* kvc_workspace_size(desc) */
} kvc_layer_plan;

/*
 * The execution plan of desc (validated as every entry point does) into
 * *plan. The streaming pass 2 counts its histogram in 16-bit LDS halves, so it
 * builds the selection histogram only while keys_per_wg < 65536. Host
 * function; only fused_scans looks at the current device (its compute-unit
 * count), and reads 0 where there is none.
 */
int kvc_plan_layer(const kvc_layer_desc* desc, kvc_layer_plan* plan);

/*
 * Rows retained per KV head: min(budgets[g], s). Writes the exclusive prefix
 * sums to offsets[0 .. hkv] (host array of hkv + 1 entries), so head g's rows
 * in the packed outputs are [offsets[g], offsets[g + 1]). Validates budgets
 * like kvc_select_topk. Pure host function.
 */
int kvc_retained_offsets(const kvc_layer_desc* desc, const int32_t* budgets, int64_t* offsets);

/*
 * Heterogeneous budgets (HeteroCache summary, Methodology, Phase 2): weight
 * w_g = 1 / s_stable[g]; budgets[g] = floor(total * w_g / sum w) and the
 * remaining total - sum floor slots go one each to the heads with the largest
 * fractional parts, lower head index first among equals. Sums run in head
 * order, in double precision. s_stable: host array of hkv finite values > 0;
 * budgets: host output of hkv entries; 0 <= total <= 2^31 - 1. Pure host.
 * Returns KVC_ERR_INVALID_ARG (writing nothing) when the values are so small
 * or so spread that the double arithmetic overflows and the budgets could
 * not sum to total.
 */
int kvc_budgets_inverse_stability(const double* s_stable, int32_t hkv, int64_t total,
                                  int32_t* budgets);

/*
 * Pass 1 (TideKV, Fig. 3 caption: first scan, stable log-sum-exp normalisers).
 *  q_win  device, bf16 [W][hq][D] (strided)       k  device, bf16 [S][hkv][D]
 *  m_out, z_out  device, fp32 [hq][W]: row max of the scaled logits (natural
 *         units) and sum_j exp(l_j - m) for query head h, window query i
 *  ws     device workspace of ws_bytes >= kvc_workspace_size(desc)
 */
int kvc_score_pass1(const kvc_layer_desc* desc, const void* q_win, const void* k,
                    float* m_out, float* z_out, void* ws, size_t ws_bytes,
                    kvc_stream_t stream);

/*
 * Pass 2 (TideKV, Fig. 3 caption: second scan, normalised weights pooled per
 * key). m, z as written by kvc_score_pass1. scores: device fp32 [hkv][S],
 * scores[g][j] = sum over window queries i and query heads h of group g of
 * exp(l - m[h][i]) / z[h][i] (0 where key j is after query i). Each head's
 * scores sum to W * G up to rounding. Needs no workspace, so it takes none
 * (unlike pass 1, which keeps its split partials there).
 */
int kvc_score_pass2(const kvc_layer_desc* desc, const void* q_win, const void* k,
                    const float* m, const float* z, float* scores,
                    kvc_stream_t stream);

/*
 * Both scans of one layer (TideKV, Fig. 3 caption: pass 1, then pass 2 over
 * the same key blocks) exactly as kvc_compress_layer runs them: m_out, z_out
 * and scores_out as kvc_score_pass1 and kvc_score_pass2 define them, bit for
 * bit. Each may be NULL (it then lives in the workspace). Where
 * kvc_compress_layer fuses the scans (kvc_plan_layer: fused_scans) this is
 * one launch; it also counts the selection histogram into the workspace
 * where the whole-layer call does, so that the launch is the one the
 * whole-layer call makes. ws: device, kvc_workspace_size(desc) bytes, 256-byte
 * aligned, no initialisation needed.
 */
int kvc_score_layer(const kvc_layer_desc* desc, const void* q_win, const void* k, float* m_out,
                    float* z_out, float* scores_out, void* ws, size_t ws_bytes,
                    kvc_stream_t stream);

/*
 * Selection (TideKV, Fig. 3 caption: top K_l - |R_mand| non-mandatory keys
 * plus the mandatory sink/recent set). scores: device fp32 [hkv][S], finite
 * and >= 0 (as pass 2 writes them); if desc->pool > 1 ranking uses the
 * max-pooled scores. budgets: HOST int32 [hkv]; each budgets[g] >= 0 and,
 * when below s, at least the size of the mandatory set
 * [0, n_sink) U [s - n_recent, s). idx_out: device int32, packed head-major
 * at kvc_retained_offsets; each head's indices ascending.
 */
int kvc_select_topk(const kvc_layer_desc* desc, const float* scores, const int32_t* budgets,
                    int32_t* idx_out, void* ws, size_t ws_bytes, kvc_stream_t stream);

/*
 * Gather (TideKV, Fig. 2 caption: retained KV and absolute positions).
 * idx: device int32 packed as kvc_select_topk writes it, entries in [0, s)
 * (the device clamps out-of-range entries into [0, s) so reads stay inside K
 * and V; such rows are not meaningful). budgets: HOST int32 [hkv] as given to
 * the selection. k_out, v_out: device bf16 [rows][D] dense, rows packed as
 * idx; pos_out: device int32 [rows] = pos_offset + idx.
 */
int kvc_gather_retained(const kvc_layer_desc* desc, const void* k, const void* v,
                        const int32_t* idx, const int32_t* budgets,
                        void* k_out, void* v_out, int32_t* pos_out,
                        kvc_stream_t stream);

/*
 * The whole layer: pass 1, pass 2, (pool), select and gather, enqueued in
 * that order on one stream (the gather runs inside the selection's last
 * kernel). m_out, z_out and scores_out may be NULL (they then live in the
 * workspace); idx_out, k_out, v_out and pos_out are required. Results equal
 * those of the four staged calls bit for bit.
 *
 * With softmax scores on the streaming scans (kvc_plan_layer: scan ==
 * KVC_SCAN_STREAM, fused_scans == 1) pass 1, the merge of its split
 * partials and pass 2 run as ONE launch whose workgroups wait for the others
 * of their head group between the phases. That launch is used only when all
 * of its workgroups (one per compute unit) can be resident at once; each wait
 * is bounded (about a second), so the launch always ends, but if other work
 * holds the device's compute units for that long the call's outputs are not
 * valid. Calls that overlap on several streams of one device should not
 * both take this path (kvc_compress_layers, when it overlaps two layers on
 * two streams, keeps its scans as three launches); setting the environment
 * variable KVC_FUSED=0 before the first call keeps the scans as separate
 * launches everywhere. The workspace needs no initialisation: the waits
 * use flags stamped with a value that is new for every launch.
 */
int kvc_compress_layer(const kvc_layer_desc* desc, const void* q_win, const void* k,
                       const void* v, const int32_t* budgets,
                       float* m_out, float* z_out, float* scores_out, int32_t* idx_out,
                       void* k_out, void* v_out, int32_t* pos_out,
                       void* ws, size_t ws_bytes, kvc_stream_t stream);

/*
 * kvc_compress_layer for callers that cannot allocate device memory: code
 * under HIP graph capture, tight serving loops, and harnesses that forbid
 * hipMalloc. Same kernels, outputs and argument rules as kvc_compress_layer,
 * without the ws / ws_bytes arguments: the workspace is a fixed scratch array
 * of KVC_NOALLOC_SCRATCH_BYTES that the library keeps on every device it runs
 * on until the process ends (its address is looked up once per device, on
 * the first call there). Nothing is allocated or freed, by the library or
 * through another library. Returns KVC_ERR_WORKSPACE, enqueueing nothing,
 * when kvc_workspace_size(desc) exceeds the scratch. Every call on a device
 * shares that device's scratch, which keeps the last call's contents (the
 * kernels clear what they count into): calls that may run at the same time on
 * one device -- different streams without an order between them, or
 * different threads -- race and give wrong results, so order them.
 */
int kvc_compress_layer_noalloc(const kvc_layer_desc* desc, const void* q_win, const void* k,
                               const void* v, const int32_t* budgets,
                               float* m_out, float* z_out, float* scores_out, int32_t* idx_out,
                               void* k_out, void* v_out, int32_t* pos_out, kvc_stream_t stream);

/*
 * Overlap coefficient between two retained index sets of one layer shape
 * (HeteroCache summary, Key Contributions item 1, the measure of how much
 * two heads' or two scorers' retained keys agree): per KV head g,
 * out[g] = |A_g & B_g| / min(|A_g|, |B_g|), and 1 when the head retains no
 * key. idx_a, idx_b: device int32 packed as kvc_select_topk writes them for
 * the same HOST budgets [hkv] (so |A_g| = |B_g|), each head's indices
 * ascending. out: device fp32 [hkv]. Needs no workspace.
 */
int kvc_overlap_coefficient(const kvc_layer_desc* desc, const int32_t* idx_a, const int32_t* idx_b,
                            const int32_t* budgets, float* out, kvc_stream_t stream);

/*
 * A layer-major sweep (TideKV, Fig. 2 caption: layers are compressed one
 * after another at their layer boundaries): n_layers layers of the one shape
 * `desc`, layer i compressed exactly as kvc_compress_layer would (same
 * outputs, bit for bit, with m, z and scores kept in the workspace).
 * aux_stream: a second stream of the caller's (not `stream`, default
 * priority), or NULL. With one, layers alternate between the two streams, so
 * that one layer's selection and gather overlap the next layer's scans (the
 * scans then stay three launches: two fused scan launches must not overlap);
 * with NULL every layer runs on `stream`, as kvc_compress_layer would. The
 * call is ordered after earlier work on `stream` (the second stream waits for
 * it through an event), and later work on `stream` is ordered after all of
 * it; the library creates no stream and keeps nothing.
 * q_win, k, v, idx_out, k_out, v_out, pos_out: HOST arrays of n_layers device
 * pointers, each as for kvc_compress_layer; budgets: HOST int32
 * [n_layers][hkv]. ws: at least 2 * kvc_workspace_size(desc) bytes with a
 * second stream (one workspace per stream), kvc_workspace_size(desc) without,
 * 256-byte aligned. n_layers == 0 enqueues nothing.
 */
int kvc_compress_layers(const kvc_layer_desc* desc, int32_t n_layers,
                        const void* const* q_win, const void* const* k, const void* const* v,
                        const int32_t* budgets, int32_t* const* idx_out,
                        void* const* k_out, void* const* v_out, int32_t* const* pos_out,
                        void* ws, size_t ws_bytes, kvc_stream_t stream, kvc_stream_t aux_stream);

/*
 * Immediate (chunk-boundary) eviction, the schedule that TideKV's layer-end
 * eviction is compared with (TideKV, Fig. 1 caption, schedule (c): chunked
 * prefill that evicts after every chunk; Table 8: Block-SnapKV): after each
 * prompt chunk, the same scorer and selection run over the keys a KV head has
 * retained so far followed by the chunk's keys, with the chunk's last w
 * queries as the observation window and one budget for every head. The
 * mandatory keys are the first n_sink and the last n_recent of those
 * accumulated keys; retained keys keep their absolute positions.
 *
 * An arena holds one boundary's accumulated keys, head-major: K and V bf16
 * [hkv][cap][D] (dense), positions int32 [hkv][cap]; rows [0, n) of every head
 * are in use, in ascending position order.
 */

/*
 * Workspace bytes kvc_evict_chunk needs for chunk descriptor `desc` and
 * arenas of `cap` rows per head (enough for every n_kept with
 * n_kept + desc->s <= cap). Pure host function; 0 if the arguments are
 * invalid (cap < desc->s or cap > 2^23).
 */
size_t kvc_chunk_workspace_size(const kvc_layer_desc* desc, int64_t cap);

/*
 * One chunk boundary. desc describes the chunk: s = its c tokens (w <= c),
 * the window, heads, options, pos_offset = absolute position of its first
 * token, and the strides of q_win ([w][hq][D], the chunk's last w queries)
 * and of k_chunk, v_chunk ([c][hkv][D]).
 *  - The chunk is appended to the current arena (k_cur, v_cur, pos_cur) at
 *    rows [n_kept, n_kept + c) of every head, with positions
 *    pos_offset + t; cap >= n_kept + c.
 *  - If n_kept + c <= budget nothing else happens: the current arena now
 *    holds n_kept + c rows, and k_next, v_next, pos_next and ws are not used
 *    (they may be NULL).
 *  - Otherwise the n_kept + c accumulated keys are scored and selected as
 *    kvc_compress_layer does for a layer of that many keys, and the `budget`
 *    retained rows of every head (ascending positions, carried from pos_cur)
 *    are written to rows [0, budget) of the next arena, which has the same
 *    cap and must not overlap the current one. budget must cover the
 *    mandatory keys of the accumulated ones. ws: at least
 *    kvc_chunk_workspace_size(desc, cap) bytes, 256-byte aligned.
 * budget >= 0; every pointer is device memory of the current device.
 */
int kvc_evict_chunk(const kvc_layer_desc* desc, const void* q_win, const void* k_chunk, const void* v_chunk,
                    int32_t budget, int64_t n_kept, int64_t cap, void* k_cur, void* v_cur, int32_t* pos_cur,
                    void* k_next, void* v_next, int32_t* pos_next, void* ws, size_t ws_bytes,
                    kvc_stream_t stream);

/* Workspace bytes of kvc_compress_chunked (two arenas of
 * min(budget + chunk, s) rows per head and one boundary's workspace); 0 if
 * the arguments are invalid. Pure host function. */
size_t kvc_chunked_workspace_size(const kvc_layer_desc* desc, int64_t chunk, int32_t budget);

/*
 * Immediate eviction over a whole resident prompt: desc describes the prompt
 * (s tokens, K and V [s][hkv][D] strided as for kvc_compress_layer,
 * pos_offset = position of token 0); the chunks are [b * chunk,
 * min((b + 1) * chunk, s)), each -- the last included -- at least w tokens.
 * q_windows: the n_chunks windows stacked along the token axis, window b
 * (the last w queries of chunk b) at token rows [b * w, (b + 1) * w) with the
 * q strides of desc. Each boundary runs as kvc_evict_chunk; the last one
 * always selects (keeping everything when budget covers the prompt) and
 * writes the final retained set: k_out, v_out bf16 [hkv][rows][D] and
 * pos_out int32 [hkv][rows], rows = min(budget, s), head-major, ascending
 * positions. ws: kvc_chunked_workspace_size(desc, chunk, budget) bytes,
 * 256-byte aligned.
 */
int kvc_compress_chunked(const kvc_layer_desc* desc, int64_t chunk, const void* q_windows, const void* k,
                         const void* v, int32_t budget, void* k_out, void* v_out, int32_t* pos_out, void* ws,
                         size_t ws_bytes, kvc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
