/*
 * kvc_prefill.h -- C ABI of the layer pieces that drive a synthetic
 * layer-major chunked prefill around the compressor (TideKV, Fig. 2
 * caption: within the active layer, chunk j's queries attend to the
 * accumulated uncompressed K/V of chunks 0..j, the output hidden rows form
 * the bridge to the next layer, and the layer-end compressor of kvc.h turns
 * the full K/V into the retained cache; Fig. 1 caption, schedule (d)).
 *
 * The pages give no layer equations. These calls implement the non-GEMM
 * parts of a Llama-family decoder layer (the GEMMs are plain library
 * matrix products left to the caller): RMSNorm, the rotary embedding with
 * the append of the chunk's K/V to the layer's cache, causal GQA attention
 * of a chunk over the cache, and SwiGLU.
 *
 * Conventions (as in kvc.h): bf16 tensors are passed as pointers to 16-bit
 * patterns, dense row-major in the layouts stated, 16-byte aligned, on the
 * current HIP device; work is enqueued on `stream`; every argument is
 * checked on the host before anything is enqueued; nothing allocates or
 * synchronises. Status codes are kvc_status values.
 */
#ifndef KVC_PREFILL_H
#define KVC_PREFILL_H

#include <stdint.h>

#include "kvc.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Shape of one layer's attention.
 *  s          rows of the layer's K/V cache: the prompt length, 1 <= s <= 2^31 - 1
 *  hq, hkv    query and KV heads, hq % hkv == 0, hq / hkv in {1, 2, 4, 8}
 *  d          head dimension: 64 or 128
 *  rope_base  rotary base (> 0): pair (i, i + d/2) of a head at absolute
 *             position p turns by p * rope_base^(-2i/d) radians
 *  scale      attention logit scale; <= 0 selects 1 / sqrt(d)
 */
typedef struct kvc_prefill_desc {
  int64_t s;
  int32_t hq;
  int32_t hkv;
  int32_t d;
  float rope_base;
  float scale;
} kvc_prefill_desc;

/*
 * RMSNorm of `rows` rows of `dim` values (dim a multiple of 8, <= 65536):
 * y = x / sqrt(mean(x^2) + eps) * w, in fp32, rounded to bf16 (nearest
 * even). x, y: [rows][dim]; w: [dim]. y may alias x. eps >= 0.
 */
int kvc_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int32_t dim, float eps,
                kvc_stream_t stream);

/*
 * Rotary embedding and K/V append for chunk tokens t in [0, n) at absolute
 * positions c0 + t. qkv: [n][(hq + 2 hkv) d], per token the hq query heads,
 * then the hkv key heads, then the hkv value heads (the QKV projection's
 * output). Writes q_out [n][hq][d] (rotated queries) and rows c0 + t of
 * k_cache and v_cache [s][hkv][d] (rotated keys; values copied).
 * Angles in fp64, cos / sin rounded to fp32, rotation in fp32, results
 * rounded to bf16. 0 <= c0, c0 + n <= s.
 */
int kvc_rope_append(const kvc_prefill_desc* desc, const void* qkv, int64_t c0, int64_t n, void* q_out,
                    void* k_cache, void* v_cache, kvc_stream_t stream);

/*
 * Causal attention of chunk queries q [n][hq][d] (positions c0 + t) over
 * cache rows [0, c0 + n) of k_cache, v_cache [s][hkv][d]: query head h reads
 * KV head h / (hq / hkv); query t sees keys at positions <= c0 + t. o_out
 * [n][hq][d] = softmax(scale * q . k) . v, with fp32 logits and sums, the
 * softmax weights rounded to bf16 for the weighted sum of values, the result
 * rounded to bf16. A query's result does not depend on c0 or n beyond its
 * own position, so chunked and one-shot attention agree bit for bit.
 * 0 <= c0, c0 + n <= s.
 */
int kvc_chunk_attention(const kvc_prefill_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                        int64_t c0, int64_t n, void* o_out, kvc_stream_t stream);

/*
 * SwiGLU: a[r][i] = silu(gu[r][i]) * gu[r][ffn + i], silu(x) = x / (1 + e^-x),
 * in fp32, rounded to bf16. gu: [rows][2 ffn] (gate columns, then up
 * columns); a: [rows][ffn]; ffn a multiple of 8.
 */
int kvc_swiglu(const void* gu, void* a, int64_t rows, int32_t ffn, kvc_stream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_PREFILL_H */
