// Host side of the prefill layer pieces' C ABI (kvc_prefill.h): argument
// validation and launches. Every check runs before the first launch.

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>

#include "prefill_internal.h"

using namespace kvc;

namespace {

int fail(int status, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
int fail(int status, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  return record_error(status, buf);
}

int launched(hipError_t e, const char* what) {
  if (e == hipSuccess) return KVC_OK;
  return fail(KVC_ERR_HIP, "%s launch: %s (%d)", what, hipGetErrorString(e), (int)e);
}

int check_ptr(const void* p, const char* name) {
  if (p == nullptr) return fail(KVC_ERR_INVALID_ARG, "%s is NULL", name);
  if (reinterpret_cast<uintptr_t>(p) % 16 != 0) return fail(KVC_ERR_ALIGN, "%s is not 16-byte aligned", name);
  return KVC_OK;
}

#define KVC_TRY(x)                 \
  do {                             \
    const int _st = (x);           \
    if (_st != KVC_OK) return _st; \
  } while (0)

int check_desc(const kvc_prefill_desc* d) {
  if (d == nullptr) return fail(KVC_ERR_INVALID_ARG, "desc is NULL");
  if (d->s < 1 || d->s > 2147483647LL) return fail(KVC_ERR_INVALID_ARG, "s=%lld outside [1, 2^31 - 1]", (long long)d->s);
  if (d->hq < 1 || d->hkv < 1 || d->hq % d->hkv != 0)
    return fail(KVC_ERR_INVALID_ARG, "hq=%d, hkv=%d: need hq a multiple of hkv", d->hq, d->hkv);
  const int g = d->hq / d->hkv;
  if (g != 1 && g != 2 && g != 4 && g != 8) return fail(KVC_ERR_UNSUPPORTED, "hq/hkv=%d (supported: 1, 2, 4, 8)", g);
  if (d->d != 64 && d->d != 128) return fail(KVC_ERR_UNSUPPORTED, "d=%d (supported: 64, 128)", d->d);
  if (!(d->rope_base > 0.f) || std::isinf(d->rope_base)) return fail(KVC_ERR_INVALID_ARG, "rope_base must be finite and > 0");
  if (std::isnan(d->scale) || std::isinf(d->scale)) return fail(KVC_ERR_INVALID_ARG, "scale is not finite");
  return KVC_OK;
}

int check_range(const kvc_prefill_desc* d, int64_t c0, int64_t n) {
  if (c0 < 0 || n < 0 || c0 + n > d->s)
    return fail(KVC_ERR_INVALID_ARG, "rows [%lld, %lld) outside the cache of %lld rows", (long long)c0,
                (long long)(c0 + n), (long long)d->s);
  return KVC_OK;
}

}  // namespace

extern "C" {

int kvc_rmsnorm(const void* x, const void* w, void* y, int64_t rows, int32_t dim, float eps, kvc_stream_t stream) {
  if (rows < 0) return fail(KVC_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  if (rows > 2147483647LL) return fail(KVC_ERR_UNSUPPORTED, "rows=%lld > 2^31 - 1", (long long)rows);
  if (dim < 8 || dim % 8 != 0 || dim > 65536) return fail(KVC_ERR_INVALID_ARG, "dim=%d: need a multiple of 8 in [8, 65536]", dim);
  if (!(eps >= 0.f) || std::isinf(eps)) return fail(KVC_ERR_INVALID_ARG, "eps must be finite and >= 0");
  KVC_TRY(check_ptr(x, "x"));
  KVC_TRY(check_ptr(w, "w"));
  KVC_TRY(check_ptr(y, "y"));
  NormArgs a{static_cast<const uint16_t*>(x), static_cast<const uint16_t*>(w), static_cast<uint16_t*>(y), rows, dim, eps};
  return launched(launch_rmsnorm(a, static_cast<hipStream_t>(stream)), "rmsnorm");
}

int kvc_rope_append(const kvc_prefill_desc* desc, const void* qkv, int64_t c0, int64_t n, void* q_out, void* k_cache,
                    void* v_cache, kvc_stream_t stream) {
  KVC_TRY(check_desc(desc));
  KVC_TRY(check_range(desc, c0, n));
  if (n > 2147483647LL) return fail(KVC_ERR_UNSUPPORTED, "n=%lld > 2^31 - 1", (long long)n);
  KVC_TRY(check_ptr(qkv, "qkv"));
  KVC_TRY(check_ptr(q_out, "q_out"));
  KVC_TRY(check_ptr(k_cache, "k_cache"));
  KVC_TRY(check_ptr(v_cache, "v_cache"));
  RopeArgs a{};
  a.qkv = static_cast<const uint16_t*>(qkv);
  a.q = static_cast<uint16_t*>(q_out);
  a.k = static_cast<uint16_t*>(k_cache);
  a.v = static_cast<uint16_t*>(v_cache);
  a.c0 = c0;
  a.n = n;
  a.hq = desc->hq;
  a.hkv = desc->hkv;
  a.d = desc->d;
  a.log2_base = std::log2((double)desc->rope_base);
  return launched(launch_rope_append(a, static_cast<hipStream_t>(stream)), "rope/append");
}

int kvc_chunk_attention(const kvc_prefill_desc* desc, const void* q, const void* k_cache, const void* v_cache,
                        int64_t c0, int64_t n, void* o_out, kvc_stream_t stream) {
  KVC_TRY(check_desc(desc));
  KVC_TRY(check_range(desc, c0, n));
  if ((n + 31) / 32 > 2147483647LL) return fail(KVC_ERR_UNSUPPORTED, "n=%lld too large", (long long)n);
  KVC_TRY(check_ptr(q, "q"));
  KVC_TRY(check_ptr(k_cache, "k_cache"));
  KVC_TRY(check_ptr(v_cache, "v_cache"));
  KVC_TRY(check_ptr(o_out, "o_out"));
  AttnArgs a{};
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k_cache);
  a.v = static_cast<const uint16_t*>(v_cache);
  a.o = static_cast<uint16_t*>(o_out);
  a.c0 = c0;
  a.n = n;
  a.hq = desc->hq;
  a.hkv = desc->hkv;
  a.g = desc->hq / desc->hkv;
  const double scale = desc->scale > 0.f ? (double)desc->scale : 1.0 / std::sqrt((double)desc->d);
  a.c = (float)(scale * 1.4426950408889634);
  return launched(launch_chunk_attention(a, desc->d, static_cast<hipStream_t>(stream)), "chunk attention");
}

int kvc_swiglu(const void* gu, void* a_out, int64_t rows, int32_t ffn, kvc_stream_t stream) {
  if (rows < 0) return fail(KVC_ERR_INVALID_ARG, "rows=%lld < 0", (long long)rows);
  if (ffn < 8 || ffn % 8 != 0) return fail(KVC_ERR_INVALID_ARG, "ffn=%d: need a multiple of 8", ffn);
  if (rows * (int64_t)(ffn / 8) > (int64_t)256 * 2147483647LL) return fail(KVC_ERR_UNSUPPORTED, "too many rows");
  KVC_TRY(check_ptr(gu, "gu"));
  KVC_TRY(check_ptr(a_out, "a"));
  SwigluArgs a{static_cast<const uint16_t*>(gu), static_cast<uint16_t*>(a_out), rows, ffn};
  return launched(launch_swiglu(a, static_cast<hipStream_t>(stream)), "swiglu");
}

}  // extern "C"
