// Internal types of the synthetic layer-major prefill kernels (the layer
// pieces around the compressor: RMSNorm, rotary embedding with the K/V
// append, chunk attention, SwiGLU).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kvc_prefill.h"

namespace kvc {

struct NormArgs {
  const uint16_t* x;
  const uint16_t* w;
  uint16_t* y;
  int64_t rows;
  int dim;
  float eps;
};

struct RopeArgs {
  const uint16_t* qkv;   // [n][(hq + 2 hkv) d]
  uint16_t* q;           // [n][hq][d]
  uint16_t* k;           // cache [s][hkv][d]
  uint16_t* v;
  int64_t c0, n;
  int hq, hkv, d;
  double log2_base;      // log2 of the rotary base
};

struct AttnArgs {
  const uint16_t* q;     // [n][hq][d]
  const uint16_t* k;     // cache [s][hkv][d]
  const uint16_t* v;
  uint16_t* o;           // [n][hq][d]
  int64_t c0, n;
  int hq, hkv, g;
  float c;               // scale * log2(e)
};

struct SwigluArgs {
  const uint16_t* gu;    // [rows][2 ffn]
  uint16_t* a;           // [rows][ffn]
  int64_t rows;
  int ffn;
};

// Record a failed call's message for kvc_last_error (defined with the other
// entry points) and return `status`.
int record_error(int status, const char* msg);

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t st);
hipError_t launch_rope_append(const RopeArgs& a, hipStream_t st);
hipError_t launch_chunk_attention(const AttnArgs& a, int d, hipStream_t st);
hipError_t launch_swiglu(const SwigluArgs& a, hipStream_t st);

}  // namespace kvc
