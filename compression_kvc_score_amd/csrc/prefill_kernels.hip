// Kernels of the synthetic layer-major chunked prefill around the compressor
// (TideKV, Fig. 2 caption: chunk j of the active layer attends to the
// accumulated K/V of chunks 0..j and its output rows form the bridge to the
// next layer). The pages give no layer equations; these implement a
// Llama-family decoder layer's non-GEMM parts:
//   rmsnorm       y = x / sqrt(mean(x^2) + eps) * w            (row per workgroup)
//   rope_append   rotary embedding of q and k at absolute positions, pairs
//                 (i, i + D/2); q to the chunk's query buffer, k and v appended
//                 to the layer's K/V cache at rows c0 + t
//   attention     causal GQA attention of a chunk's queries over cache rows
//                 [0, c0 + n), online softmax, bf16 MFMA
//   swiglu        silu(gate) * up
// Activations are bf16 between kernels; arithmetic is fp32 (fp64 for the
// rotation angles).

#include "prefill_internal.h"

namespace kvc {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ float lo_f32(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float hi_f32(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (finite values)
__device__ __forceinline__ uint32_t bf16_bits(float f) {
  const uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}
__device__ __forceinline__ uint32_t pack2(float lo, float hi) { return bf16_bits(lo) | (bf16_bits(hi) << 16); }

// ---------------------------------------------------------------------------
// RMSNorm: one 256-thread workgroup per row; the sum of squares is reduced in
// a fixed order (lane butterfly, then the four wavefronts in order).
// ---------------------------------------------------------------------------
constexpr int kNormThreads = 256;

__global__ void __launch_bounds__(kNormThreads) rmsnorm_kernel(NormArgs a) {
  __shared__ float part[kNormThreads / 64];
  const int64_t row = blockIdx.x;
  const uint16_t* x = a.x + row * a.dim;
  uint16_t* y = a.y + row * a.dim;
  const int nch = a.dim / 8;
  float ss = 0.f;
  for (int c = threadIdx.x; c < nch; c += kNormThreads) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + c * 8);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      ss = fmaf(lo_f32(w[i]), lo_f32(w[i]), ss);
      ss = fmaf(hi_f32(w[i]), hi_f32(w[i]), ss);
    }
  }
  for (int off = 32; off >= 1; off >>= 1) ss += __shfl_xor(ss, off);
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / 64; ++i) tot += part[i];
  const float r = 1.0f / sqrtf(tot / (float)a.dim + a.eps);
  for (int c = threadIdx.x; c < nch; c += kNormThreads) {
    const uint4 u = *reinterpret_cast<const uint4*>(x + c * 8);
    const uint4 g = *reinterpret_cast<const uint4*>(a.w + c * 8);
    const uint32_t xw[4] = {u.x, u.y, u.z, u.w}, ww[4] = {g.x, g.y, g.z, g.w};
    uint32_t o[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      o[i] = pack2(lo_f32(xw[i]) * r * lo_f32(ww[i]), hi_f32(xw[i]) * r * hi_f32(ww[i]));
    *reinterpret_cast<uint4*>(y + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// ---------------------------------------------------------------------------
// Rotary embedding and K/V append: one workgroup per token. The angles
// p * base^(-2i/D) and their cos / sin are computed in fp64 once per token
// (positions reach 2^17, where an fp32 angle would be off by 2^-6 rad), kept
// in LDS as fp32 and applied to every q and k head; each thread turns four
// pairs (8-byte loads of both halves).
// ---------------------------------------------------------------------------
constexpr int kRopeThreads = 256;
constexpr int kMaxHalf = 256;  // d <= 512

__global__ void __launch_bounds__(kRopeThreads) rope_append_kernel(RopeArgs a) {
  __shared__ float cs[kMaxHalf], sn[kMaxHalf];
  const int64_t t = blockIdx.x;
  const int64_t p = a.c0 + t;
  const int half = a.d / 2;
  for (int i = threadIdx.x; i < half; i += kRopeThreads) {
    const double ang = (double)p * exp2(-(2.0 * i / a.d) * a.log2_base);
    double s, c;
    sincos(ang, &s, &c);
    cs[i] = (float)c;
    sn[i] = (float)s;
  }
  __syncthreads();
  const int width = (a.hq + 2 * a.hkv) * a.d;
  const uint16_t* row = a.qkv + t * width;
  const int quads = half / 4;
  const int nrot = (a.hq + a.hkv) * quads;
  for (int e = threadIdx.x; e < nrot; e += kRopeThreads) {
    const int hh = e / quads, i = (e % quads) * 4;
    const uint2 u0 = *reinterpret_cast<const uint2*>(row + hh * a.d + i);
    const uint2 u1 = *reinterpret_cast<const uint2*>(row + hh * a.d + half + i);
    const float x0[4] = {lo_f32(u0.x), hi_f32(u0.x), lo_f32(u0.y), hi_f32(u0.y)};
    const float x1[4] = {lo_f32(u1.x), hi_f32(u1.x), lo_f32(u1.y), hi_f32(u1.y)};
    float y0[4], y1[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      y0[j] = x0[j] * cs[i + j] - x1[j] * sn[i + j];
      y1[j] = x1[j] * cs[i + j] + x0[j] * sn[i + j];
    }
    uint16_t* dst = hh < a.hq ? a.q + (t * a.hq + hh) * a.d
                              : a.k + ((a.c0 + t) * a.hkv + (hh - a.hq)) * a.d;
    *reinterpret_cast<uint2*>(dst + i) = make_uint2(pack2(y0[0], y0[1]), pack2(y0[2], y0[3]));
    *reinterpret_cast<uint2*>(dst + half + i) = make_uint2(pack2(y1[0], y1[1]), pack2(y1[2], y1[3]));
  }
  const int vch = a.hkv * a.d / 8;
  const uint16_t* vsrc = row + (a.hq + a.hkv) * a.d;
  uint16_t* vdst = a.v + (a.c0 + t) * a.hkv * a.d;
  for (int c = threadIdx.x; c < vch; c += kRopeThreads)
    *reinterpret_cast<uint4*>(vdst + c * 8) = *reinterpret_cast<const uint4*>(vsrc + c * 8);
}

// ---------------------------------------------------------------------------
// SwiGLU: one thread per eight outputs.
// ---------------------------------------------------------------------------
__device__ __forceinline__ float silu(float x) { return x / (1.0f + expf(-x)); }

__global__ void __launch_bounds__(256) swiglu_kernel(SwigluArgs a) {
  const int per = a.ffn / 8;
  const int64_t e = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (e >= a.rows * per) return;
  const int64_t r = e / per;
  const int c = (int)(e % per);
  const uint16_t* src = a.gu + r * 2 * a.ffn + c * 8;
  const uint4 g = *reinterpret_cast<const uint4*>(src);
  const uint4 u = *reinterpret_cast<const uint4*>(src + a.ffn);
  const uint32_t gw[4] = {g.x, g.y, g.z, g.w}, uw[4] = {u.x, u.y, u.z, u.w};
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    o[i] = pack2(silu(lo_f32(gw[i])) * lo_f32(uw[i]), silu(hi_f32(gw[i])) * hi_f32(uw[i]));
  *reinterpret_cast<uint4*>(a.a + r * a.ffn + c * 8) = make_uint4(o[0], o[1], o[2], o[3]);
}

// ---------------------------------------------------------------------------
// Chunk attention. A workgroup owns one KV head and 32 consecutive queries of
// the chunk, with one wavefront per query head of the group (G wavefronts),
// so the group shares every K/V tile staged in LDS. Per 32-key tile each
// wavefront computes S^T = K . Q^T on v_mfma_f32_32x32x16_bf16 (a lane owns
// one query and 16 keys: key 8(r/4) + 4 half + r%4 of register r), runs the
// online softmax in base 2, and accumulates O^T = V^T . P^T: the B operand is
// P straight from the registers (k-slot j of lane half `half` in k-slice s is
// the key 16s + 8(j/4) + 4 half + j%4 held in register 8s + j), the A operand
// reads V^T from LDS in that same key order: V is staged transposed
// ([d][key slot], rows padded to 40 slots) with the keys of each lane half's
// k-slice adjacent, so each lane's eight keys are one 16-byte read. Tiles are double-buffered through registers and LDS; the
// causal mask is applied on tiles that reach past the workgroup's first
// query. The running max is only raised when a tile's max exceeds it by more
// than 8 in base-2 units (weights up to 2^8 stay exact in fp32 and bf16), so
// most tiles skip rescaling the output accumulators; lanes that do not raise
// it scale by exactly 1. Workgroups with the most keys start first.
// ---------------------------------------------------------------------------
// x combined with x of lane l ^ 32 through one swap of the wavefront halves
// in the VALU (a __shfl_xor is an LDS permute round trip); both orders of the
// operands give the same bits.
__device__ __forceinline__ float max_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float add_other_half(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ f32x16_t mfma32(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

template <int D, int G>
__global__ void __launch_bounds__(64 * G) __attribute__((amdgpu_waves_per_eu(1, 2))) chunk_attention_kernel(AttnArgs a) {
  constexpr int CH = D / 8;         // 16-byte chunks per row
  constexpr int NST = D / 16;       // MFMA k-steps over D
  constexpr int DT = D / 32;        // 32-row tiles of O^T
  constexpr int PITCH = D + 8;      // +16 B per row: row-strided b128 reads stay conflict free
  constexpr int VP = 40;            // key slots per row of V^T (80 bytes: rows stay 16-byte aligned)
  constexpr int NT = 64 * G;
  constexpr int PER = (32 * CH + NT - 1) / NT;  // staged chunks per thread per matrix
  constexpr bool FULL = (32 * CH) % NT == 0;    // every thread stages PER chunks (no guard)
  __shared__ __align__(16) uint16_t ks[2][32 * PITCH];
  __shared__ __align__(16) uint16_t vt[2][D * VP];

  const int g = blockIdx.y;
  const int qt = gridDim.x - 1 - blockIdx.x;
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, l32 = lane & 31, half = lane >> 5;
  const int h = g * G + wave;
  const int64_t t0 = (int64_t)qt * 32;
  const int64_t p0 = a.c0 + t0;
  const int64_t pq = p0 + l32;
  const int64_t kmax = a.c0 + a.n - 1;                      // last cache row written
  const int64_t last_q = (p0 + 31 < kmax ? p0 + 31 : kmax);  // last valid query of the tile
  const int n_kt = (int)(last_q / 32) + 1;
  const int64_t tok = a.hkv * (int64_t)D;                    // cache token stride

  bf16x8_t qf[NST];
  {
    const int64_t tq = t0 + l32 < a.n ? t0 + l32 : a.n - 1;
    const uint16_t* qrow = a.q + (tq * a.hq + h) * D + half * (D / 2);
#pragma unroll
    for (int st = 0; st < NST; ++st) qf[st] = *reinterpret_cast<const bf16x8_t*>(qrow + 8 * st);
  }

  // two register sets: tile kt + 2 loads while tile kt is computed, so a
  // load has two tiles of work to land before its store to LDS
  // (passed by value: an array behind a reference would be moved to LDS)
  struct TileRegs {
    uint4 k[PER], v[PER];
  };
  auto load_tile = [&](int kt) {
    TileRegs r;
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = threadIdx.x + j * NT;
      if (FULL || u < 32 * CH) {
        // 16 keys per wavefront, each key row read in runs of 64 bytes
        int64_t key = (int64_t)kt * 32 + u % 16 + 16 * (u / (16 * CH));
        key = key < kmax ? key : kmax;
        const int64_t off = key * tok + (int64_t)g * D + ((u / 16) % CH) * 8;
        r.k[j] = *reinterpret_cast<const uint4*>(a.k + off);
        r.v[j] = *reinterpret_cast<const uint4*>(a.v + off);
      }
    }
    return r;
  };
  auto store_tile = [&](int b, TileRegs r) {
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int u = threadIdx.x + j * NT;
      if (FULL || u < 32 * CH) {
        const int key = u % 16 + 16 * (u / (16 * CH)), c = (u / 16) % CH;
        *reinterpret_cast<uint4*>(&ks[b][key * PITCH + c * 8]) = r.k[j];
        // The four lanes of a quad hold keys k0..k0+3 (same eight d values):
        // transpose their 4x4 dwords across the quad (two DPP swap steps) so
        // that lane q holds d values 2q, 2q + 1 of all four keys, then write
        // two 8-byte rows of V^T.
        uint32_t w[4] = {r.v[j].x, r.v[j].y, r.v[j].z, r.v[j].w};
        const int q = threadIdx.x & 3;
        {
          const uint32_t s0 = (q & 1) ? w[0] : w[1], s1 = (q & 1) ? w[2] : w[3];
          const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0xB1, 0xF, 0xF, false);
          const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0xB1, 0xF, 0xF, false);
          if (q & 1) { w[0] = r0; w[2] = r1; } else { w[1] = r0; w[3] = r1; }
        }
        {
          const uint32_t s0 = (q & 2) ? w[0] : w[2], s1 = (q & 2) ? w[1] : w[3];
          const uint32_t r0 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s0, 0x4E, 0xF, 0xF, false);
          const uint32_t r1 = (uint32_t)__builtin_amdgcn_mov_dpp((int)s1, 0x4E, 0xF, 0xF, false);
          if (q & 2) { w[0] = r0; w[1] = r1; } else { w[2] = r0; w[3] = r1; }
        }
        const int k0 = key & ~3;
        // key slot of k0 in a V^T row: keys 16s + 8a + 4h + i sit at 16s + 8h + 4a + i,
        // so the eight keys a lane half feeds one MFMA k-slice are adjacent
        const int slot = (k0 & ~15) | (((k0 >> 2) & 1) << 3) | (((k0 >> 3) & 1) << 2);
        uint16_t* row = &vt[b][(c * 8 + 2 * q) * VP + slot];
        *reinterpret_cast<uint2*>(row) =
            make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x05040100u), __builtin_amdgcn_perm(w[3], w[2], 0x05040100u));
        *reinterpret_cast<uint2*>(row + VP) =
            make_uint2(__builtin_amdgcn_perm(w[1], w[0], 0x07060302u), __builtin_amdgcn_perm(w[3], w[2], 0x07060302u));
      }
    }
  };

  float m = -INFINITY, l = 0.f;
  const float thr = 8.0f / a.c;  // lag of the running max allowed, in raw dot units
  f32x16_t o[DT];
#pragma unroll
  for (int dt = 0; dt < DT; ++dt) o[dt] = f32x16_t{};

  auto compute = [&](int kt) {
    const int b = kt & 1;
    f32x16_t s = {};
    const uint16_t* kr = &ks[b][l32 * PITCH + half * (D / 2)];
#pragma unroll
    for (int st = 0; st < NST; ++st) s = mfma32(*reinterpret_cast<const bf16x8_t*>(kr + 8 * st), qf[st], s);

    const int64_t kb = (int64_t)kt * 32;
    if (kb + 31 > p0) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int64_t key = kb + 8 * (r >> 2) + 4 * half + (r & 3);
        if (key > pq) s[r] = -INFINITY;
      }
    }
    float tmax = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) tmax = fmaxf(tmax, s[r]);
    tmax = max_other_half(tmax);               // finite: key 0 is seen by every query
    const bool up = tmax > m + thr;            // always on the first tile (m = -inf)
    if (__ballot(up) != 0) {
      const float corr = up ? __builtin_amdgcn_exp2f((m - tmax) * a.c) : 1.0f;
      m = up ? tmax : m;
      l *= corr;
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[dt][r] *= corr;
    }
    const float mc = m * a.c;
    float psum = 0.f;
    float p[16];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      p[r] = __builtin_amdgcn_exp2f(fmaf(s[r], a.c, -mc));
      psum += p[r];
    }
    l += psum;

#pragma unroll
    for (int ks_ = 0; ks_ < 2; ++ks_) {
      bf16x8_t pb;
#pragma unroll
      for (int j = 0; j < 8; ++j) pb[j] = (__bf16)p[8 * ks_ + j];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        // slots 16s + 8 half + 0..7 hold keys 16s + 8(j/4) + 4 half + j%4
        const bf16x8_t va =
            *reinterpret_cast<const bf16x8_t*>(&vt[b][(dt * 32 + l32) * VP + 16 * ks_ + 8 * half]);
        o[dt] = mfma32(va, pb, o[dt]);
      }
    }
  };

  // tile kt + 1 is in one register set, the other is free for tile kt + 2;
  // tiles past the end load clamped rows and are never read
  TileRegs rA = load_tile(0);
  TileRegs rB = load_tile(1);
  store_tile(0, rA);
  __syncthreads();
  for (int kt = 0; kt < n_kt; kt += 2) {
    rA = load_tile(kt + 2);
    compute(kt);
    store_tile((kt + 1) & 1, rB);
    __syncthreads();
    if (kt + 1 >= n_kt) break;
    rB = load_tile(kt + 3);
    compute(kt + 1);
    store_tile(kt & 1, rA);
    __syncthreads();
  }

  const float lt = add_other_half(l);
  const float inv = 1.0f / lt;
  if (t0 + l32 < a.n) {
    uint16_t* orow = a.o + ((t0 + l32) * a.hq + h) * D;
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int d = dt * 32 + 8 * q4 + 4 * half;
        *reinterpret_cast<uint2*>(orow + d) =
            make_uint2(pack2(o[dt][4 * q4] * inv, o[dt][4 * q4 + 1] * inv),
                       pack2(o[dt][4 * q4 + 2] * inv, o[dt][4 * q4 + 3] * inv));
      }
  }
}

template <int D>
hipError_t launch_attention_d(const AttnArgs& a, hipStream_t st) {
  AttnArgs args = a;
  void* kargs[] = {&args};
  const dim3 grid((unsigned)((a.n + 31) / 32), (unsigned)a.hkv);
  const void* fn;
  switch (a.g) {
    case 1: fn = reinterpret_cast<const void*>(&chunk_attention_kernel<D, 1>); break;
    case 2: fn = reinterpret_cast<const void*>(&chunk_attention_kernel<D, 2>); break;
    case 4: fn = reinterpret_cast<const void*>(&chunk_attention_kernel<D, 4>); break;
    case 8: fn = reinterpret_cast<const void*>(&chunk_attention_kernel<D, 8>); break;
    default: return hipErrorInvalidValue;
  }
  return hipLaunchKernel(fn, grid, dim3(64 * a.g), kargs, 0, st);
}

}  // namespace

hipError_t launch_rmsnorm(const NormArgs& a, hipStream_t st) {
  if (a.rows == 0) return hipSuccess;
  NormArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rmsnorm_kernel), dim3((unsigned)a.rows), dim3(kNormThreads),
                         kargs, 0, st);
}

hipError_t launch_rope_append(const RopeArgs& a, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  RopeArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&rope_append_kernel), dim3((unsigned)a.n), dim3(kRopeThreads),
                         kargs, 0, st);
}

hipError_t launch_chunk_attention(const AttnArgs& a, int d, hipStream_t st) {
  if (a.n == 0) return hipSuccess;
  return d == 64 ? launch_attention_d<64>(a, st) : launch_attention_d<128>(a, st);
}

hipError_t launch_swiglu(const SwigluArgs& a, hipStream_t st) {
  const int64_t units = a.rows * (a.ffn / 8);
  if (units == 0) return hipSuccess;
  SwigluArgs args = a;
  void* kargs[] = {&args};
  return hipLaunchKernel(reinterpret_cast<const void*>(&swiglu_kernel), dim3((unsigned)((units + 255) / 256)),
                         dim3(256), kargs, 0, st);
}

}  // namespace kvc
