// Device helpers and internal launcher declarations shared by the HIP sources of the X-MoD
// layer library (gfx950, wave64). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace xmod {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest even (inputs are finite).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return (uint32_t)f32_to_bf16(lo) | ((uint32_t)f32_to_bf16(hi) << 16);
}
// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4 &v, float *f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
__device__ __forceinline__ uint4 pack8(const float *f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Gated residual of one element, in the fixed order g = varsigma*r, t = a + f, p = g*t,
// y = X + p, each rounded in fp32 (no contraction). Shared by the standalone scatter and the
// fused down-projection epilogue so both give identical bits.
__device__ __forceinline__ float gated_residual(float X, float g, float a, float f) {
  const float t = __fadd_rn(a, f);
  const float p = __fmul_rn(g, t);
  return __fadd_rn(X, p);
}
// Dense residual: y = X + (a + f).
__device__ __forceinline__ float dense_residual(float X, float a, float f) {
  return __fadd_rn(X, __fadd_rn(a, f));
}

}  // namespace xmod

// ---- launchers (host side, defined in the .hip files) ---------------------------------------
namespace xmod {

hipError_t launch_router(const uint16_t *x, const uint16_t *w, float beta, const float *bias,
                         float tau, float *logits, int64_t rows, int d, hipStream_t s);

hipError_t launch_topk(const float *logits, int B, int T, int k, int32_t *idx, float *gate,
                       float *bias, float delta, hipStream_t s);

// Gather rows (via idx, or identity when idx == nullptr) and optionally RMSNorm them.
hipError_t launch_gather_rows(const uint16_t *x, const int32_t *idx, const uint16_t *gain,
                              float eps, bool normalize, int B, int T, int d, int k,
                              uint16_t *out, hipStream_t s);

// v[m] = RMSNorm(X[m] + a[m]; gain), X gathered from x via idx (identity when nullptr); a fp32.
hipError_t launch_residual_rmsnorm(const uint16_t *x, const int32_t *idx, const float *a,
                                   const uint16_t *gain, float eps, int B, int T, int d, int k,
                                   uint16_t *v, hipStream_t s);

// Standalone gated scatter (gate != nullptr) or dense residual (gate == nullptr, idx == nullptr).
hipError_t launch_scatter(uint16_t *x, const int32_t *idx, const float *gate, float varsigma,
                          const uint16_t *a, const uint16_t *f, int B, int T, int d, int k,
                          hipStream_t s);

enum GemmEpilogue { EPI_STORE = 0, EPI_SWIGLU = 1, EPI_RESIDUAL = 2, EPI_STORE_F32 = 3 };

struct GemmArgs {
  const uint16_t *A;  int lda;     // [M, K] activations
  const uint16_t *B;  int ldb;     // [N, K] weights (EPI_SWIGLU: gate weights, N = F)
  const uint16_t *B2;              // EPI_SWIGLU: up weights [N, K], same ldb
  uint16_t *C;        int ldc;     // EPI_STORE / EPI_SWIGLU bf16 output [M, N]
  float *Cf;                       // EPI_STORE_F32 fp32 output [M, N], same ldc
  int M, N, K;
  // EPI_RESIDUAL: output row m is x[b*T + idx[m]] (identity when idx == nullptr); the
  // accumulator is f (kept fp32), added as X + varsigma*gate[m]*(a + f), or X + (a + f) if
  // gate == nullptr; a is fp32 [M, N] with leading dimension ldc, as is x.
  uint16_t *x; const int32_t *idx; const float *gate; float varsigma;
  const float *a; int T; int k;
};

hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, hipStream_t s);

hipError_t launch_attention(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, int B, int k,
                            int Hq, int Hkv, int hd, hipStream_t s);

}  // namespace xmod
