// Row-wise kernels of the X-MoD sparse layer (gfx950, wave64): gather/pack of the selected
// rows with the RMSNorm before attention, the RMSNorm before the FFN on X + a (a in fp32), and
// the standalone gated scatter of the X-MoD review's Eq. (7). One wave owns one row of d <= 8192 bf16 values held
// in registers (16-byte chunks, 64 lanes side by side, so every access is coalesced).
// Packed row m maps to a row of x through a RowMap (top-k: b*T + idx[m] with m = b*k + j;
// threshold routing: a flat list with a device-side count; dense layers: identity).
#include "common.h"

namespace xmod {

template <int NI, bool NORM>
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t *__restrict__ x,
                                                          RowMap map,
                                                          const uint16_t *__restrict__ gain,
                                                          float eps, int d, int64_t rows,
                                                          uint16_t *__restrict__ out,
                                                          uint16_t *__restrict__ xraw) {
  const int lane = threadIdx.x & 63;
  const int64_t n_rows = rowmap_count(map, rows);
  for (int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); m < n_rows;
       m += (int64_t)gridDim.x * 4) {
  const int nch = d >> 3;
  const uint16_t *src = x + rowmap_x(map, m) * d;
  uint4 v[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < nch ? *(const uint4 *)(src + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
  }
  uint16_t *dst = out + m * d;
  if (!NORM) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) *(uint4 *)(dst + (size_t)c * 8) = v[i];
    }
    continue;
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    float f[8];
    unpack8(v[i], f);
#pragma unroll
    for (int e = 0; e < 8; ++e) ss = fmaf(f[e], f[e], ss);
  }
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float f[8], g[8];
      if (xraw) *(uint4 *)(xraw + m * d + (size_t)c * 8) = v[i];  // the gathered row itself
      unpack8(v[i], f);
      unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = f[e] * rinv * g[e];
      *(uint4 *)(dst + (size_t)c * 8) = pack8(f);
    }
  }
  }  // row loop
}

template <int NI>
__global__ __launch_bounds__(256) void residual_rmsnorm_kernel(
    const uint16_t *__restrict__ x, RowMap map, const float *__restrict__ a,
    const uint16_t *__restrict__ gain, float eps, int d, int64_t rows,
    uint16_t *__restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t n_rows = rowmap_count(map, rows);
  for (int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); m < n_rows;
       m += (int64_t)gridDim.x * 4) {
  const int nch = d >> 3;
  const uint16_t *src = x + rowmap_x(map, m) * d;
  const float *arow = a + m * d;
  float h[NI][8];
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float xf[8];
      unpack8(*(const uint4 *)(src + (size_t)c * 8), xf);
      const float4 a0 = *(const float4 *)(arow + (size_t)c * 8);
      const float4 a1 = *(const float4 *)(arow + (size_t)c * 8 + 4);
      const float af[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        h[i][e] = xf[e] + af[e];
        ss = fmaf(h[i][e], h[i][e], ss);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) h[i][e] = 0.f;
    }
  }
  ss = wave_sum(ss);
  const float rinv = 1.0f / sqrtf(ss / (float)d + eps);
  uint16_t *dst = out + m * d;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float g[8], f[8];
      unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
#pragma unroll
      for (int e = 0; e < 8; ++e) f[e] = h[i][e] * rinv * g[e];
      *(uint4 *)(dst + (size_t)c * 8) = pack8(f);
    }
  }
  }  // row loop
}

template <int NI>
__global__ __launch_bounds__(256) void scatter_kernel(uint16_t *__restrict__ x, RowMap map,
                                                      const float *__restrict__ gate,
                                                      float varsigma,
                                                      const uint16_t *__restrict__ a,
                                                      const uint16_t *__restrict__ f, int d,
                                                      int64_t rows) {
  const int lane = threadIdx.x & 63;
  const int64_t n_rows = rowmap_count(map, rows);
  for (int64_t m = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6); m < n_rows;
       m += (int64_t)gridDim.x * 4) {
  const int nch = d >> 3;
  uint16_t *xr = x + rowmap_x(map, m) * d;
  const float g = gate ? __fmul_rn(varsigma, gate[m]) : 0.f;
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      float X[8], A[8], F[8], Y[8];
      unpack8(*(const uint4 *)(xr + (size_t)c * 8), X);
      unpack8(*(const uint4 *)(a + m * d + (size_t)c * 8), A);
      unpack8(*(const uint4 *)(f + m * d + (size_t)c * 8), F);
#pragma unroll
      for (int e = 0; e < 8; ++e)
        Y[e] = gate ? gated_residual(X[e], g, A[e], F[e]) : dense_residual(X[e], A[e], F[e]);
      *(uint4 *)(xr + (size_t)c * 8) = pack8(Y);
    }
  }
  }  // row loop
}

// Per-head RMSNorm (QK-norm) and rotary embedding of the packed queries and keys, in place.
// Query head h of a row sits at columns h*HD, key head g at (Hq + g)*HD. One head is handled by
// HD/2 lanes: lane i holds the pair (i, i + HD/2) that the rotation mixes. The rotation angle
// is pos * theta^(-2i/HD), taken in double and reduced to [-pi, pi] before the fp32 sine and
// cosine, so long positions lose no accuracy.
template <int HD>
__global__ __launch_bounds__(256) void qk_form_kernel(uint16_t *__restrict__ qkv, int ldq,
                                                      RowMap map, int64_t rows, int Hq, int Hkv,
                                                      const uint16_t *__restrict__ q_norm,
                                                      const uint16_t *__restrict__ k_norm,
                                                      float eps, float theta) {
  constexpr int P = HD / 2;     // lanes per head
  constexpr int TPW = 64 / P;   // heads per wave
  const int lane = threadIdx.x & 63, sub = lane / P, i = lane % P;
  const int nh = Hq + Hkv;
  const int64_t n_tasks = rowmap_count(map, rows) * nh;
  const double inv_freq = theta > 0.f ? pow((double)theta, -2.0 * i / HD) : 0.0;
  const int64_t stride = (int64_t)gridDim.x * 4 * TPW;
  for (int64_t t0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * TPW; t0 < n_tasks;
       t0 += stride) {
    const int64_t task = t0 + sub;
    const bool valid = task < n_tasks;
    const int64_t m = valid ? task / nh : 0;
    const int h = valid ? (int)(task % nh) : 0;
    const uint16_t *gain = h < Hq ? q_norm : k_norm;
    uint16_t *z = qkv + m * ldq + (int64_t)h * HD;
    float z1 = valid ? bf16_to_f32(z[i]) : 0.f, z2 = valid ? bf16_to_f32(z[i + P]) : 0.f;
    float ss = z1 * z1 + z2 * z2;
#pragma unroll
    for (int o = P / 2; o > 0; o >>= 1) ss += __shfl_xor(ss, o, 64);  // within the head's lanes
    if (valid && gain) {
      const float r = 1.0f / sqrtf(ss / (float)HD + eps);
      z1 = z1 * r * bf16_to_f32(gain[i]);
      z2 = z2 * r * bf16_to_f32(gain[i + P]);
    }
    if (valid && theta > 0.f) {
      const int64_t pos = rowmap_x(map, m) % map.T;
      double ang = (double)pos * inv_freq;
      ang -= 6.283185307179586 * rint(ang * 0.15915494309189535);
      float sn, cs;
      sincosf((float)ang, &sn, &cs);
      const float r1 = z1 * cs - z2 * sn, r2 = z2 * cs + z1 * sn;
      z1 = r1;
      z2 = r2;
    }
    if (valid && (gain || theta > 0.f)) {
      z[i] = f32_to_bf16(z1);
      z[i + P] = f32_to_bf16(z2);
    }
  }
}

static int ni_for(int d) { return ((d >> 3) + 63) / 64; }

#define XMOD_NI_SWITCH(ni, MACRO)                 \
  switch (ni) {                                   \
    case 1: MACRO(1); break;                      \
    case 2: MACRO(2); break;                      \
    case 3: MACRO(3); break;                      \
    case 4: MACRO(4); break;                      \
    case 5: case 6: MACRO(6); break;              \
    case 7: case 8: MACRO(8); break;              \
    default: MACRO(16); break;                    \
  }

// Four rows per workgroup; with a device-side row count the grid is capped and the waves
// loop, so a bound far above the actual count costs no idle workgroups.
static dim3 row_grid(const RowMap &map, int64_t rows) {
  const int64_t wgs = (rows + 3) / 4;
  return dim3((unsigned)(map.n_dev ? (wgs < 2048 ? wgs : 2048) : wgs));
}

hipError_t launch_gather_rows(const uint16_t *x, const RowMap &map, const uint16_t *gain,
                              float eps, bool normalize, int64_t rows, int d, uint16_t *out,
                              hipStream_t s, uint16_t *xraw) {
  if (rows < 1) return hipSuccess;
  const dim3 grid = row_grid(map, rows);
#define L_(NI)                                                                                  \
  if (normalize)                                                                                \
    hipLaunchKernelGGL((gather_rows_kernel<NI, true>), grid, dim3(256), 0, s, x, map, gain, eps, \
                       d, rows, out, xraw);                                                     \
  else                                                                                          \
    hipLaunchKernelGGL((gather_rows_kernel<NI, false>), grid, dim3(256), 0, s, x, map, gain,    \
                       eps, d, rows, out, nullptr)
  XMOD_NI_SWITCH(ni_for(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_residual_rmsnorm(const uint16_t *x, const RowMap &map, const float *a,
                                   const uint16_t *gain, float eps, int64_t rows, int d,
                                   uint16_t *v, hipStream_t s) {
  if (rows < 1) return hipSuccess;
  const dim3 grid = row_grid(map, rows);
#define L_(NI)                                                                              \
  hipLaunchKernelGGL((residual_rmsnorm_kernel<NI>), grid, dim3(256), 0, s, x, map, a, gain, \
                     eps, d, rows, v)
  XMOD_NI_SWITCH(ni_for(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_scatter(uint16_t *x, const RowMap &map, const float *gate, float varsigma,
                          const uint16_t *a, const uint16_t *f, int64_t rows, int d,
                          hipStream_t s) {
  if (rows < 1) return hipSuccess;
  const dim3 grid = row_grid(map, rows);
#define L_(NI)                                                                                 \
  hipLaunchKernelGGL((scatter_kernel<NI>), grid, dim3(256), 0, s, x, map, gate, varsigma, a, f, \
                     d, rows)
  XMOD_NI_SWITCH(ni_for(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_qk_form(uint16_t *qkv, int ld_qkv, const RowMap &map, int64_t rows, int Hq,
                          int Hkv, int hd, const uint16_t *q_norm, const uint16_t *k_norm,
                          float eps, float theta, hipStream_t s) {
  if (rows < 1 || (!q_norm && !k_norm && !(theta > 0.f))) return hipSuccess;
  const int64_t waves = (rows * (Hq + Hkv) * (hd / 2) + 63) / 64;
  const int64_t wgs = (waves + 3) / 4;
  const dim3 grid((unsigned)(wgs < 4096 ? wgs : 4096));
  if (hd == 128)
    hipLaunchKernelGGL(qk_form_kernel<128>, grid, dim3(256), 0, s, qkv, ld_qkv, map, rows, Hq,
                       Hkv, q_norm, k_norm, eps, theta);
  else
    hipLaunchKernelGGL(qk_form_kernel<64>, grid, dim3(256), 0, s, qkv, ld_qkv, map, rows, Hq,
                       Hkv, q_norm, k_norm, eps, theta);
  return hipGetLastError();
}

}  // namespace xmod
