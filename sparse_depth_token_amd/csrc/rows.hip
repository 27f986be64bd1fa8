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
                                                          uint16_t *__restrict__ out) {
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
                              hipStream_t s) {
  if (rows < 1) return hipSuccess;
  const dim3 grid = row_grid(map, rows);
#define L_(NI)                                                                                  \
  if (normalize)                                                                                \
    hipLaunchKernelGGL((gather_rows_kernel<NI, true>), grid, dim3(256), 0, s, x, map, gain, eps, \
                       d, rows, out);                                                           \
  else                                                                                          \
    hipLaunchKernelGGL((gather_rows_kernel<NI, false>), grid, dim3(256), 0, s, x, map, gain,    \
                       eps, d, rows, out)
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

}  // namespace xmod
