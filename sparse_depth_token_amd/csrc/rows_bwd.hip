// Row-wise kernels of the backward pass of the X-MoD Sparse(K) layer (gfx950, wave64).
//
// The forward of a selected row (X-MoD review, Eq. (7) with the gate r of Eq. (8)):
//   u = RMSNorm(X; g1), h = X + a, v = RMSNorm(h; g2), y = X + (varsigma r) (a + f).
// For the upstream gradient G = dy of a selected row:
//   dt = varsigma r G (the gradient reaching a and f), dc = G . (a + f), dr = varsigma dc,
//   d varsigma += r dc, and the router logit gets dr r (1 - r) (the sigmoid's derivative);
//   dh = RMSNorm'(h)^T dv (dv from the FFN's backward), da = dt + dh,
//   dX = G + dh + RMSNorm'(X)^T du (du from the QKV projection's backward).
// For every token, selected or not, the routing loss of the page's "training-time top-k,
// eval-time causal threshold" section (Eq. (9): binary cross-entropy of the top-k decision q
// against sigmoid(s), averaged over the n = B*T tokens) adds coef (sigmoid(s) - q) / n to the
// logit's gradient ds; the router s = w_r . x + beta passes ds w_r to dx and ds x to d w_r.
// RMSNorm'(z)^T g for a row z with r = (mean(z^2) + eps)^(-1/2) and gain gamma:
//   r (g gamma) - (r^3 / d) ((g gamma) . z) z, and d gamma += g z r.
//
// The forward updates x in place (selected rows then hold y), so the router-weight gradient of
// a selected token is taken from the saved packed row X (in the RMSNorm-1 kernel), that of an
// unselected token from x (in the router kernel).
//
// One wave per row, 8 columns per lane per 512-column step. Column sums (gain and router-weight
// gradients) and scalar sums are accumulated per lane over the rows a wave visits, added over
// the workgroup's four waves in LDS and written as one partial row per workgroup; a final
// two-level sum adds the partial rows. Every sum runs in a fixed order, so the results do not
// depend on scheduling.
#include "common.h"

namespace xmod {

__device__ __forceinline__ void load8f(const float *p, float *f) {
  const f32x4 a = *(const f32x4 *)p, b = *(const f32x4 *)(p + 4);
  f[0] = a[0]; f[1] = a[1]; f[2] = a[2]; f[3] = a[3];
  f[4] = b[0]; f[5] = b[1]; f[6] = b[2]; f[7] = b[3];
}
__device__ __forceinline__ void store8f(float *p, const float *f) {
  f32x4 a, b;
  a[0] = f[0]; a[1] = f[1]; a[2] = f[2]; a[3] = f[3];
  b[0] = f[4]; b[1] = f[5]; b[2] = f[6]; b[3] = f[7];
  *(f32x4 *)p = a;
  *(f32x4 *)(p + 4) = b;
}
// log(1 + e^z) without overflow or cancellation
__device__ __forceinline__ float softplus(float z) {
  return fmaxf(z, 0.f) + log1pf(expf(-fabsf(z)));
}

// Sum of the four waves' per-lane column accumulators (columns 8 c + e for chunk c = lane +
// 64 i), in wave order, through LDS; the workgroup's partial row goes to dst[0, d).
template <int NI>
__device__ __forceinline__ void wg_colsum_store(const float (&acc)[NI][8], float *red, int d,
                                                float *__restrict__ dst) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, nch = d >> 3;
  __syncthreads();  // a previous use of `red` is complete
#pragma unroll
  for (int step = 0; step < 4; ++step) {
    if (w == step) {
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = lane + 64 * i;
        if (c < nch)
#pragma unroll
          for (int e = 0; e < 8; ++e) red[c * 8 + e] = (step == 0 ? 0.f : red[c * 8 + e]) + acc[i][e];
      }
    }
    __syncthreads();
  }
  for (int c = threadIdx.x; c < d; c += 256) dst[c] = red[c];
}
// The same for one number per wave (lane 0's value).
__device__ __forceinline__ void wg_sum_store(float v, float *red4, float *dst) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  if (lane == 0) red4[w] = v;
  __syncthreads();
  if (threadIdx.x == 0) *dst = ((red4[0] + red4[1]) + red4[2]) + red4[3];
}

__global__ __launch_bounds__(256) void zero16_kernel(uint4 *__restrict__ p, int64_t n16) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n16;
       i += (int64_t)gridDim.x * 256)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

hipError_t launch_zero(void *p, size_t bytes, hipStream_t s) {
  const int64_t n16 = (int64_t)(bytes / 16);
  if (n16 < 1) return hipSuccess;
  const int64_t wgs = (n16 + 255) / 256;
  hipLaunchKernelGGL(zero16_kernel, dim3((unsigned)(wgs < 4096 ? wgs : 4096)), dim3(256), 0, s,
                     (uint4 *)p, n16);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void copy32_kernel(uint32_t *__restrict__ dst,
                                                     const uint32_t *__restrict__ src, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
    dst[i] = src[i];
}

hipError_t launch_copy32(void *dst, const void *src, int64_t n_words, hipStream_t s) {
  if (n_words < 1) return hipSuccess;
  const int64_t wgs = (n_words + 255) / 256;
  hipLaunchKernelGGL(copy32_kernel, dim3((unsigned)(wgs < 1024 ? wgs : 1024)), dim3(256), 0, s,
                     (uint32_t *)dst, (const uint32_t *)src, n_words);
  return hipGetLastError();
}

// Workgroups of the row kernels over the packed rows and over every token; each writes one
// partial row of its column sums. The router pass over every token is HBM-bound: its grid is
// what stays resident at once (three workgroups per CU at d = 2048), so no second, thinly
// occupied round of workgroups trails the first.
constexpr int BWD_ROW_WGS = 512;
constexpr int BWD_ROUTE_WGS = 768;

// ---- gated residual ------------------------------------------------------------------------
template <int NI>
__global__ __launch_bounds__(256) void resid_bwd_kernel(
    const uint16_t *__restrict__ dy, RowMap map, const float *__restrict__ a,
    const float *__restrict__ f, const float *__restrict__ gate, float varsigma, int d, int64_t M,
    int64_t M_pad, uint16_t *__restrict__ dt, float *__restrict__ dell,
    float *__restrict__ dell_tok, uint8_t *__restrict__ q_tok, float *__restrict__ vs_part) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = d >> 3;
  float vs_acc = 0.f;
  for (int64_t m = wave; m < M_pad; m += (int64_t)gridDim.x * 4) {
    uint16_t *dtr = dt + m * d;
    if (m >= M) {  // padding rows of the packed operands are zero
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (lane + 64 * i < nch) *(uint4 *)(dtr + (size_t)(lane + 64 * i) * 8) = make_uint4(0, 0, 0, 0);
      continue;
    }
    const int64_t xrow = rowmap_x(map, m);
    const float r = gate[m];
    const float cg = __fmul_rn(varsigma, r);
    float dc = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        float G[8], A[8], Fv[8], o[8];
        unpack8(*(const uint4 *)(dy + xrow * d + (size_t)c * 8), G);
        load8f(a + m * d + (size_t)c * 8, A);
        load8f(f + m * d + (size_t)c * 8, Fv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          dc = fmaf(G[e], __fadd_rn(A[e], Fv[e]), dc);
          o[e] = cg * G[e];
        }
        *(uint4 *)(dtr + (size_t)c * 8) = pack8(o);
      }
    }
    dc = wave_sum(dc);
    if (lane == 0) {
      const float dl = varsigma * dc * r * (1.f - r);
      dell[m] = dl;
      dell_tok[xrow] = dl;
      q_tok[xrow] = 1;
      vs_acc = fmaf(r, dc, vs_acc);
    }
  }
  __shared__ float red4[4];
  wg_sum_store(vs_acc, red4, vs_part + blockIdx.x);
}

// ---- RMSNorm before the FFN ------------------------------------------------------------------
template <int NI>
__global__ __launch_bounds__(256) void rms2_bwd_kernel(
    const uint16_t *__restrict__ dy, RowMap map, const uint16_t *__restrict__ X,
    const float *__restrict__ a, const float *__restrict__ dv, const uint16_t *__restrict__ gain,
    float eps, const uint16_t *__restrict__ dt, int d, int64_t M, int64_t M_pad,
    uint16_t *__restrict__ da, float *__restrict__ dXacc, float *__restrict__ g_part) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = d >> 3;
  float gacc[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) gacc[i][e] = 0.f;
  for (int64_t m = wave; m < M_pad; m += (int64_t)gridDim.x * 4) {
    if (m >= M) {
#pragma unroll
      for (int i = 0; i < NI; ++i)
        if (lane + 64 * i < nch)
          *(uint4 *)(da + m * d + (size_t)(lane + 64 * i) * 8) = make_uint4(0, 0, 0, 0);
      continue;
    }
    uint4 xv[NI];
    float ss = 0.f, sg = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      xv[i] = make_uint4(0, 0, 0, 0);
      if (c < nch) {
        xv[i] = *(const uint4 *)(X + m * d + (size_t)c * 8);
        float Xf[8], A[8], D[8], g[8];
        unpack8(xv[i], Xf);
        load8f(a + m * d + (size_t)c * 8, A);
        load8f(dv + m * d + (size_t)c * 8, D);
        unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float h = Xf[e] + A[e];
          ss = fmaf(h, h, ss);
          sg = fmaf(D[e] * g[e], h, sg);
        }
      }
    }
    ss = wave_sum(ss);
    sg = wave_sum(sg);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    const float cf = r * r * r * sg / (float)d;
    const uint16_t *gy = dy + rowmap_x(map, m) * d;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        float Xf[8], A[8], D[8], g[8], T[8], G[8], o[8], dx[8];
        unpack8(xv[i], Xf);
        load8f(a + m * d + (size_t)c * 8, A);
        load8f(dv + m * d + (size_t)c * 8, D);
        unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
        unpack8(*(const uint4 *)(dt + m * d + (size_t)c * 8), T);
        unpack8(*(const uint4 *)(gy + (size_t)c * 8), G);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float h = Xf[e] + A[e];
          const float dh = r * (D[e] * g[e]) - cf * h;
          o[e] = T[e] + dh;
          dx[e] = G[e] + dh;
          gacc[i][e] = fmaf(D[e] * h, r, gacc[i][e]);
        }
        *(uint4 *)(da + m * d + (size_t)c * 8) = pack8(o);
        store8f(dXacc + m * d + (size_t)c * 8, dx);
      }
    }
  }
  __shared__ float red[NI * 512];
  wg_colsum_store<NI>(gacc, red, d, g_part + (int64_t)blockIdx.x * d);
}

// ---- RMSNorm before attention; writes the selected rows of dx ---------------------------------
template <int NI>
__global__ __launch_bounds__(256) void rms1_bwd_kernel(
    const uint16_t *__restrict__ X, RowMap map, const float *__restrict__ du,
    const uint16_t *__restrict__ gain, float eps, const float *__restrict__ dXacc,
    const float *__restrict__ s_tok, const float *__restrict__ dell, float coef_n,
    const uint16_t *__restrict__ w_r, int d, int64_t M, uint16_t *__restrict__ dx,
    float *__restrict__ g_part, float *__restrict__ wr_part) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = d >> 3;
  float gacc[NI][8], wacc[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) { gacc[i][e] = 0.f; wacc[i][e] = 0.f; }
  for (int64_t m = wave; m < M; m += (int64_t)gridDim.x * 4) {
    uint4 xv[NI];
    float ss = 0.f, sg = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      xv[i] = make_uint4(0, 0, 0, 0);
      if (c < nch) {
        xv[i] = *(const uint4 *)(X + m * d + (size_t)c * 8);
        float Xf[8], D[8], g[8];
        unpack8(xv[i], Xf);
        load8f(du + m * d + (size_t)c * 8, D);
        unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          ss = fmaf(Xf[e], Xf[e], ss);
          sg = fmaf(D[e] * g[e], Xf[e], sg);
        }
      }
    }
    ss = wave_sum(ss);
    sg = wave_sum(sg);
    const float r = 1.0f / sqrtf(ss / (float)d + eps);
    const float cf = r * r * r * sg / (float)d;
    const int64_t xrow = rowmap_x(map, m);
    const float p = 1.0f / (1.0f + expf(-s_tok[xrow]));
    const float ds = dell[m] + coef_n * (p - 1.0f);  // a selected token: q = 1
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      if (c < nch) {
        float Xf[8], D[8], g[8], acc[8], w[8], o[8];
        unpack8(xv[i], Xf);
        load8f(du + m * d + (size_t)c * 8, D);
        unpack8(*(const uint4 *)(gain + (size_t)c * 8), g);
        load8f(dXacc + m * d + (size_t)c * 8, acc);
        unpack8(*(const uint4 *)(w_r + (size_t)c * 8), w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float dX1 = r * (D[e] * g[e]) - cf * Xf[e];
          o[e] = acc[e] + dX1 + ds * w[e];
          gacc[i][e] = fmaf(D[e] * Xf[e], r, gacc[i][e]);
          wacc[i][e] = fmaf(ds, Xf[e], wacc[i][e]);
        }
        *(uint4 *)(dx + xrow * d + (size_t)c * 8) = pack8(o);
      }
    }
  }
  __shared__ float red[NI * 512];
  wg_colsum_store<NI>(gacc, red, d, g_part + (int64_t)blockIdx.x * d);
  wg_colsum_store<NI>(wacc, red, d, wr_part + (int64_t)blockIdx.x * d);
}

// ---- router and routing loss over every token; writes the unselected rows of dx --------------
template <int NI>
__global__ __launch_bounds__(256) void route_bwd_kernel(
    const uint16_t *__restrict__ x, const uint16_t *__restrict__ dy,
    const float *__restrict__ s_tok, const float *__restrict__ dell_tok,
    const uint8_t *__restrict__ q_tok, float coef_n, const uint16_t *__restrict__ w_r, int d,
    int64_t rows, uint16_t *__restrict__ dx, float *__restrict__ wr_part,
    float *__restrict__ beta_part, float *__restrict__ loss_part) {
  const int lane = threadIdx.x & 63;
  const int wave = blockIdx.x * 4 + (threadIdx.x >> 6);
  const int nch = d >> 3;
  float wacc[NI][8], wr[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) unpack8(*(const uint4 *)(w_r + (size_t)c * 8), wr[i]);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      wacc[i][e] = 0.f;
      if (c >= nch) wr[i][e] = 0.f;
    }
  }
  float bacc = 0.f, lacc = 0.f;
  const int64_t stride = (int64_t)gridDim.x * 4;
  // two rows per step, their loads issued together
  for (int64_t t0 = wave; t0 < rows; t0 += 2 * stride) {
    int64_t tt[2] = {t0, t0 + stride};
    float ds[2];
    bool sel[2];
    uint4 xv[2][NI], gv[2][NI];
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      const bool ok = tt[r] < rows;
      const int64_t t = ok ? tt[r] : t0;
      const float sv = s_tok[t];
      const bool q = q_tok[t] != 0;
      const float p = 1.0f / (1.0f + expf(-sv));
      ds[r] = dell_tok[t] + coef_n * (p - (q ? 1.0f : 0.0f));
      sel[r] = q || !ok;  // nothing to write (a selected row's dx and router-weight term come
                          // from the saved X)
      if (ok) {
        // -log p = softplus(-s), -log(1 - p) = softplus(s)
        lacc += q ? softplus(-sv) : softplus(sv);
        bacc += ds[r];
      }
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = lane + 64 * i;
        xv[r][i] = gv[r][i] = make_uint4(0, 0, 0, 0);
        if (c < nch && !sel[r]) {
          xv[r][i] = *(const uint4 *)(x + t * d + (size_t)c * 8);
          gv[r][i] = *(const uint4 *)(dy + t * d + (size_t)c * 8);
        }
      }
    }
#pragma unroll
    for (int r = 0; r < 2; ++r) {
      if (sel[r]) continue;
#pragma unroll
      for (int i = 0; i < NI; ++i) {
        const int c = lane + 64 * i;
        if (c < nch) {
          float Xf[8], G[8], o[8];
          unpack8(xv[r][i], Xf);
          unpack8(gv[r][i], G);
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            wacc[i][e] = fmaf(ds[r], Xf[e], wacc[i][e]);
            o[e] = G[e] + ds[r] * wr[i][e];
          }
          *(uint4 *)(dx + tt[r] * d + (size_t)c * 8) = pack8_int(o);  // (fewer spills)
        }
      }
    }
  }
  __shared__ float red[NI * 512];
  __shared__ float red4[4];
  wg_colsum_store<NI>(wacc, red, d, wr_part + (int64_t)blockIdx.x * d);
  wg_sum_store(bacc, red4, beta_part + blockIdx.x);
  __syncthreads();
  wg_sum_store(lacc, red4, loss_part + blockIdx.x);
}

// ---- fixed-order sums of partial rows --------------------------------------------------------
// Level 0: job j's partial rows are split in COLSUM_CHUNKS chunks; workgroup (column block,
// chunk) sums its chunk for 64 columns (four waves take every fourth row, combined in LDS) into
// tmp_j[chunk][c]. Level 1 sums the chunks: out_j[c] = scale_j * sum over chunks.
constexpr int COLSUM_CHUNKS = 16;

__global__ __launch_bounds__(256) void colsum_multi_kernel(ColsumJobs J, int level) {
  __shared__ float sh[4][64];
  int j = 0;
  while (j + 1 < J.n && (int)blockIdx.x >= J.job[j + 1].blk0) ++j;
  const ColsumJob &b = J.job[j];
  const int lane = threadIdx.x & 63, grp = threadIdx.x >> 6;
  const int c = ((int)blockIdx.x - b.blk0) * 64 + lane;
  const float *part = level == 0 ? b.part : b.tmp;
  const int n_part = level == 0 ? b.n_part : COLSUM_CHUNKS;
  const int chunk = level == 0 ? (b.n_part + COLSUM_CHUNKS - 1) / COLSUM_CHUNKS : COLSUM_CHUNKS;
  const int p0 = blockIdx.y * chunk, p1 = min(p0 + chunk, n_part);
  float acc = 0.f;
  if (c < b.n)
    for (int p = p0 + grp; p < p1; p += 4) acc += part[(int64_t)p * b.n + c];
  sh[grp][lane] = acc;
  __syncthreads();
  if (grp == 0 && c < b.n) {
    const float v = ((sh[0][lane] + sh[1][lane]) + sh[2][lane]) + sh[3][lane];
    if (level == 0) b.tmp[(int64_t)blockIdx.y * b.n + c] = v;
    else b.out[c] = b.scale * v;
  }
}

hipError_t launch_colsum_multi(ColsumJobs J, hipStream_t s) {
  int blocks = 0;
  for (int j = 0; j < J.n; ++j) {
    J.job[j].blk0 = blocks;
    blocks += (J.job[j].n + 63) / 64;
  }
  hipLaunchKernelGGL(colsum_multi_kernel, dim3(blocks, COLSUM_CHUNKS), dim3(256), 0, s, J, 0);
  hipLaunchKernelGGL(colsum_multi_kernel, dim3(blocks, 1), dim3(256), 0, s, J, 1);
  return hipGetLastError();
}

int bwd_row_wgs() { return BWD_ROW_WGS; }
int bwd_route_wgs() { return BWD_ROUTE_WGS; }

static int ni_of(int d) { return ((d >> 3) + 63) / 64; }

#define XMOD_BWD_NI_SWITCH(ni, MACRO) \
  switch (ni) {                       \
    case 1: MACRO(1); break;          \
    case 2: MACRO(2); break;          \
    case 3: MACRO(3); break;          \
    case 4: MACRO(4); break;          \
    case 5: case 6: MACRO(6); break;  \
    case 7: case 8: MACRO(8); break;  \
    default: MACRO(16); break;        \
  }

hipError_t launch_resid_bwd(const uint16_t *dy, const RowMap &map, const float *a, const float *f,
                            const float *gate, float varsigma, int d, int64_t M, int64_t M_pad,
                            uint16_t *dt, float *dell, float *dell_tok, uint8_t *q_tok,
                            float *vs_part, hipStream_t s) {
#define L_(NI)                                                                                  \
  hipLaunchKernelGGL((resid_bwd_kernel<NI>), dim3(BWD_ROW_WGS), dim3(256), 0, s, dy, map, a, f, \
                     gate, varsigma, d, M, M_pad, dt, dell, dell_tok, q_tok, vs_part)
  XMOD_BWD_NI_SWITCH(ni_of(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_rms2_bwd(const uint16_t *dy, const RowMap &map, const uint16_t *X,
                           const float *a, const float *dv, const uint16_t *gain, float eps,
                           const uint16_t *dt, int d, int64_t M, int64_t M_pad, uint16_t *da,
                           float *dXacc, float *g_part, hipStream_t s) {
#define L_(NI)                                                                                \
  hipLaunchKernelGGL((rms2_bwd_kernel<NI>), dim3(BWD_ROW_WGS), dim3(256), 0, s, dy, map, X, a, \
                     dv, gain, eps, dt, d, M, M_pad, da, dXacc, g_part)
  XMOD_BWD_NI_SWITCH(ni_of(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_rms1_bwd(const uint16_t *X, const RowMap &map, const float *du,
                           const uint16_t *gain, float eps, const float *dXacc,
                           const float *s_tok, const float *dell, float coef_n,
                           const uint16_t *w_r, int d, int64_t M, uint16_t *dx, float *g_part,
                           float *wr_part, hipStream_t s) {
#define L_(NI)                                                                                 \
  hipLaunchKernelGGL((rms1_bwd_kernel<NI>), dim3(BWD_ROW_WGS), dim3(256), 0, s, X, map, du, gain, \
                     eps, dXacc, s_tok, dell, coef_n, w_r, d, M, dx, g_part, wr_part)
  XMOD_BWD_NI_SWITCH(ni_of(d), L_)
#undef L_
  return hipGetLastError();
}

hipError_t launch_route_bwd(const uint16_t *x, const uint16_t *dy, const float *s_tok,
                            const float *dell_tok, const uint8_t *q_tok, float coef_n,
                            const uint16_t *w_r, int d, int64_t rows, uint16_t *dx,
                            float *wr_part, float *beta_part, float *loss_part, hipStream_t s) {
#define L_(NI)                                                                                \
  hipLaunchKernelGGL((route_bwd_kernel<NI>), dim3(BWD_ROUTE_WGS), dim3(256), 0, s, x, dy, s_tok, \
                     dell_tok, q_tok, coef_n, w_r, d, rows, dx, wr_part, beta_part, loss_part)
  XMOD_BWD_NI_SWITCH(ni_of(d), L_)
#undef L_
  return hipGetLastError();
}

}  // namespace xmod
