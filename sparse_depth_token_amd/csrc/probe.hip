// Ceiling probes for the measurement: what this part sustains on the two kinds of work the
// layer's kernels are bound by, measured in the same run as the layer, beside the vendor peaks.
//  * MFMA: every wave issues independent v_mfma_f32_32x32x16_bf16 back to back (four
//    accumulators, no memory traffic in the loop).
//  * HBM read: a grid-stride pass of 16-byte loads over a buffer, 4, 8 or 16 of them in flight
//    per thread, every 32-bit word added into a per-thread sum (kept, so that nothing is
//    skipped; the sums are checkable on the host).
//  * HBM read, chunked: every workgroup reads its own contiguous share of the buffer with
//    non-temporal 16-byte loads (the nt bit: the caches do not keep the lines), four 4 KB
//    blocks of the share in flight per workgroup. This is the faster way to stream a buffer
//    larger than the last-level cache; the grid-stride form is the one a cache flush uses,
//    since its lines do displace what the caches held.
#include "common.h"

namespace xmod {

// PROBE_WGS workgroups of 256 threads (4 per CU, one wave per SIMD each), out[PROBE_WGS * 256]
constexpr int PROBE_WGS = 1024;

__global__ __launch_bounds__(256) void probe_mfma_kernel(float *__restrict__ out, int iters) {
  // all-ones operands: every MFMA adds 16 to each accumulator element (exact below 2^24)
  bf16x8 a, b;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    a[e] = (__bf16)1.0f;
    b[e] = (__bf16)1.0f;
  }
  f32x16 acc[4];
#pragma unroll
  for (int t = 0; t < 4; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[t][e] = 0.f;
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[t], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) s += acc[t][0];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// D independent 16-byte loads in flight per thread (1024 threads per CU: 16 D KB per CU)
template <int D>
__global__ __launch_bounds__(256) void probe_read_kernel(const uint4 *__restrict__ src, int64_t n16,
                                                         uint32_t *__restrict__ out) {
  uint32_t s = 0;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  for (; i + (D - 1) * stride < n16; i += D * stride) {
    uint4 v[D];
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] = src[i + j * stride];
#pragma unroll
    for (int j = 0; j < D; ++j) s += v[j].x + v[j].y + v[j].z + v[j].w;
  }
  for (; i < n16; i += stride) {
    const uint4 v = src[i];
    s += v.x + v.y + v.z + v.w;
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(256) void probe_read_chunked_kernel(const uint4 *__restrict__ src,
                                                                 int64_t n16,
                                                                 uint32_t *__restrict__ out) {
  constexpr int D = 4;
  const probe_u32x4 *p = (const probe_u32x4 *)src;
  const int64_t per = (n16 + gridDim.x - 1) / gridDim.x;
  const int64_t lo = (int64_t)blockIdx.x * per;
  const int64_t hi = lo + per < n16 ? lo + per : n16;
  uint32_t s = 0;
  int64_t i = lo + threadIdx.x;
  for (; i + (D - 1) * 256 < hi; i += D * 256) {
    probe_u32x4 v[D];
#pragma unroll
    for (int j = 0; j < D; ++j) v[j] = __builtin_nontemporal_load(p + i + j * 256);
#pragma unroll
    for (int j = 0; j < D; ++j) s += v[j][0] + v[j][1] + v[j][2] + v[j][3];
  }
  for (; i < hi; i += 256) {
    const probe_u32x4 v = __builtin_nontemporal_load(p + i);
    s += v[0] + v[1] + v[2] + v[3];
  }
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

hipError_t launch_probe_mfma(float *out, int iters, hipStream_t s) {
  hipLaunchKernelGGL(probe_mfma_kernel, dim3(PROBE_WGS), dim3(256), 0, s, out, iters);
  return hipGetLastError();
}

hipError_t launch_probe_read(const void *src, size_t bytes, int depth, uint32_t *out,
                             hipStream_t s) {
  const uint4 *p = (const uint4 *)src;
  const int64_t n16 = (int64_t)(bytes / 16);
  if (depth == 16)
    hipLaunchKernelGGL(probe_read_kernel<16>, dim3(PROBE_WGS), dim3(256), 0, s, p, n16, out);
  else if (depth == 8)
    hipLaunchKernelGGL(probe_read_kernel<8>, dim3(PROBE_WGS), dim3(256), 0, s, p, n16, out);
  else
    hipLaunchKernelGGL(probe_read_kernel<4>, dim3(PROBE_WGS), dim3(256), 0, s, p, n16, out);
  return hipGetLastError();
}

hipError_t launch_probe_read_chunked(const void *src, size_t bytes, uint32_t *out, hipStream_t s) {
  hipLaunchKernelGGL(probe_read_chunked_kernel, dim3(PROBE_WGS), dim3(256), 0, s,
                     (const uint4 *)src, (int64_t)(bytes / 16), out);
  return hipGetLastError();
}

}  // namespace xmod
