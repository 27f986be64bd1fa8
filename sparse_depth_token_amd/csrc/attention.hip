// Causal attention over the packed selected rows of each sequence (gfx950, MFMA bf16).
//
// The X-MoD review's Table 7 gives a sparse layer's KV context as the selected subset: packed
// row j of a sequence attends to packed rows 0..j only. Query head h reads KV head
// floor(h * Hkv / Hq) (the grouped-query mapping of the MoDA notes' section 2.1, written
// 0-based). Softmax uses the scale 1/sqrt(head_dim) and the usual online recurrence (running
// max, rescaled running sum and output), so the k x k score matrix is never stored.
//
// Work split: one workgroup = (q-tile of 128 packed rows, query head, sequence); its 4 waves
// own 32 query rows each. Key/value tiles of 64 rows are staged in LDS: K row-major (padded),
// V transposed (hd rows of 64 keys, padded) so that the P*V product reads 8 keys of one hd row
// per lane. Scores are computed transposed, S^T = K Q^T, so that each lane holds one query's
// scores: lane l owns query l % 32 and keys 8(e/4) + 4(l/32) + e%4 of each 32-key block. The
// same lane then holds query l % 32 of O^T = V^T P^T, so the softmax statistics never leave
// the lane pair (l, l ^ 32). The P fragment is fed as the second MFMA operand in the key
// order the score accumulator already has; V^T is read in that same key order.
#include "common.h"

namespace xmod {

template <int HD>
__global__ __launch_bounds__(256) void attn_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                   uint16_t *__restrict__ o, int ldo, int k,
                                                   int Hq, int Hkv, float scale_log2) {
  constexpr int BQ = 128, BKV = 64, KS = HD / 16, NT_HD = HD / 32;
  constexpr int KROW = HD + 8;   // K tile row stride (elements)
  constexpr int VROW = BKV + 4;  // V^T row stride (elements)
  __shared__ __attribute__((aligned(16))) uint16_t Ks[BKV * KROW];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[HD * VROW];

  const int nqt = (k + BQ - 1) / BQ;
  const int qt = nqt - 1 - (int)blockIdx.x;  // longest (latest) q-tiles first
  const int h = blockIdx.y, b = blockIdx.z;
  const int gkv = (h * Hkv) / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int gq = lane >> 5, r32 = lane & 31;
  const int q_pos = qt * BQ + wid * 32 + r32;
  const int64_t row0 = (int64_t)b * k;

  bf16x8 qf[KS];
  {
    const int qr = min(q_pos, k - 1);
    const uint16_t *qp = qkv + (row0 + qr) * ldq + h * HD + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) qf[s] = *(const bf16x8 *)(qp + s * 16);
  }
  f32x16 oacc[NT_HD];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) oacc[t][e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;

  const int q_hi = min(qt * BQ + BQ, k);
  const int n_kv = (q_hi + BKV - 1) / BKV;
  const uint16_t *kbase = qkv + row0 * ldq + Hq * HD + gkv * HD;
  const uint16_t *vbase = kbase + Hkv * HD;

#pragma unroll 1
  for (int jt = 0; jt < n_kv; ++jt) {
    const int key0 = jt * BKV;
    __syncthreads();
    // K tile: 64 keys x HD, 16-byte chunks
#pragma unroll
    for (int c = tid; c < BKV * HD / 8; c += 256) {
      const int r = c / (HD / 8), ch = c % (HD / 8);
      const int key = min(key0 + r, k - 1);
      *(uint4 *)(Ks + r * KROW + ch * 8) = *(const uint4 *)(kbase + (int64_t)key * ldq + ch * 8);
    }
    // V tile transposed: a thread takes two adjacent keys x 8 hd and writes 8 key pairs.
#pragma unroll
    for (int c = tid; c < (BKV / 2) * (HD / 8); c += 256) {
      const int rp = c / (HD / 8), ch = c % (HD / 8);
      const int k0 = min(key0 + 2 * rp, k - 1), k1 = min(key0 + 2 * rp + 1, k - 1);
      const uint4 v0 = *(const uint4 *)(vbase + (int64_t)k0 * ldq + ch * 8);
      const uint4 v1 = *(const uint4 *)(vbase + (int64_t)k1 * ldq + ch * 8);
      const uint32_t a0[4] = {v0.x, v0.y, v0.z, v0.w}, a1[4] = {v1.x, v1.y, v1.z, v1.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t lo = (a0[e] & 0xFFFFu) | (a1[e] << 16);
        const uint32_t hi = (a0[e] >> 16) | (a1[e] & 0xFFFF0000u);
        *(uint32_t *)(Vt + (ch * 8 + 2 * e) * VROW + 2 * rp) = lo;
        *(uint32_t *)(Vt + (ch * 8 + 2 * e + 1) * VROW + 2 * rp) = hi;
      }
    }
    __syncthreads();

    // S^T[key, query] for 64 keys x this wave's 32 queries
    f32x16 sacc[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
#pragma unroll
      for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 kf = *(const bf16x8 *)(Ks + (t * 32 + r32) * KROW + s * 16 + gq * 8);
        sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
      }
    }
    // causal mask and online softmax (statistics shared by lanes l and l^32)
    float mt = -INFINITY;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = key0 + t * 32 + 8 * (e >> 2) + 4 * gq + (e & 3);
        if (key > q_pos || key >= k) sacc[t][e] = -INFINITY;
        mt = fmaxf(mt, sacc[t][e]);
      }
    mt = fmaxf(mt, __shfl_xor(mt, 32, 64));
    const float m_new = fmaxf(m_run, mt);
    const float corr = exp2f((m_run - m_new) * scale_log2);
    const float mb = m_new * scale_log2;
    float psum = 0.f;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float p = exp2f(fmaf(sacc[t][e], scale_log2, -mb));
        sacc[t][e] = p;
        psum += p;
      }
    l_run = l_run * corr + psum;
    m_run = m_new;
#pragma unroll
    for (int t = 0; t < NT_HD; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) oacc[t][e] *= corr;

    // O^T[hd, query] += V^T[hd, key] P^T[key, query], 16 keys per MFMA
#pragma unroll
    for (int s = 0; s < BKV / 16; ++s) {
      bf16x8 pf;
#pragma unroll
      for (int j = 0; j < 8; ++j) pf[j] = (__bf16)sacc[s >> 1][8 * (s & 1) + j];
#pragma unroll
      for (int t = 0; t < NT_HD; ++t) {
        const uint16_t *vr = Vt + (t * 32 + r32) * VROW + 16 * s + 4 * gq;
        const uint2 lo = *(const uint2 *)vr;
        const uint2 hi = *(const uint2 *)(vr + 8);
        const uint4 vv = make_uint4(lo.x, lo.y, hi.x, hi.y);
        bf16x8 vf;
        __builtin_memcpy(&vf, &vv, 16);
        oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[t], 0, 0, 0);
      }
    }
  }

  const float l_tot = l_run + __shfl_xor(l_run, 32, 64);
  const float inv = 1.0f / l_tot;
  if (q_pos < k) {
    uint16_t *op = o + (row0 + q_pos) * ldo + h * HD;
#pragma unroll
    for (int t = 0; t < NT_HD; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int hd = t * 32 + 8 * q4 + 4 * gq;
        *(uint2 *)(op + hd) = make_uint2(pack_bf16x2(oacc[t][4 * q4] * inv, oacc[t][4 * q4 + 1] * inv),
                                         pack_bf16x2(oacc[t][4 * q4 + 2] * inv, oacc[t][4 * q4 + 3] * inv));
      }
  }
}

hipError_t launch_attention(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, int B, int k,
                            int Hq, int Hkv, int hd, hipStream_t s) {
  const dim3 grid((unsigned)((k + 127) / 128), (unsigned)Hq, (unsigned)B);
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
  if (hd == 128)
    hipLaunchKernelGGL((attn_kernel<128>), grid, dim3(256), 0, s, qkv, ld_qkv, o, ld_o, k, Hq, Hkv,
                       scale_log2);
  else
    hipLaunchKernelGGL((attn_kernel<64>), grid, dim3(256), 0, s, qkv, ld_qkv, o, ld_o, k, Hq, Hkv,
                       scale_log2);
  return hipGetLastError();
}

}  // namespace xmod
