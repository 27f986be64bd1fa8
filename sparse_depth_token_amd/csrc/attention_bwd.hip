// Backward of the causal attention over the packed selected rows (gfx950, MFMA bf16).
//
// The forward (attention.hip) computes, per sequence, query head h and its key/value head g,
// S = Q K^T over the packed rows (key j visible to query q when j <= q), P = softmax(S / sqrt(hd))
// and O = P V, and saves lse_q = log2 of the softmax normaliser in the units of its weights, so
// P[q][j] = exp2(S[q][j] * scale_log2 - lse_q). The gradients for an output gradient dO are
//   D_q = sum_i dO[q][i] O[q][i]                         (one number per query and head)
//   dP = dO V^T,  dS = P * (dP - D_q)
//   dQ = scale * dS K,  dK = scale * dS^T Q,  dV = P^T dO,    scale = 1/sqrt(hd),
// with dK and dV summed over the query heads that share a key/value head (grouped-query
// attention). Two kernels, no atomics:
//  * dQ: one wave per 32 queries, the forward's layout (the lane owns a query and 16 scores of
//    each 32-key block); key/value tiles of 64 rows stream through a two-stage LDS ring. A
//    workgroup's 256 queries are one tile of 256 rows (latest tiles dispatched first) when the
//    grid holds more workgroups than CUs, so both waves of every SIMD stay busy to the last key
//    tile; else an early and a late tile of 128 rows, so every workgroup has the same causal
//    work and the longest one holds half as many long rows.
//  * dK/dV: one wave per 32 keys (the lane owns a key and 16 scores of each 32-query block); the
//    wave's key and value fragments stay in registers while query and dO tiles of 64 rows (with
//    their lse and D) stream through the ring, over every query head of the group.
// P and dS enter the matrix cores as bf16, as in the forward; accumulation is fp32.
//
// Tiles that are read both row-wise (ds_read_b128: 16 consecutive rows, one 16-byte chunk) and
// transposed (ds_read_b64_tr_b16: per half-wave 4 consecutive rows x 4 consecutive chunks) keep
// their chunks XOR-swizzled so that both patterns hit distinct banks.
#include "common.h"

namespace xmod {

__device__ __forceinline__ void bwd_dma16(const void *gsrc, uint16_t *lds_block) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_block, 16,
                                   0, 0);
}

template <int HD>
struct BwdCfg {
  static constexpr int KS = HD / 16;     // 16-wide k-steps over hd
  static constexpr int NT_HD = HD / 32;  // 32-column blocks of hd
  static constexpr int CPR = HD / 8;     // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;   // rows per 1 KB DMA block
  // read row-wise and transposed: a bijection of the row's low bits for 16 consecutive rows,
  // and 4 consecutive rows x 4 consecutive chunks onto 16 distinct 16-byte bank slots
  static __device__ __forceinline__ int swz_rt(int r) {
    return HD == 128 ? 4 * (r & 3) + ((r >> 2) & 3) : 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
  }
  // read row-wise only
  static __device__ __forceinline__ int swz_r(int r) {
    return HD == 128 ? (r & 15) : ((r >> 1) & 7);
  }
};

// Transposing read of a 32-column x 16-row fragment half (4 rows) into 4 bf16 per lane. Issued
// as assembly: the compiler's own form of the read would wait for every pending DMA copy.
__device__ __forceinline__ u32x2 tr_read(uint32_t addr) {
  u32x2 v;
  asm volatile("ds_read_b64_tr_b16 %0, %1" : "=v"(v) : "v"(addr));
  return v;
}

__device__ __forceinline__ uint32_t lds_u32(const uint16_t *p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)p;
}

// Byte offset, within a tile of HD-element rows swizzled by swz_rt, that lane `lane` addresses
// as the source of the transposing read of (16-row step 0, 32-column block t, half hh): row
// 4 (g >> 1) + e + 8 hh, column 32 t + 16 (g & 1) + 4 a (g = lane / 16, e = lane / 4 % 4,
// a = lane % 4). The reader receives column 32 t + lane % 32 and rows 16 s + 4 (lane / 32) +
// (0..3, or 8..11 for hh = 1), the row order of a score accumulator's 16-wide fragment.
template <int HD>
__device__ __forceinline__ uint32_t tr_offset(int lane, int t, int hh) {
  const int g = lane >> 4, e = (lane >> 2) & 3, a = lane & 3;
  const int row = 4 * (g >> 1) + e + 8 * hh;
  const int col = 32 * t + 16 * (g & 1) + 4 * a;
  const int phys = (col >> 3) ^ BwdCfg<HD>::swz_rt(row);
  return 2u * (uint32_t)(row * HD + (phys << 3) + (col & 7));
}

// D[row][h] = sum over the head's hd columns of dO * O (fp32). One wave per row.
template <int HD>
__global__ __launch_bounds__(256) void attn_bwd_delta_kernel(const uint16_t *__restrict__ o,
                                                             int ldo, const uint16_t *__restrict__ dO,
                                                             int lddo, float *__restrict__ D,
                                                             int64_t rows, int Hq) {
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;
  const int lane = threadIdx.x & 63;
  const int dq = Hq * HD;
  for (int c0 = 0; c0 < dq; c0 += 512) {
    const int c = c0 + lane * 8;
    float acc = 0.f;
    if (c < dq) {
      float a[8], b[8];
      unpack8(*(const uint4 *)(o + row * ldo + c), a);
      unpack8(*(const uint4 *)(dO + row * lddo + c), b);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf(a[e], b[e], acc);
    }
    // the HD / 8 lanes of one head are aligned (512 is a multiple of HD)
#pragma unroll
    for (int off = HD / 16; off > 0; off >>= 1) acc += __shfl_xor(acc, off, 64);
    if (c < dq && (lane & (HD / 8 - 1)) == 0) D[row * Hq + c / HD] = acc;
  }
}

// Writes a wave's 32 rows x HD accumulator block (lane: row r32, columns 32 t + 8 q4 + 4 gq +
// 0..3 in element 4 q4 + 0..3 of acc[t]) times `mul` as bf16 rows dst + r * ld, for rows r with
// r0 + r < r_end, staged through the wave's 32 x HD slice of LDS.
template <int HD>
__device__ __forceinline__ void store_rows(const f32x16 *acc, float mul, uint16_t *ow, int lane,
                                           uint16_t *dst, int64_t ld, int r0, int r_end) {
  constexpr int CPR = HD / 8, NT_HD = HD / 32;
  const int r32 = lane & 31, gq = lane >> 5;
#pragma unroll
  for (int t = 0; t < NT_HD; ++t)
#pragma unroll
    for (int q4 = 0; q4 < 4; ++q4) {
      const int c = 4 * t + q4;
      *(uint2 *)(ow + r32 * HD + ((c ^ (r32 & (CPR - 1))) * 8) + 4 * gq) =
          make_uint2(pack_bf16x2(acc[t][4 * q4] * mul, acc[t][4 * q4 + 1] * mul),
                     pack_bf16x2(acc[t][4 * q4 + 2] * mul, acc[t][4 * q4 + 3] * mul));
    }
  constexpr int RPI = 64 / CPR;  // rows per store instruction
#pragma unroll
  for (int i = 0; i < 32 / RPI; ++i) {
    const int r = RPI * i + lane / CPR, c = lane % CPR;
    const uint4 v = *(const uint4 *)(ow + r * HD + ((c ^ (r & (CPR - 1))) * 8));
    if (r0 + r < r_end) *(uint4 *)(dst + (int64_t)r * ld + c * 8) = v;
  }
}

// ---- dQ ----------------------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(512, 1) void attn_bwd_dq_kernel(
    const uint16_t *__restrict__ qkv, int ldq, const uint16_t *__restrict__ dO, int lddo,
    const float *__restrict__ lse, const float *__restrict__ Dl, uint16_t *__restrict__ dqkv,
    int ldd, int k, int Hq, int Hkv, float scale_log2, float scale, int paired) {
  using C = BwdCfg<HD>;
  constexpr int BQ = 256, BQP = 128, BKV = 64, KS = C::KS, NT_HD = C::NT_HD;
  constexpr int TILE = BKV * HD, STAGE = 2 * TILE;       // K tile, then V tile
  constexpr int NBLK = 2 * TILE * 2 / 1024, NDMA = NBLK / 8;
  static_assert(NBLK % 8 == 0, "DMA blocks split over the eight waves");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];

  const int h = blockIdx.x, b = blockIdx.y, u = blockIdx.z;
  const int64_t row0 = (int64_t)b * k;
  const int gkv = (h * Hkv) / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int gq = lane >> 5, r32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  // this wave's first query, whether it has a share, and the workgroup's last query + 1
  int q_first, key_hi;
  bool active;
  if (paired) {
    const int nqt = (k + BQP - 1) / BQP, qt_hi = nqt - 1 - u;
    const bool later = wid < 4;
    q_first = (later ? qt_hi : u) * BQP + (wid & 3) * 32;
    active = later || u != qt_hi;  // the middle tile of an odd count: waves 0-3 only
    key_hi = min(qt_hi * BQP + BQP, k);
  } else {
    const int qt = (k + BQ - 1) / BQ - 1 - u;
    q_first = qt * BQ + wid * 32;
    active = true;
    key_hi = min(qt * BQ + BQ, k);
  }
  active = active && q_first < k;  // a ragged last tile leaves later waves empty
  const int q_pos = q_first + r32;
  const int q_last = active ? q_first + 31 : -1;
  const int n_kv = (key_hi + BKV - 1) / BKV;
  const char *kbase = (const char *)(qkv + row0 * ldq + Hq * HD + gkv * HD);
  const char *vbase = kbase + (size_t)Hkv * HD * 2;

  // DMA: block i (< NBLK / 2: K, else V) by wave i % 8; lane l lands at row RPB * blk + l / CPR,
  // physical chunk l % CPR; rows past the sequence read its last row.
  auto issue_tile = [&](int jt, int stage) {
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int i = 8 * n + wv;
      const bool is_v = i >= NBLK / 2;
      const int blk = is_v ? i - NBLK / 2 : i;
      const int row = C::RPB * blk + lane / C::CPR;
      const int lc = (lane % C::CPR) ^ (is_v ? C::swz_r(row) : C::swz_rt(row));
      const int grow = min(jt * BKV + row, k - 1);
      bwd_dma16((is_v ? vbase : kbase) + (size_t)grow * ldq * 2 + lc * 16,
                lds + stage + (is_v ? TILE : 0) + C::RPB * blk * HD);
    }
  };
  issue_tile(0, 0);

  // this lane's query: Q and dO fragments (8 consecutive hd per k-step), lse and D
  bf16x8 qf[KS], dof[KS];
  const int qr = min(q_pos, k - 1);
  {
    const uint16_t *qp = qkv + (row0 + qr) * ldq + h * HD + gq * 8;
    const uint16_t *dp = dO + (row0 + qr) * lddo + h * HD + gq * 8;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      qf[s] = *(const bf16x8 *)(qp + s * 16);
      dof[s] = *(const bf16x8 *)(dp + s * 16);
    }
  }
  const float lse_q = lse[(row0 + qr) * Hq + h], d_q = Dl[(row0 + qr) * Hq + h];
  f32x16 dqacc[NT_HD];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) dqacc[t][e] = 0.f;

  // row-wise fragment offsets (elements): row 32 t + r32, logical chunk 2 s + gq
  int k_off[KS], v_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    k_off[s] = r32 * HD + (((2 * s + gq) ^ C::swz_rt(r32)) << 3);
    v_off[s] = TILE + r32 * HD + (((2 * s + gq) ^ C::swz_r(r32)) << 3);
  }
  uint32_t kt_off[NT_HD][2];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t) {
    kt_off[t][0] = tr_offset<HD>(lane, t, 0);
    kt_off[t][1] = tr_offset<HD>(lane, t, 1);
  }
  const uint32_t lds_base = lds_u32(lds);

  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

#pragma unroll 1
  for (int jt = 0; jt < n_kv; ++jt) {
    const int st = (jt & 1) * STAGE;
    if (jt + 1 < n_kv) issue_tile(jt + 1, STAGE - st);
    const uint16_t *Ks = lds + st;
    const int key0 = jt * BKV;
    if (key0 <= q_last) {
      // S^T and dP^T for 64 keys x this wave's 32 queries (K and V fragments first)
      f32x16 sacc[2], dpacc[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) { sacc[t][e] = 0.f; dpacc[t][e] = 0.f; }
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          const bf16x8 kf = *(const bf16x8 *)(Ks + t * 32 * HD + k_off[s]);
          const bf16x8 vf = *(const bf16x8 *)(Ks + t * 32 * HD + v_off[s]);
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[s], sacc[t], 0, 0, 0);
          dpacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, dof[s], dpacc[t], 0, 0, 0);
        }
      }
      // P and dS (keys past the query or the sequence: P = 0)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = key0 + t * 32 + 8 * (e >> 2) + 4 * gq + (e & 3);
          const float pv = (key > q_pos || key >= k)
                               ? 0.f
                               : __builtin_amdgcn_exp2f(fmaf(sacc[t][e], scale_log2, -lse_q));
          sacc[t][e] = pv * (dpacc[t][e] - d_q);
        }
      // dQ^T[hd, query] += K^T[hd, key] dS^T[key, query], 16 keys per MFMA
      const uint32_t kst = lds_base + 2u * (uint32_t)st;
#pragma unroll
      for (int s = 0; s < BKV / 16; ++s) {
        u32x2 kr[NT_HD][2];
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          kr[t][0] = tr_read(kst + kt_off[t][0] + 2u * 16u * HD * s);
          kr[t][1] = tr_read(kst + kt_off[t][1] + 2u * 16u * HD * s);
        }
        bf16x8 dsf;
#pragma unroll
        for (int j = 0; j < 8; ++j) dsf[j] = (__bf16)sacc[s >> 1][8 * (s & 1) + j];
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          asm volatile("" : "+v"(kr[t][0]), "+v"(kr[t][1]));
          bf16x8 kf;
          __builtin_memcpy(&kf, &kr[t][0], 8);
          __builtin_memcpy((char *)&kf + 8, &kr[t][1], 8);
          dqacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, dsf, dqacc[t], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // this wave's copies landed
    __syncthreads();
  }

  if (active)
    store_rows<HD>(dqacc, scale, lds + wid * 32 * HD, lane,
                   dqkv + (row0 + q_first) * ldd + h * HD, ldd, q_first, k);
}

// ---- dK and dV ---------------------------------------------------------------------------------
template <int HD>
__global__ __launch_bounds__(256, 1) void attn_bwd_dkdv_kernel(
    const uint16_t *__restrict__ qkv, int ldq, const uint16_t *__restrict__ dO, int lddo,
    const float *__restrict__ lse, const float *__restrict__ Dl, uint16_t *__restrict__ dqkv,
    int ldd, int k, int Hq, int Hkv, float scale_log2, float scale) {
  using C = BwdCfg<HD>;
  constexpr int BKEY = 128, BQ = 64, KS = C::KS, NT_HD = C::NT_HD;
  constexpr int TILE = BQ * HD;                   // Q tile, then dO tile
  constexpr int STAGE = 2 * TILE + 4 * BQ;        // + lse and D (BQ floats each)
  constexpr int NBLK = 2 * TILE * 2 / 1024, NDMA = NBLK / 4;
  static_assert(NBLK % 4 == 0, "DMA blocks split over the four waves");
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * STAGE];

  const int g = blockIdx.x, b = blockIdx.y, kb = blockIdx.z;
  const int G = Hq / Hkv;
  const int64_t row0 = (int64_t)b * k;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int gq = lane >> 5, r32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int key_w = kb * BKEY + wid * 32;  // this wave's first key
  const int key = key_w + r32;             // this lane's key
  const int nqt = (k + BQ - 1) / BQ;
  const int qt0 = (kb * BKEY) / BQ;        // first query tile that sees the block's keys
  const int n_qt = nqt - qt0;
  const int n_it = G * n_qt;               // (head, query tile) steps

  auto issue_tile = [&](int it, int stage) {
    const int hq = g * G + it / n_qt, qt = qt0 + it % n_qt;
    const char *qb = (const char *)(qkv + row0 * ldq + hq * HD);
    const char *db = (const char *)(dO + row0 * lddo + hq * HD);
#pragma unroll
    for (int n = 0; n < NDMA; ++n) {
      const int i = 4 * n + wv;
      const bool is_d = i >= NBLK / 2;
      const int blk = is_d ? i - NBLK / 2 : i;
      const int row = C::RPB * blk + lane / C::CPR;
      const int lc = (lane % C::CPR) ^ C::swz_rt(row);
      const int grow = min(qt * BQ + row, k - 1);
      bwd_dma16((is_d ? db + (size_t)grow * lddo * 2 : qb + (size_t)grow * ldq * 2) + lc * 16,
                lds + stage + (is_d ? TILE : 0) + C::RPB * blk * HD);
    }
  };
  // lse and D of a step's BQ queries: loaded by threads < BQ, written to LDS a step later
  auto load_stats = [&](int it, float &lv, float &dv) {
    const int hq = g * G + it / n_qt, qt = qt0 + it % n_qt;
    const int q = min(qt * BQ + tid, k - 1);
    lv = lse[(row0 + q) * Hq + hq];
    dv = Dl[(row0 + q) * Hq + hq];
  };
  auto put_stats = [&](int stage, float lv, float dv) {
    float *f = (float *)(lds + stage + 2 * TILE);
    f[tid] = lv;
    f[BQ + tid] = dv;
  };

  // this lane's key: K and V fragments (8 consecutive hd per k-step)
  bf16x8 kf[KS], vf[KS];
  {
    const int kr = min(key, k - 1);
    const uint16_t *kp = qkv + (row0 + kr) * ldq + Hq * HD + g * HD + gq * 8;
    const uint16_t *vp = kp + Hkv * HD;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      kf[s] = *(const bf16x8 *)(kp + s * 16);
      vf[s] = *(const bf16x8 *)(vp + s * 16);
    }
  }
  f32x16 dk[NT_HD], dv[NT_HD];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t)
#pragma unroll
    for (int e = 0; e < 16; ++e) { dk[t][e] = 0.f; dv[t][e] = 0.f; }

  int q_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) q_off[s] = r32 * HD + (((2 * s + gq) ^ C::swz_rt(r32)) << 3);
  uint32_t t_off[NT_HD][2];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t) {
    t_off[t][0] = tr_offset<HD>(lane, t, 0);
    t_off[t][1] = tr_offset<HD>(lane, t, 1);
  }
  const uint32_t lds_base = lds_u32(lds);

  float lv = 0.f, dvl = 0.f;
  issue_tile(0, 0);
  if (tid < BQ) load_stats(0, lv, dvl);
  __builtin_amdgcn_s_waitcnt(0);
  if (tid < BQ) put_stats(0, lv, dvl);
  __syncthreads();

#pragma unroll 1
  for (int it = 0; it < n_it; ++it) {
    const int st = (it & 1) * STAGE;
    if (it + 1 < n_it) {
      issue_tile(it + 1, STAGE - st);
      if (tid < BQ) load_stats(it + 1, lv, dvl);
    }
    const int qt = qt0 + it % n_qt;
    const uint16_t *Qs = lds + st;
    const uint16_t *Ds = lds + st + TILE;
    const float *stats = (const float *)(lds + st + 2 * TILE);
#pragma unroll
    for (int u = 0; u < BQ / 32; ++u) {
      const int q_lo = qt * BQ + 32 * u;
      // queries all before this wave's keys, or past the sequence, or keys past it: nothing
      if (q_lo + 31 < key_w || q_lo >= k || key_w >= k) continue;
      // S and dP for 32 queries x this wave's 32 keys (query fragments first)
      f32x16 sacc, dpacc;
#pragma unroll
      for (int e = 0; e < 16; ++e) { sacc[e] = 0.f; dpacc[e] = 0.f; }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        const bf16x8 qfr = *(const bf16x8 *)(Qs + u * 32 * HD + q_off[s]);
        const bf16x8 dfr = *(const bf16x8 *)(Ds + u * 32 * HD + q_off[s]);
        sacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qfr, kf[s], sacc, 0, 0, 0);
        dpacc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dfr, vf[s], dpacc, 0, 0, 0);
      }
      // lse and D of the lane's 16 queries 8 (e / 4) + 4 gq + e % 4
      f32x4 l4[4], d4[4];
#pragma unroll
      for (int e4 = 0; e4 < 4; ++e4) {
        l4[e4] = *(const f32x4 *)(stats + 32 * u + 8 * e4 + 4 * gq);
        d4[e4] = *(const f32x4 *)(stats + BQ + 32 * u + 8 * e4 + 4 * gq);
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int q = q_lo + 8 * (e >> 2) + 4 * gq + (e & 3);
        const float pv = (q < key || q >= k)
                             ? 0.f
                             : __builtin_amdgcn_exp2f(fmaf(sacc[e], scale_log2, -l4[e >> 2][e & 3]));
        dpacc[e] = pv * (dpacc[e] - d4[e >> 2][e & 3]);
        sacc[e] = pv;
      }
      // dV^T[hd, key] += dO^T[hd, q] P[q, key];  dK^T[hd, key] += Q^T[hd, q] dS[q, key]
      const uint32_t qst = lds_base + 2u * (uint32_t)st;
#pragma unroll
      for (int s2 = 0; s2 < 2; ++s2) {
        const uint32_t row_b = 2u * (uint32_t)(16 * (2 * u + s2) * HD);
        u32x2 qr[NT_HD][2], dr[NT_HD][2];
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          qr[t][0] = tr_read(qst + t_off[t][0] + row_b);
          qr[t][1] = tr_read(qst + t_off[t][1] + row_b);
          dr[t][0] = tr_read(qst + 2u * TILE + t_off[t][0] + row_b);
          dr[t][1] = tr_read(qst + 2u * TILE + t_off[t][1] + row_b);
        }
        bf16x8 pf, dsf;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          pf[j] = (__bf16)sacc[8 * s2 + j];
          dsf[j] = (__bf16)dpacc[8 * s2 + j];
        }
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          asm volatile("" : "+v"(qr[t][0]), "+v"(qr[t][1]), "+v"(dr[t][0]), "+v"(dr[t][1]));
          bf16x8 qtf, dtf;
          __builtin_memcpy(&qtf, &qr[t][0], 8);
          __builtin_memcpy((char *)&qtf + 8, &qr[t][1], 8);
          __builtin_memcpy(&dtf, &dr[t][0], 8);
          __builtin_memcpy((char *)&dtf + 8, &dr[t][1], 8);
          dv[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(dtf, pf, dv[t], 0, 0, 0);
          dk[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtf, dsf, dk[t], 0, 0, 0);
        }
      }
    }
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));  // copies and stat loads
    if (it + 1 < n_it && tid < BQ) put_stats(STAGE - st, lv, dvl);
    __syncthreads();
  }

  // dK = scale * dK^T and dV = dV^T, one wave's 32 keys each (LDS ring free after the barrier)
  uint16_t *ow = lds + wid * 32 * HD;
  uint16_t *kdst = dqkv + (row0 + key_w) * ldd + Hq * HD + g * HD;
  store_rows<HD>(dk, scale, ow, lane, kdst, ldd, key_w, k);
  store_rows<HD>(dv, 1.0f, ow, lane, kdst + Hkv * HD, ldd, key_w, k);
}

hipError_t launch_attention_bwd(const uint16_t *qkv, int ld_qkv, const uint16_t *o, int ld_o,
                                const float *lse, const uint16_t *dO, int ld_do, float *D,
                                uint16_t *dqkv, int ld_dqkv, int B, int k, int Hq, int Hkv,
                                int hd, hipStream_t s) {
  const int64_t rows = (int64_t)B * k;
  const float scale = 1.0f / sqrtf((float)hd);
  const float scale_log2 = 1.4426950408889634f * scale;
  const dim3 g_delta((unsigned)((rows + 3) / 4));
  // dQ grid (head, sequence, unit), the unit slowest: 256-row q-tiles when there are more of
  // them than CUs, else pairs of 128-row tiles
  const int nqt = (k + 255) / 256;
  const int paired = (long)Hq * B * nqt <= 256;  // MI355X: 256 CUs
  const dim3 g_dq((unsigned)Hq, (unsigned)B, (unsigned)(paired ? ((k + 127) / 128 + 1) / 2 : nqt));
  // dK/dV grid (key/value head, sequence, key block), the key block slowest: the first key
  // blocks see the most queries, so every head's and sequence's longest workgroups go first
  const dim3 g_kv((unsigned)Hkv, (unsigned)B, (unsigned)((k + 127) / 128));
  if (hd == 128) {
    hipLaunchKernelGGL(attn_bwd_delta_kernel<128>, g_delta, dim3(256), 0, s, o, ld_o, dO, ld_do, D,
                       rows, Hq);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<128>, g_dq, dim3(512), 0, s, qkv, ld_qkv, dO, ld_do, lse,
                       D, dqkv, ld_dqkv, k, Hq, Hkv, scale_log2, scale, paired);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<128>, g_kv, dim3(256), 0, s, qkv, ld_qkv, dO, ld_do,
                       lse, D, dqkv, ld_dqkv, k, Hq, Hkv, scale_log2, scale);
  } else {
    hipLaunchKernelGGL(attn_bwd_delta_kernel<64>, g_delta, dim3(256), 0, s, o, ld_o, dO, ld_do, D,
                       rows, Hq);
    hipLaunchKernelGGL(attn_bwd_dq_kernel<64>, g_dq, dim3(512), 0, s, qkv, ld_qkv, dO, ld_do, lse,
                       D, dqkv, ld_dqkv, k, Hq, Hkv, scale_log2, scale, paired);
    hipLaunchKernelGGL(attn_bwd_dkdv_kernel<64>, g_kv, dim3(256), 0, s, qkv, ld_qkv, dO, ld_do,
                       lse, D, dqkv, ld_dqkv, k, Hq, Hkv, scale_log2, scale);
  }
  return hipGetLastError();
}

}  // namespace xmod
