// bf16 "NT" GEMM on CDNA4 matrix cores: C[M,N] = A[M,K] * B[N,K]^T, fp32 accumulation.
//
// Used for the four projections of the X-MoD layer on the packed selected rows: QKV, O
// (fp32 output), gate/up (SwiGLU fused into the epilogue) and down (gated residual + scatter
// into x fused into the epilogue). Both operands are K-contiguous rows, the natural operand
// layout of v_mfma_f32_32x32x16_bf16: every lane reads 8 consecutive bf16 (16 bytes) of a row.
//
// Design (gfx950, wave64):
//  * Workgroup tile BM x BN, BK = 64, four waves in a 2 x 2 grid, each computing a WM x WN
//    sub-tile as (WM/32) x (WN/32) MFMA 32x32x16 tiles (accumulators live in AGPRs). Larger
//    per-wave tiles cut LDS bytes per MFMA: 128x128 needs 512 B of fragments per MFMA.
//  * The weight fragment is the MFMA's first operand and the activation fragment its second,
//    so each lane ends with 4 consecutive output columns of one row.
//  * Software pipeline: the next k-tile is copied global -> LDS by the DMA form of the load
//    (global_load_lds_dwordx4: 16 bytes per lane, no staging registers) while the current tile
//    is multiplied; operand fragments are double-buffered in registers, so the LDS reads of
//    k-step s+1 are in flight under the MFMAs of k-step s; one barrier per k-tile. The loop is
//    unrolled over the two LDS stages so every stage offset is a constant.
//  * LDS rows are 128 bytes (64 bf16); 16-byte chunks are XOR-swizzled with (r ^ (r >> 3)) & 7
//    so the 16 lanes of one LDS cycle hit distinct banks on reads and writes.
//  * Workgroup ids are remapped so each XCD (own L2) works on a contiguous range of tiles, and
//    tiles are visited in groups of 8 row-blocks for L2 reuse.
//  * The epilogue goes through LDS (bf16 or fp32 tile) so global stores and the residual's
//    reads of x and a are full 16-byte row chunks.
#include "common.h"

namespace xmod {

constexpr int GEMM_BK = 64;

#ifndef XMOD_GEMM_SCHED
#define XMOD_GEMM_SCHED 0
#endif

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

// 16-byte global -> LDS copy (DMA form): lane l of the wave writes bytes [16l, 16l+16) of the
// 1 KB LDS block at `lds_block` (wave-uniform).
__device__ __forceinline__ void dma16(const void *gsrc, uint16_t *lds_block) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_block, 16,
                                   0, 0);
}

template <int BM, int BN, int WM, int WN, int EPI>
struct GemmCfg {
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_ELEMS = BM * GEMM_BK, B_ELEMS = BN * GEMM_BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int BN_OUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  static constexpr bool F32_TILE = EPI == EPI_STORE_F32 || EPI == EPI_RESIDUAL;
  static constexpr int CS = F32_TILE ? BN_OUT + 4 : BN_OUT + 8;  // C-tile row stride (elems)
  static constexpr int NSTAGE = 3;                          // LDS ring depth
  static constexpr int LDS_MAIN = NSTAGE * STAGE * 2;
  static constexpr int LDS_C = BM * CS * (F32_TILE ? 4 : 2);
  static constexpr int LDS_BYTES = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  static_assert(BM % 32 == 0 && BN % 32 == 0, "tiles are filled in 32-row DMA blocks");
  static_assert(EPI != EPI_SWIGLU || WN % 64 == 0, "SwiGLU pairs gate/up 32-column blocks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <int BM, int BN, int WM, int WN, int EPI>
__global__ __launch_bounds__((GemmCfg<BM, BN, WM, WN, EPI>::NT)) void gemm_kernel(GemmArgs g) {
  using C = GemmCfg<BM, BN, WM, WN, EPI>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r32 = lane & 31, gq = lane >> 5;
  const int M = g.M, K = g.K;
  const int n_out = g.N;  // output columns (F for SwiGLU)
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (n_out + C::BN_OUT - 1) / C::BN_OUT;

  // --- tile id: XCD-contiguous remap, then grouped row-block order ---
  int wg = blockIdx.x;
  {
    const int nwg = gridDim.x, q = nwg / 8, rem = nwg % 8;
    const int xcd = wg % 8, loc = wg / 8;
    wg = xcd * q + (xcd < rem ? xcd : rem) + loc;
  }
  constexpr int GROUP = 8;
  const int per_group = GROUP * tiles_n;
  const int group = wg / per_group;
  const int first_m = group * GROUP;
  const int gsz = min(tiles_m - first_m, GROUP);
  const int tm = first_m + (wg % per_group) % gsz;
  const int tn = (wg % per_group) / gsz;
  const int m0 = tm * BM;
  const int n0 = tn * C::BN_OUT;  // first output column

  // --- DMA descriptors (rows fixed across k-tiles) ---
  // Wave w fills 1 KB blocks of a tile: its i-th block holds tile rows 32i + 8w .. +8, and lane
  // l lands at byte 16*l of the block, i.e. row 32i + 8w + l/8, physical chunk l%8. Rows are
  // XOR-swizzled, so lane l fetches logical chunk (l%8) ^ swz(row). Element offsets fit in 32
  // bits (every operand here holds fewer than 2^31 elements).
  static_assert(C::NT == 256, "four waves per workgroup");
  const int nk = K / GEMM_BK;
  const int nk_last = nk - 1;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  const int lrow = 8 * wv + (lane >> 3);
  constexpr int NA = BM / 32, NB = BN / 32;  // DMA blocks per wave per tile
  uint32_t a_off[NA], b_off[NB];
#pragma unroll
  for (int i = 0; i < NA; ++i) {
    const int row = 32 * i + lrow;
    const int gm = min(m0 + row, M - 1);
    a_off[i] = ((uint32_t)gm * (uint32_t)g.lda + (((lane & 7) ^ swz(row)) << 3)) * 2u;
  }
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int row = 32 * i + lrow;
    // SwiGLU: 32-row blocks alternate gate (even i) and up (odd i) weights.
    int gn = EPI == EPI_SWIGLU ? n0 + (i >> 1) * 32 + lrow : n0 + row;
    gn = min(gn, g.N - 1);
    b_off[i] = ((uint32_t)gn * (uint32_t)g.ldb + (((lane & 7) ^ swz(row)) << 3)) * 2u;
  }
  const char *a_bytes = (const char *)g.A;
  const char *b_bytes[2] = {(const char *)g.B, (const char *)(EPI == EPI_SWIGLU ? g.B2 : g.B)};
  // Copy k-tile kt (clamped to the last one) into the stage at element offset `stage`.
  // Sources are a uniform base plus a 32-bit byte offset per lane.
  auto issue_tile = [&](int kt, int stage) {
    const uint32_t kb = (uint32_t)min(kt, nk_last) * (GEMM_BK * 2);
#pragma unroll
    for (int i = 0; i < NA; ++i)
      dma16(a_bytes + (a_off[i] + kb), lds + stage + (32 * i + 8 * wv) * GEMM_BK);
#pragma unroll
    for (int i = 0; i < NB; ++i)
      dma16(b_bytes[EPI == EPI_SWIGLU ? (i & 1) : 0] + (b_off[i] + kb),
            lds + stage + C::A_ELEMS + (32 * i + 8 * wv) * GEMM_BK);
  };

  // --- fragment read offsets within a stage ---
  // Fragment rows are wm0 + 32i + r32 (A) and wn0 + 32j + r32 (B), with wm0, wn0 multiples of
  // 64, so swz(row) = swz(r32) ^ (4i & 7): two chunk offsets per k-step (even / odd tile) and a
  // constant 32-row stride that folds into the instruction's immediate offset.
  const int wm0 = (wid / C::NWN) * WM, wn0 = (wid % C::NWN) * WN;
  const int a_base = (wm0 + r32) * GEMM_BK;
  const int b_base = C::A_ELEMS + (wn0 + r32) * GEMM_BK;
  const int sw_lane = swz(r32);

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  bf16x8 fa[2][C::TM], fb[2][C::TN];

  auto load_frags = [&](const uint16_t *st, int ks, int buf) {
    const int c_even = ((2 * ks + gq) ^ sw_lane) << 3, c_odd = c_even ^ 32;
    const uint16_t *pa0 = st + a_base + c_even, *pa1 = st + a_base + c_odd;
    const uint16_t *pb0 = st + b_base + c_even, *pb1 = st + b_base + c_odd;
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      fa[buf][i] = *(const bf16x8 *)(((i & 1) ? pa1 : pa0) + 32 * GEMM_BK * i);
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      fb[buf][j] = *(const bf16x8 *)(((j & 1) ? pb1 : pb0) + 32 * GEMM_BK * j);
  };
  // Multiply one staged k-tile (4 k-steps); fragments of k-step 0 are already loaded.
  // A scheduling barrier closes every k-step, so the compiler cannot regroup the MFMAs into
  // per-accumulator chains: each step issues its TM*TN independent MFMAs while the next step's
  // fragment reads are in flight.
  auto compute_tile = [&](const uint16_t *st) {
#pragma unroll
    for (int ks = 0; ks < GEMM_BK / 16; ++ks) {
      const int buf = ks & 1;
      if (ks + 1 < GEMM_BK / 16) load_frags(st, ks + 1, buf ^ 1);
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
          acc[i][j] =
              __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
#if XMOD_GEMM_SCHED == 1
      if (ks + 1 < GEMM_BK / 16) {
        constexpr int NDS = C::TM + C::TN, NMF = C::TM * C::TN;
#pragma unroll
        for (int q = 0; q < NDS; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
        }
        __builtin_amdgcn_sched_group_barrier(0x008, NMF - NDS, 0);
      }
#endif
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // Three-stage ring: tiles kt+1 and kt+2 are in flight while tile kt is multiplied. Before
  // each barrier a wave waits only until its loads of the next tile have landed (the loads of
  // the tile after it may stay outstanding: vmcnt <= NA + NB), then the barrier publishes the
  // tile to all waves. vmcnt counts this wave's vector-memory loads, which return in order.
  constexpr int NDMA = NA + NB;
  constexpr int WAIT_NEXT = (NDMA & 15) | (7 << 4) | (15 << 8) | ((NDMA >> 4) << 14);
  static_assert(NDMA < 64, "vmcnt field");
  constexpr int S0 = 0, S1 = C::STAGE, S2 = 2 * C::STAGE;
  issue_tile(0, S0);
  issue_tile(1, S1);
  __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
  __syncthreads();
  load_frags(lds + S0, 0, 0);
#pragma unroll 1
  for (int kt = 0;; kt += 3) {
    issue_tile(kt + 2, S2);
    compute_tile(lds + S0);
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __builtin_amdgcn_s_barrier();
    load_frags(lds + S1, 0, 0);
    if (kt + 1 >= nk) break;
    issue_tile(kt + 3, S0);
    compute_tile(lds + S1);
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __builtin_amdgcn_s_barrier();
    load_frags(lds + S2, 0, 0);
    if (kt + 2 >= nk) break;
    issue_tile(kt + 4, S1);
    compute_tile(lds + S2);
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __builtin_amdgcn_s_barrier();
    load_frags(lds + S0, 0, 0);
    if (kt + 3 >= nk) break;
  }
  __syncthreads();  // the last fragment reads are done before LDS is reused for the C tile

  // --- epilogue: accumulators -> C tile in LDS ---
  // Lane holds output row wm0 + 32i + r32 and columns (within its 32-block) 8(e/4) + 4gq + e%4.
  if (EPI == EPI_SWIGLU) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int row = wm0 + 32 * i + r32;
#pragma unroll
      for (int p = 0; p < C::TN / 2; ++p) {
        const int colblk = (wn0 / 64 + p) * 32;  // output columns of this gate/up pair
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float zg = acc[i][2 * p][4 * q4 + e];
            const float zu = acc[i][2 * p + 1][4 * q4 + e];
            v[e] = zg / (1.0f + __expf(-zg)) * zu;
          }
          const int col = colblk + 8 * q4 + 4 * gq;
          u32x2 w2;
          w2[0] = pack_bf16x2(v[0], v[1]);
          w2[1] = pack_bf16x2(v[2], v[3]);
          *(u32x2 *)(lds + row * C::CS + col) = w2;
        }
      }
    }
  } else if (C::F32_TILE) {
    float *lf = (float *)lds;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int row = wm0 + 32 * i + r32;
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = wn0 + 32 * j + 8 * q4 + 4 * gq;
          f32x4 v4;
          v4[0] = acc[i][j][4 * q4];
          v4[1] = acc[i][j][4 * q4 + 1];
          v4[2] = acc[i][j][4 * q4 + 2];
          v4[3] = acc[i][j][4 * q4 + 3];
          *(f32x4 *)(lf + row * C::CS + col) = v4;
        }
    }
  } else {
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int row = wm0 + 32 * i + r32;
#pragma unroll
      for (int j = 0; j < C::TN; ++j) {
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int col = wn0 + 32 * j + 8 * q4 + 4 * gq;
          u32x2 w2;
          w2[0] = pack_bf16x2(acc[i][j][4 * q4 + 0], acc[i][j][4 * q4 + 1]);
          w2[1] = pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
          *(u32x2 *)(lds + row * C::CS + col) = w2;
        }
      }
    }
  }
  __syncthreads();

  // --- epilogue: LDS C tile -> global, 8 columns per thread per step ---
  constexpr int CPR = C::BN_OUT / 8;  // chunks per row
  constexpr int CHUNKS = BM * CPR;
#pragma unroll 2
  for (int id = tid; id < CHUNKS; id += C::NT) {
    const int r = id / CPR, cc = id % CPR;
    const int m = m0 + r, n = n0 + cc * 8;
    if (m >= M || n >= n_out) continue;
    if (EPI == EPI_RESIDUAL) {
      const float *lf = (const float *)lds + r * C::CS + cc * 8;
      const f32x4 f0 = *(const f32x4 *)lf, f1 = *(const f32x4 *)(lf + 4);
      const int64_t xrow =
          g.idx ? (int64_t)(m / g.k) * g.T + min(max(g.idx[m], 0), g.T - 1) : (int64_t)m;
      uint16_t *xp = g.x + xrow * g.ldc + n;
      const float *ap = g.a + (size_t)m * g.ldc + n;
      const f32x4 a0 = *(const f32x4 *)ap, a1 = *(const f32x4 *)(ap + 4);
      const u32x4 xv = *(const u32x4 *)xp;
      const float gg = g.gate ? __fmul_rn(g.varsigma, g.gate[m]) : 0.f;
      u32x4 yv;
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        const float xlo = __uint_as_float(xv[h] << 16), xhi = __uint_as_float(xv[h] & 0xFFFF0000u);
        const float alo = h < 2 ? a0[2 * h] : a1[2 * h - 4], ahi = h < 2 ? a0[2 * h + 1] : a1[2 * h - 3];
        const float flo = h < 2 ? f0[2 * h] : f1[2 * h - 4], fhi = h < 2 ? f0[2 * h + 1] : f1[2 * h - 3];
        const float ylo = g.gate ? gated_residual(xlo, gg, alo, flo) : dense_residual(xlo, alo, flo);
        const float yhi = g.gate ? gated_residual(xhi, gg, ahi, fhi) : dense_residual(xhi, ahi, fhi);
        yv[h] = pack_bf16x2(ylo, yhi);
      }
      *(u32x4 *)xp = yv;
    } else if (EPI == EPI_STORE_F32) {
      const float *lf = (const float *)lds + r * C::CS + cc * 8;
      float *cp = g.Cf + (size_t)m * g.ldc + n;
      *(f32x4 *)cp = *(const f32x4 *)lf;
      *(f32x4 *)(cp + 4) = *(const f32x4 *)(lf + 4);
    } else {
      *(u32x4 *)(g.C + (size_t)m * g.ldc + n) = *(const u32x4 *)(lds + r * C::CS + cc * 8);
    }
  }
}

template <int BM, int BN, int WM, int WN, int EPI>
static hipError_t run_gemm(const GemmArgs &g, hipStream_t s) {
  using C = GemmCfg<BM, BN, WM, WN, EPI>;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + C::BN_OUT - 1) / C::BN_OUT;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI>), dim3(tiles_m * tiles_n), dim3(C::NT), 0,
                     s, g);
  return hipGetLastError();
}

// Tile choice: 256x128 (four 128x64 wave tiles) when there are enough tiles to fill the chip,
// else 128x128 for small problems.
template <int EPI>
static hipError_t dispatch(const GemmArgs &g, hipStream_t s) {
  const int half = EPI == EPI_SWIGLU ? 2 : 1;
  const long t128 = (long)((g.M + 255) / 256) * ((g.N + 128 / half - 1) / (128 / half));
  if (t128 >= 160) return run_gemm<256, 128, 128, 64, EPI>(g, s);
  return run_gemm<128, 128, 64, 64, EPI>(g, s);
}

hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, hipStream_t s) {
  switch (epi) {
    case EPI_STORE: return dispatch<EPI_STORE>(g, s);
    case EPI_STORE_F32: return dispatch<EPI_STORE_F32>(g, s);
    case EPI_SWIGLU: return dispatch<EPI_SWIGLU>(g, s);
    default: return dispatch<EPI_RESIDUAL>(g, s);
  }
}

}  // namespace xmod
