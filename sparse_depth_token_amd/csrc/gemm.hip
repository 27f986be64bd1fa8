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
//  * Software pipeline: the next k-tile's 16-byte global loads are issued before the current
//    tile's MFMAs; operand fragments are double-buffered in registers, so the LDS reads of
//    k-step s+1 are in flight under the MFMAs of k-step s; one barrier per k-tile.
//  * LDS rows are 128 bytes (64 bf16); 16-byte chunks are XOR-swizzled with (r ^ (r >> 3)) & 7
//    so the 16 lanes of one LDS cycle hit distinct banks on reads and writes.
//  * Workgroup ids are remapped so each XCD (own L2) works on a contiguous range of tiles, and
//    tiles are visited in groups of 8 row-blocks for L2 reuse.
//  * The epilogue goes through LDS (bf16 or fp32 tile) so global stores and the residual's
//    reads of x and a are full 16-byte row chunks.
#include "common.h"

namespace xmod {

constexpr int GEMM_BK = 64;

__device__ __forceinline__ int swz(int r) { return (r ^ (r >> 3)) & 7; }

template <int BM, int BN, int WM, int WN, int EPI>
struct GemmCfg {
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = NW * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int A_ELEMS = BM * GEMM_BK, B_ELEMS = BN * GEMM_BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;
  static constexpr int LA = BM * 8 / NT, LB = BN * 8 / NT;  // 16-byte loads per thread
  static constexpr int BN_OUT = EPI == EPI_SWIGLU ? BN / 2 : BN;
  static constexpr bool F32_TILE = EPI == EPI_STORE_F32 || EPI == EPI_RESIDUAL;
  static constexpr int CS = F32_TILE ? BN_OUT + 4 : BN_OUT + 8;  // C-tile row stride (elems)
  static constexpr int LDS_MAIN = 2 * STAGE * 2;
  static constexpr int LDS_C = BM * CS * (F32_TILE ? 4 : 2);
  static constexpr int LDS_BYTES = LDS_MAIN > LDS_C ? LDS_MAIN : LDS_C;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "tile loads must divide evenly");
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

  // --- global load descriptors (rows fixed across k-tiles) ---
  // Thread tid loads 16-byte chunk ch = tid % 8 of tile rows r0 + 32*i, r0 = tid / 8 < 32.
  // Element offsets fit in 32 bits (every operand here holds fewer than 2^31 elements).
  // swz(r0 + 32*i) = swz(r0) ^ (4i & 7): the LDS offsets follow from one per-thread value.
  const int r0 = tid >> 3, ch0 = tid & 7;
  const int sw0 = ch0 ^ swz(r0);
  uint32_t a_off[C::LA], b_off[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int gm = min(m0 + r0 + 32 * i, M - 1);
    a_off[i] = (uint32_t)gm * (uint32_t)g.lda + ch0 * 8;
  }
  // With four waves NT = 256, so the i-th chunk row is r0 + 32*i; for SwiGLU the 32-row
  // blocks of the B tile alternate gate (even i) and up (odd i) weights.
  static_assert(C::NT == 256, "four waves per workgroup");
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    int gn = EPI == EPI_SWIGLU ? n0 + (i >> 1) * 32 + r0 : n0 + r0 + 32 * i;
    gn = min(gn, g.N - 1);
    b_off[i] = (uint32_t)gn * (uint32_t)g.ldb + ch0 * 8;
  }
  auto b_src = [&](int i) { return (EPI == EPI_SWIGLU && (i & 1)) ? g.B2 : g.B; };
  auto lds_off = [&](int i) {  // LDS element offset of this thread's i-th chunk within a tile
    return (r0 + 32 * i) * GEMM_BK + ((sw0 ^ ((4 * i) & 7)) << 3);
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

  u32x4 ra[C::LA], rb[C::LB];
  bf16x8 fa[2][C::TM], fb[2][C::TN];
  const int nk = K / GEMM_BK;

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

#pragma unroll
  for (int i = 0; i < C::LA; ++i) ra[i] = *(const u32x4 *)(g.A + a_off[i]);
#pragma unroll
  for (int i = 0; i < C::LB; ++i) rb[i] = *(const u32x4 *)(b_src(i) + b_off[i]);
#pragma unroll
  for (int i = 0; i < C::LA; ++i) *(u32x4 *)(lds + lds_off(i)) = ra[i];
#pragma unroll
  for (int i = 0; i < C::LB; ++i) *(u32x4 *)(lds + C::A_ELEMS + lds_off(i)) = rb[i];
  __syncthreads();
  load_frags(lds, 0, 0);

#pragma unroll 1
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    const bool more = kt + 1 < nk;
    if (more) {
      const int koff = (kt + 1) * GEMM_BK;
#pragma unroll
      for (int i = 0; i < C::LA; ++i) ra[i] = *(const u32x4 *)(g.A + a_off[i] + koff);
#pragma unroll
      for (int i = 0; i < C::LB; ++i) rb[i] = *(const u32x4 *)(b_src(i) + b_off[i] + koff);
    }
    const uint16_t *st = lds + cur * C::STAGE;
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
    }
    if (more) {
      uint16_t *nx = lds + (cur ^ 1) * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::LA; ++i) *(u32x4 *)(nx + lds_off(i)) = ra[i];
#pragma unroll
      for (int i = 0; i < C::LB; ++i) *(u32x4 *)(nx + C::A_ELEMS + lds_off(i)) = rb[i];
    }
    __syncthreads();
    if (more) load_frags(lds + (cur ^ 1) * C::STAGE, 0, 0);
  }

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

// Tile choice: 256x256 (128x128 per wave) for the SwiGLU GEMM when it still gives at least
// one tile per CU, else 256x128, else 128x128 for small problems. (The fp32-tile epilogues
// need BN <= 128; the plain-store 256x256 variant does not fit its accumulators in registers.)
template <int EPI>
static hipError_t dispatch(const GemmArgs &g, hipStream_t s) {
  const int half = EPI == EPI_SWIGLU ? 2 : 1;
  const long t256 = (long)((g.M + 255) / 256) * ((g.N + 256 / half - 1) / (256 / half));
  const long t128 = (long)((g.M + 255) / 256) * ((g.N + 128 / half - 1) / (128 / half));
  if constexpr (EPI == EPI_SWIGLU) {
    if (t256 >= 256) return run_gemm<256, 256, 128, 128, EPI>(g, s);
  }
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
