// bf16 GEMM on CDNA4 matrix cores: C[M,N] = sum_k A(m, k) B(n, k), fp32 accumulation.
//
// Used for the four projections of the X-MoD layer on the packed selected rows: QKV, O
// (fp32 output), gate/up (SwiGLU fused into the epilogue) and down (gated residual + scatter
// into x fused into the epilogue), and for their gradients. In the forward ("NT") both operands
// are K-contiguous rows, the natural operand layout of v_mfma_f32_32x32x16_bf16: every lane
// reads 8 consecutive bf16 (16 bytes) of a row. The backward multiplies by a weight read along
// its output dimension ("NN": B stored [K, N]) and forms weight gradients as sums over tokens
// ("TN": A stored [K, M], B stored [K, N]). A k-major operand is staged in LDS as it lies in
// memory (k-rows of the tile's M or N extent) and its fragments are read with the transposing
// LDS read ds_read_b64_tr_b16: within each 16-lane group, lane 4a+b receives element b of the
// 8-byte reads of lanes 4e+a (e = 0..3), so four lanes reading 4 consecutive k-rows at 4
// consecutive columns give each lane 4 consecutive k of one column; two such reads make the
// 8-k fragment the MFMA expects, in the same k order as a k-contiguous fragment.
//
// Design (gfx950, wave64):
//  * Workgroup tile BM x BN x BK, four or eight compute waves in a grid, each computing a
//    WM x WN sub-tile as (WM/32) x (WN/32) MFMA 32x32x16 tiles (fp32 accumulators in
//    registers), plus (optionally) four loader waves that only copy k-tiles into LDS.
//  * The weight fragment is the MFMA's first operand and the activation fragment its second,
//    so each lane ends with 4 consecutive output columns of one row.
//  * k-tiles are copied global -> LDS by the DMA form of the load (buffer_load_dwordx4 ... lds
//    through one buffer resource per operand: 16 bytes per lane, no staging registers, the
//    k-tile's offset a scalar operand) into an NS-stage LDS ring: tiles kt+1 .. kt+NS-1
//    are in flight while tile kt is multiplied. Before each barrier a wave waits only for its
//    own loads of the next tile. When the compute waves copy their own tiles, the copies are
//    spread over the k-steps (the CU's vector-memory path moves 64 bytes per clock).
//  * Operand fragments are double-buffered in registers. Every k-step is laid out slot by slot
//    (one MFMA per slot, scheduling barriers between slots): the next k-step's fragment reads
//    go out in the first slots, the DMA copies in the later ones.
//  * LDS rows (BK bf16) are split in 16-byte chunks, XOR-swizzled per row so that the lanes of
//    one LDS cycle read distinct banks.
//  * Workgroup ids are remapped so each XCD (own L2) works on a contiguous range of tiles, and
//    tiles are visited in groups of 8 row-blocks for L2 reuse.
//  * The epilogue goes through LDS (bf16 or fp32 tile, in row chunks when the fp32 tile does
//    not fit) so global stores and the residual's reads of x and a are 16-byte row chunks.
//    The exception is the forward SwiGLU product on large grids: a CU-sized grid walks the
//    tiles, the copy ring runs on from one tile into the next (the next tile's first k-tiles
//    are copied under this one's last k-steps) and the epilogue stores from registers.
#include "common.h"

namespace xmod {

// The logistic function of the SwiGLU epilogues by the hardware's exp2 and reciprocal (about one
// ulp each; the products are rounded to bf16 next), where 1 / (1 + e^-z) with a correctly
// rounded division costs about ten vector instructions per element.
__device__ __forceinline__ float swiglu_sigmoid(float z) {
  return __builtin_amdgcn_rcpf(1.0f + __builtin_amdgcn_exp2f(z * -1.4426950408889634f));
}

// 16-byte global -> LDS copy (DMA form, through a buffer resource): lane l of the wave writes
// bytes [16l, 16l+16) of the 1 KB LDS block at `lds_block` (wave-uniform), read from byte
// voff + soff of the resource. voff is the lane's part of the offset, fixed across k-tiles;
// soff is the k-tile's part, uniform, so a copy costs no vector arithmetic.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, uint32_t voff, uint32_t soff,
                                      uint16_t *lds_block) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(
      r, (__attribute__((address_space(3))) void *)lds_block, 16, voff, soff, 0, 0);
}
// A raw buffer resource over an operand: every byte offset the kernel forms is below 2^32 (the
// operands hold fewer than 2^31 elements), and the kernel clamps its rows itself, so the
// record count is the largest one (no range check).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t operand_rsrc(const void *p) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, (int)0xFFFFFFFFu,
                                           0x00020000);
}

// Physical 16-byte chunk index of logical chunk c in LDS row r (rows of BK bf16), for the
// fragment read (32 consecutive rows, one logical chunk per half-wave). Both forms were measured
// free of bank conflicts on gfx950 with that exact pattern (SQ_LDS_BANK_CONFLICT = 0), which
// other candidates are not (64-byte rows swizzled by ((r >> 1) ^ (r >> 3)) & 3: two-way).
//  BK = 64 (8 chunks, 128-byte rows): c ^ ((r ^ (r >> 3)) & 7).
//  BK = 32 (4 chunks, 64-byte rows): c ^ ((r >> 2) & 3).
// Neither depends on the row's 32-row block, so a fragment's chunk offsets are the same for
// every 32-row block of a wave's tile (BK = 64: up to the XOR with 4i & 7).
template <int BK>
__device__ __forceinline__ int swz(int r) {
  if (BK == 64) return (r ^ (r >> 3)) & 7;
  return (r >> 2) & 3;
}

// Physical 16-byte chunk of logical chunk c in k-row r of a k-major tile (rows of at least 16
// chunks): c ^ 4(r % 4). A transposing read by 32 lanes covers 4 consecutive k-rows and 4
// consecutive chunks; the XOR spreads those 16 (row, chunk) pairs over all 64 banks.
__device__ __forceinline__ int swz_km(int r) { return 4 * (r & 3); }

template <int BM, int BN, int WM, int WN, int BK, int NS, int EPI, int LAY, int NL>
struct GemmCfg {
  // NW compute waves; NL loader waves (0: the compute waves copy their own k-tiles)
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN, NT = (NW + NL) * 64;
  static constexpr int NDW = NL ? NL : NW;  // waves that issue the DMA copies
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr bool A_KM = LAY == LAY_TN, B_KM = LAY != LAY_NT;  // k-major operands
  static constexpr int A_ELEMS = BM * BK, B_ELEMS = BN * BK;
  static constexpr int STAGE = A_ELEMS + B_ELEMS;            // elements per LDS stage
  static constexpr int NSTAGE = NS;                          // LDS ring depth
  static constexpr int CPR = BK / 8;                         // 16-byte chunks per LDS row
  static constexpr int RPB = 64 / CPR;                       // rows per 1 KB DMA block
  // DMA blocks per copying wave per tile (1 KB each, whatever the layout)
  static constexpr int NA = BM * BK / 512 / NDW, NB = BN * BK / 512 / NDW;
  static constexpr bool SWIGLU_FWD = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE;
  static constexpr int BN_OUT = SWIGLU_FWD ? BN / 2 : BN;
  static constexpr bool F32_TILE =
      EPI == EPI_STORE_F32 || EPI == EPI_RESIDUAL || EPI == EPI_SWIGLU_BWD;
  static constexpr int ESZ = F32_TILE ? 4 : 2;
  // C-tile row stride (elements); EPI_SWIGLU_SAVE holds g, zg and zu side by side
  static constexpr int CS = F32_TILE ? BN_OUT + 4
                            : EPI == EPI_SWIGLU_SAVE ? 3 * BN_OUT + 8 : BN_OUT + 8;
  static constexpr int LDS_MAIN = NSTAGE * STAGE * 2;
  // C-tile rows per epilogue pass: BM / 2^j, the largest that fits in the ring's LDS
  static constexpr int RCH_FIT = LDS_MAIN / (CS * ESZ);
  static constexpr int RCH = BM <= RCH_FIT ? BM : BM / 2 <= RCH_FIT ? BM / 2 : BM / 4 <= RCH_FIT ? BM / 4 : BM / 8;
  static constexpr int NCH = BM / RCH;
  static constexpr int LDS_BYTES = LDS_MAIN;
  // waves per SIMD: (NW + NL) / 4 per workgroup, two workgroups per CU when the LDS allows it
  static constexpr int WAVES_PER_EU = ((NW + NL) / 4) * (LDS_BYTES <= 80 * 1024 ? 2 : 1);
  static_assert(NW == 4 || NW == 8, "four or eight compute waves per workgroup");
  static_assert(NL == 0 || NL == 4, "no loader waves, or one per SIMD");
  static_assert(BK == 32 || BK == 64, "k-tile of 32 or 64");
  static_assert(NS >= 2, "at least one k-tile in flight");
  static_assert(NA >= 1 && NB >= 1 && BM * BK % (512 * NDW) == 0 && BN * BK % (512 * NDW) == 0,
                "DMA blocks");
  static_assert(!SWIGLU_FWD || WN % 64 == 0, "SwiGLU pairs gate/up 32-column blocks");
  static_assert(!SWIGLU_FWD || LAY == LAY_NT, "the forward SwiGLU interleaves k-contiguous B rows");
  static_assert((!A_KM || BM >= 128) && (!B_KM || BN >= 128), "k-major rows of >= 16 chunks");
  static_assert(RCH >= 32 && BM % RCH == 0 && WM % 32 == 0, "epilogue row chunks");
  static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one gfx950 CU");
};

template <int BM, int BN, int WM, int WN, int BK, int NS, int EPI, int LAY, int NL, int SCHED>
__global__ __launch_bounds__((GemmCfg<BM, BN, WM, WN, BK, NS, EPI, LAY, NL>::NT),
                             (GemmCfg<BM, BN, WM, WN, BK, NS, EPI, LAY, NL>::WAVES_PER_EU)) void
gemm_kernel(GemmArgs g) {
  using C = GemmCfg<BM, BN, WM, WN, BK, NS, EPI, LAY, NL>;
  __shared__ __attribute__((aligned(16))) uint16_t lds[C::LDS_BYTES / 2];
  // residual epilogue: the destination row in x and the gate factor of each tile row
  constexpr bool RES = EPI == EPI_RESIDUAL;
  __shared__ int64_t s_xrow[RES ? BM : 1];
  __shared__ float s_gate[RES ? BM : 1];

  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int r32 = lane & 31, gq = lane >> 5;
  // With loader waves, waves NW .. NW+NL-1 only copy k-tiles into LDS and the compute waves
  // issue no vector-memory instruction in the k loop: a copy held up in the memory pipeline
  // (64 bytes per clock per CU) then stalls a wave that has no MFMA to issue.
  const bool loader = NL > 0 && wid >= C::NW;
  // rows: the device-side count when there is one (the grid covers the bound g.M)
  const int M = g.map.n_dev ? min(*g.map.n_dev, g.M) : g.M, K = g.K;
  const int n_out = g.N;  // output columns (F for SwiGLU)
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (n_out + C::BN_OUT - 1) / C::BN_OUT;
  const int n_tiles = tiles_m * tiles_n;
  if ((int)blockIdx.x >= n_tiles) return;  // whole workgroup, before any barrier

  // Tiles are visited in a grid-stride loop: one tile per workgroup when the grid covers them
  // all, several when the row count is device-side and the grid is only CU-sized.
  // SCHED 2 (persistent walk over a CU-sized grid): the copy ring runs on across tiles. The
  // last NS - 1 k-steps of a tile copy the first NS - 1 k-tiles of the workgroup's next tile,
  // and the last k-step reads that tile's first fragments; the epilogue stores from registers
  // and leaves LDS alone, so the next tile's k loop starts without waiting for a copy.
  constexpr bool PF = SCHED == 2;
  static_assert(!PF || (EPI == EPI_SWIGLU && NL == 0), "persistent walk: forward SwiGLU tiles");
  bf16x8 fa[2][C::TM], fb[2][C::TN];
  int st_cur = 0, st_dma = (NS - 1) * C::STAGE;  // ring stages: next to multiply, next to fill
  for (int tile = blockIdx.x; tile < n_tiles; tile += gridDim.x) {
  if (!PF && tile != (int)blockIdx.x) __syncthreads();  // the previous epilogue is done with LDS

  // --- tile id: XCD-contiguous remap, then grouped row-block order ---
  auto tile_origin = [&](int t, int &m0_, int &n0_) {
    int wg = t;
    {
      const int nwg = n_tiles, q = nwg / 8, rem = nwg % 8;
      const int xcd = wg % 8, loc = wg / 8;
      wg = xcd * q + (xcd < rem ? xcd : rem) + loc;
    }
    constexpr int GROUP = 8;
    const int per_group = GROUP * tiles_n;
    const int group = wg / per_group;
    const int first_m = group * GROUP;
    const int gsz = min(tiles_m - first_m, GROUP);
    m0_ = (first_m + (wg % per_group) % gsz) * BM;
    n0_ = ((wg % per_group) / gsz) * C::BN_OUT;  // first output column
  };
  int m0, n0;
  tile_origin(tile, m0, n0);
  // The residual epilogue's per-row operands (the row map's entry and the gate factor), loaded
  // now into registers (thread t: tile row t) so that their latency passes under the k loop,
  // and parked in LDS after it: the epilogue's loads of x then depend on no other global load.
  int64_t ep_xrow = 0;
  float ep_gate = 0.f;
  if (RES && tid < BM && m0 + tid < M) {
    ep_xrow = rowmap_x(g.map, m0 + tid);
    if (g.gate) {
      const float gm = g.gate[m0 + tid];
      ep_gate = g.residual_form == 1 ? gm : __fmul_rn(g.varsigma, gm);
    }
  }

  // --- DMA descriptors (rows fixed across k-tiles) ---
  // 1 KB block b of a tile holds rows RPB*b .. RPB*b + RPB-1 and is filled by wave b % NW with
  // its instruction b / NW; lane l lands at byte 16*l, i.e. row RPB*b + l / CPR, physical chunk
  // l % CPR, so it fetches logical chunk (l % CPR) ^ swz(row). Element offsets fit in 32 bits
  // (every operand here holds fewer than 2^31 elements); the DMA takes byte offsets.
  const int nk = K / BK;
  const int nk_last = nk - 1;
  const int wv = __builtin_amdgcn_readfirstlane(NL > 0 ? wid - C::NW : wid);  // copying-wave index
  // A k-major operand's block b holds k-rows (512/R) b .. of the tile's R columns; lane l lands
  // at k-row (512/R) b + l / (R/8), physical chunk l % (R/8), so it fetches logical chunk
  // (l % (R/8)) ^ swz_km(k-row) (columns past the matrix are clamped: only stores are masked).
  auto dma_offsets = [&](int tm0, int tn0, uint32_t (&ao)[C::NA], uint32_t (&bo)[C::NB]) {
#pragma unroll
    for (int i = 0; i < C::NA; ++i) {
      if (C::A_KM) {
        constexpr int CPT = BM / 8, RPT = 64 / CPT;
        const int krow = RPT * (C::NDW * i + wv) + lane / CPT;
        const int gm = min(tm0 + (((lane % CPT) ^ swz_km(krow)) << 3), M - 8);
        ao[i] = ((uint32_t)krow * (uint32_t)g.lda + (uint32_t)gm) * 2u;
      } else {
        const int row = C::RPB * (C::NDW * i + wv) + lane / C::CPR;
        const int gm = min(tm0 + row, M - 1);
        ao[i] = ((uint32_t)gm * (uint32_t)g.lda + (((lane % C::CPR) ^ swz<BK>(row)) << 3)) * 2u;
      }
    }
#pragma unroll
    for (int i = 0; i < C::NB; ++i) {
      if (C::B_KM) {
        constexpr int CPT = BN / 8, RPT = 64 / CPT;
        const int krow = RPT * (C::NDW * i + wv) + lane / CPT;
        const int gn = min(tn0 + (((lane % CPT) ^ swz_km(krow)) << 3), g.N - 8);
        bo[i] = ((uint32_t)krow * (uint32_t)g.ldb + (uint32_t)gn) * 2u;
      } else {
        const int row = C::RPB * (C::NDW * i + wv) + lane / C::CPR;
        // SwiGLU: 32-row blocks of the B tile alternate gate and up weights.
        int gn = C::SWIGLU_FWD ? tn0 + (row >> 6) * 32 + (row & 31) : tn0 + row;
        gn = min(gn, g.N - 1);
        bo[i] = ((uint32_t)gn * (uint32_t)g.ldb + (((lane % C::CPR) ^ swz<BK>(row)) << 3)) * 2u;
      }
    }
  };
  uint32_t a_off[C::NA], b_off[C::NB], a_nx[C::NA], b_nx[C::NB];
  dma_offsets(m0, n0, a_off, b_off);
  const bool has_next = PF && tile + (int)gridDim.x < n_tiles;
  if (has_next) {
    int m1, n1;
    tile_origin(tile + gridDim.x, m1, n1);
    dma_offsets(m1, n1, a_nx, b_nx);
  }
  const __amdgpu_buffer_rsrc_t rs_a = operand_rsrc(g.A), rs_b = operand_rsrc(g.B);
  const __amdgpu_buffer_rsrc_t rs_b2 = operand_rsrc(g.B2 ? g.B2 : g.B);
  auto b_half = [&](int i) {  // which weight matrix DMA block i of B reads (SwiGLU: gate / up)
    return C::SWIGLU_FWD ? (((C::RPB * (C::NDW * i + wv)) >> 5) & 1) : 0;  // wave-uniform
  };
  // Copies [lo, hi) of the tile's NA + NB DMA blocks (A blocks first) of k-tile kt, clamped to
  // the last one, into the stage at element offset `stage`. A k-tile of a k-major operand
  // starts BK rows further down; a k-major B switches to B2 at k-row K1 (tile-aligned).
  auto issue_part = [&](int kt, int stage, int lo, int hi) {
    const bool nx = PF && kt > nk_last && has_next;  // the next tile's k-tile kt - nk
    const int ktc = nx ? kt - nk : min(kt, nk_last);
    const uint32_t kb = (uint32_t)ktc * (BK * 2);
    const uint32_t kb_a = C::A_KM ? (uint32_t)ktc * BK * (uint32_t)g.lda * 2u : kb;
    bool km_second = false;
    uint32_t kb_b = kb;
    if (C::B_KM) {
      int kr = ktc * BK;
      if (g.K1 > 0 && kr >= g.K1) {
        km_second = true;
        kr -= g.K1;
      }
      kb_b = (uint32_t)kr * (uint32_t)g.ldb * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::NA; ++i)
      if (i >= lo && i < hi)
        dma16(rs_a, nx ? a_nx[i] : a_off[i], kb_a, lds + stage + 512 * (C::NDW * i + wv));
#pragma unroll
    for (int i = 0; i < C::NB; ++i)
      if (C::NA + i >= lo && C::NA + i < hi)
        dma16((C::B_KM ? km_second : b_half(i) != 0) ? rs_b2 : rs_b, nx ? b_nx[i] : b_off[i],
              kb_b,
              lds + stage + C::A_ELEMS + 512 * (C::NDW * i + wv));
  };
  auto issue_tile = [&](int kt, int stage) { issue_part(kt, stage, 0, C::NA + C::NB); };

  // --- fragment read offsets within a stage ---
  // Fragment rows are wm0 + 32i + r32 (A) and wn0 + 32j + r32 (B). For BK = 64,
  // swz(32 q + r32) = swz(r32) ^ (4 q & 7): the chunk XOR flips with the parity of the
  // fragment's 32-row block q = wm0 / 32 + i (wn0 / 32 + j), so a k-step needs two chunk offsets
  // (even / odd block) plus a constant 32-row stride folded into the immediate offset. A wave
  // tile 32 rows wide starts on an odd block in every other wave; its block parity offset
  // (a_par, b_par: 0 or 32 elements) is folded into the base.
  const int wm0 = (wid / C::NWN) * WM, wn0 = (wid % C::NWN) * WN;
  const int a_par = (BK == 64 && WM % 64 != 0) ? (((wm0 >> 5) & 1) << 5) : 0;
  const int b_par = (BK == 64 && WN % 64 != 0) ? (((wn0 >> 5) & 1) << 5) : 0;
  const int a_base = (wm0 + r32) * BK;
  const int b_base = C::A_ELEMS + (wn0 + r32) * BK;
  const int sw_lane = swz<BK>(r32);
  // k-major fragments: as the source of a transposing read, lane l addresses k-row
  // 16 ks + 8 (g >> 1) + e (+ 4 for the second read) and column 32 i + 16 (g & 1) + 4 a of the
  // wave's rows, g = l / 16, e = l / 4 % 4, a = l % 4; it receives column 32 i + l % 32 and
  // k 16 ks + 8 (l / 32) + 0..3 (4..7), the k-contiguous fragment's order. Byte offsets within
  // a stage; the k-row's swizzle depends on e only, so (ks, second read) go in the immediate.
  const int g16 = lane >> 4, e4 = (lane >> 2) & 3, a4 = lane & 3;
  const int krow0 = 8 * (g16 >> 1) + e4;
  uint32_t akm[C::TM], bkm[C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i) {
    const int col = wm0 + 32 * i + 16 * (g16 & 1) + 4 * a4;
    akm[i] = 2u * (uint32_t)(krow0 * BM + ((((col >> 3) ^ swz_km(krow0)) << 3) | (col & 7)));
  }
#pragma unroll
  for (int j = 0; j < C::TN; ++j) {
    const int col = wn0 + 32 * j + 16 * (g16 & 1) + 4 * a4;
    bkm[j] = 2u * (uint32_t)(C::A_ELEMS + krow0 * BN +
                             ((((col >> 3) ^ swz_km(krow0)) << 3) | (col & 7)));
  }
  auto lds_addr = [](const uint16_t *p) {
    return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const uint16_t *)p;
  };

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  // Fragment f of k-step ks of stage st into buffer buf, in first-use order of the MFMA loop
  // below (row-major over (i, j)): A0, B0 .. B(TN-1), A1 .. A(TM-1).
  // Two transposing reads (k 0..3 and 4..7 of the lane's 8) of a k-major fragment. The
  // compiler does not see these loads: the k-step that uses the fragment waits for them.
  auto tr_frag = [&](uint32_t addr, int ks, int R) {
    u32x2 lo, hi;
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(lo) : "v"(addr), "i"(2 * 16 * ks * R));
    asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                 : "=v"(hi) : "v"(addr), "i"(2 * (16 * ks + 4) * R));
    u32x4 w;
    w[0] = lo[0]; w[1] = lo[1]; w[2] = hi[0]; w[3] = hi[1];
    return __builtin_bit_cast(bf16x8, w);
  };
  auto load_frag = [&](const uint16_t *st, int ks, int buf, int f) {
    const int c_even = ((2 * ks + gq) ^ sw_lane) << 3;
    const int c_odd = BK == 64 ? c_even ^ 32 : c_even;
    if (f >= 1 && f <= C::TN) {
      const int j = f - 1;
      if (C::B_KM)
        fb[buf][j] = tr_frag(lds_addr(st) + bkm[j], ks, BN);
      else
        fb[buf][j] = *(const bf16x8 *)(st + b_base + (((j & 1) ? c_odd : c_even) ^ b_par) +
                                       32 * BK * j);
    } else {
      const int i = f == 0 ? 0 : f - C::TN;
      if (C::A_KM)
        fa[buf][i] = tr_frag(lds_addr(st) + akm[i], ks, BM);
      else
        fa[buf][i] = *(const bf16x8 *)(st + a_base + (((i & 1) ? c_odd : c_even) ^ a_par) +
                                       32 * BK * i);
    }
  };
  constexpr int NMF = C::TM * C::TN, NFR = C::TM + C::TN;
  constexpr int HALF = NMF > 1 ? NMF / 2 : 1;
  constexpr int FPS = (NFR + HALF - 1) / HALF;  // fragment reads per early slot

  // NS-stage ring: while tile kt is multiplied, tiles kt+1 .. kt+NS-1 are in flight. vmcnt
  // counts this wave's vector-memory loads, which complete in order, so "vmcnt <= loads of
  // NS-2 tiles" means tile kt+1 has landed.
  constexpr int NDMA = C::NA + C::NB;
  constexpr int VM = (NS - 2) * NDMA;
  static_assert(VM < 64, "vmcnt field");
  constexpr int WAIT_NEXT = (VM & 15) | (7 << 4) | (15 << 8) | ((VM >> 4) << 14);
  constexpr int WAIT_NEXT_LDS0 = (VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14);
  constexpr int KS = BK / 16;  // k-steps per tile
  // the copies of a k-tile are spread over the first KS - 1 k-steps of the tile before it
  constexpr int SH = (NDMA + KS - 2) / (KS - 1);  // DMA blocks per k-step

  // One k-step as NMF slots of one MFMA each, in a fixed order (a scheduling barrier closes
  // every slot; each MFMA takes 8 passes, during which the wave issues the slot's other
  // instructions). The next k-step's fragment reads go out in the first slots, so they land
  // long before they are needed; the k-step's share [dma_lo, dma_hi) of the DMA copies goes
  // out one or two per slot in the later slots, so copies never hold up MFMA issue for long.
  // Left to itself the compiler sinks the fragment reads below the MFMAs and waits on them at
  // the start of every k-step, and issues the copies in one burst.
  auto kstep = [&](int buf, const uint16_t *ld_st, int ld_ks, int ld_buf, int dma_kt,
                   int dma_stage, int dma_lo, int dma_hi) {
    if (C::A_KM || C::B_KM) {
      // this k-step's transposed fragments (read during the previous one) have landed; the
      // empty statements tie every fragment register to the wait
      asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
#pragma unroll
      for (int j = 0; j < C::TN; ++j) asm volatile("" : "+v"(fb[buf][j]));
#pragma unroll
      for (int i = 0; i < C::TM; ++i) asm volatile("" : "+v"(fa[buf][i]));
    }
#pragma unroll
    for (int t = 0; t < NMF; ++t) {
      const int i = t / C::TN, j = t % C::TN;
      acc[i][j] =
          __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[buf][j], fa[buf][i], acc[i][j], 0, 0, 0);
#pragma unroll
      for (int f = t * FPS; f < (t + 1) * FPS; ++f)
        if (f < NFR) load_frag(ld_st, ld_ks, ld_buf, f);
      if constexpr (NMF > HALF) {
        if (t >= HALF && dma_hi > dma_lo) {
          const int per = (dma_hi - dma_lo + (NMF - HALF) - 1) / (NMF - HALF);
          const int lo = dma_lo + (t - HALF) * per;
          issue_part(dma_kt, dma_stage, lo, min(lo + per, dma_hi));
        }
      } else if (dma_hi > dma_lo) {  // one MFMA per k-step: its copies go out in that slot
        issue_part(dma_kt, dma_stage, dma_lo, dma_hi);
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // One k-tile, pipelined across the barrier that publishes the next tile: the last k-step's
  // fragments are read (and waited for) before the barrier, so no wave still reads this stage
  // when another wave's DMA overwrites it in the next step; after the barrier the next tile's
  // first fragments are read while the last k-step's MFMAs run from registers. The DMA copies
  // of tile dma_kt are spread over the k-steps before the barrier.
  // (with loader waves the compute waves copy nothing and wait only for their LDS reads)
  constexpr int WAIT_LDS0 = (15) | (7 << 4) | (0 << 8) | (3 << 14);
  auto step = [&](const uint16_t *st, const uint16_t *st_next, int dma_kt, int dma_stage) {
#pragma unroll
    for (int ks = 0; ks < KS - 1; ++ks)
      kstep(ks & 1, st, ks + 1, (ks + 1) & 1, dma_kt, dma_stage, NL ? 0 : ks * SH,
            NL ? 0 : min((ks + 1) * SH, NDMA));
    __builtin_amdgcn_s_waitcnt(NL ? WAIT_LDS0 : WAIT_NEXT_LDS0);
    __builtin_amdgcn_s_barrier();
    kstep((KS - 1) & 1, st_next, 0, 0, 0, 0, 0, 0);
  };
  static_assert(((KS - 1) & 1) == 1, "the last k-step uses fragment buffer 1");

  // Tile kt lives in stage kt % NS. Step kt refills stage (kt - 1) % NS, read in step kt - 1
  // and released by that step's barrier, with tile kt + NS - 1 (clamped to the last tile: the
  // surplus copies land in stages no later step reads, and keep the vmcnt accounting uniform).
  // One loop body with rotating stage offsets (kept in scalar registers): a single exit keeps
  // the accumulators in one register assignment for the epilogue. Loader and compute waves
  // meet at the same barriers: one after the first tile, one per k-tile, one after the loop.
  if constexpr (SCHED == 1) {
    // Alternating groups: waves 0-3 and 4-7 (one of each per SIMD) take turns between a load
    // phase (both k-steps' fragments of a k-tile into registers, this wave's share of the DMA
    // copies of the tile NS - 1 ahead) and a compute phase (that k-tile's MFMAs from
    // registers), one barrier between phases, the second group one phase behind the first:
    // while one wave of a SIMD computes, the other loads.
    static_assert(NL == 0 && C::NW == 8 && KS == 2 && !C::A_KM && !C::B_KM, "alternating schedule");
    const int grp = wid >> 2;
    constexpr int WAIT_PH = (NDMA & 15) | (7 << 4) | (0 << 8) | ((NDMA >> 4) << 14);
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) issue_tile(t, t * C::STAGE);
    __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (15 << 8) | (0 << 14));  // every copy landed
    __syncthreads();
    st_cur = 0;
    st_dma = (NS - 1) * C::STAGE;
    if (grp == 1) __builtin_amdgcn_s_barrier();
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int f = 0; f < NFR; ++f) load_frag(lds + st_cur, ks, ks, f);
      issue_tile(kt + NS - 1, st_dma);
      // this phase's fragments have landed; the copies of the previous load phase too
      __builtin_amdgcn_s_waitcnt(WAIT_PH);
      __builtin_amdgcn_s_barrier();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
#pragma unroll
        for (int t = 0; t < NMF; ++t) {
          const int i = t / C::TN, j = t % C::TN;
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fb[ks][j], fa[ks][i], acc[i][j], 0,
                                                             0, 0);
        }
      __builtin_amdgcn_sched_barrier(0);
      __builtin_amdgcn_s_barrier();
      st_dma = st_cur;
      st_cur = st_cur == (NS - 1) * C::STAGE ? 0 : st_cur + C::STAGE;
    }
    if (grp == 0) __builtin_amdgcn_s_barrier();
  } else if (loader) {
#pragma unroll
    for (int t = 0; t < NS - 1; ++t) issue_tile(t, t * C::STAGE);
    __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
    __syncthreads();
    st_cur = 0;
    st_dma = (NS - 1) * C::STAGE;
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      // stage st_dma was released by the previous barrier; tile kt + 1 lands before this one
      issue_tile(kt + NS - 1, st_dma);
      __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
      __builtin_amdgcn_s_barrier();
      st_dma = st_cur;
      st_cur = st_cur == (NS - 1) * C::STAGE ? 0 : st_cur + C::STAGE;
    }
  } else {
    if (!PF || tile == (int)blockIdx.x) {
      if (NL == 0) {
#pragma unroll
        for (int t = 0; t < NS - 1; ++t) issue_tile(t, t * C::STAGE);
        __builtin_amdgcn_s_waitcnt(WAIT_NEXT);
      }
      __syncthreads();
#pragma unroll
      for (int f = 0; f < NFR; ++f) load_frag(lds, 0, 0, f);
      st_cur = 0;
      st_dma = (NS - 1) * C::STAGE;
    }
#pragma unroll 1
    for (int kt = 0; kt < nk; ++kt) {
      const int st_next = st_cur == (NS - 1) * C::STAGE ? 0 : st_cur + C::STAGE;
      step(lds + st_cur, lds + st_next, kt + NS - 1, st_dma);
      st_dma = st_cur;
      st_cur = st_next;
    }
  }
  if constexpr (PF) {
    // SwiGLU straight from the accumulators: each lane holds 4 consecutive output columns of
    // one row (8-byte stores; the L2 merges a row's pieces). LDS keeps the next tile's copies.
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      const int m = m0 + wm0 + 32 * i + r32;
#pragma unroll
      for (int p = 0; p < C::TN / 2; ++p)
#pragma unroll
        for (int q4 = 0; q4 < 4; ++q4) {
          const int n = n0 + (wn0 / 64 + p) * 32 + 8 * q4 + 4 * gq;
          float v[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float zg = acc[i][2 * p][4 * q4 + e];
            const float zu = acc[i][2 * p + 1][4 * q4 + e];
            v[e] = zg * swiglu_sigmoid(zg) * zu;
          }
          u32x2 w2;
          w2[0] = pack_bf16x2(v[0], v[1]);
          w2[1] = pack_bf16x2(v[2], v[3]);
          if (m < M && n < n_out) *(u32x2 *)(g.C + (size_t)m * g.ldc + n) = w2;
        }
    }
    continue;
  }
  if (RES && tid < BM) {
    s_xrow[tid] = ep_xrow;
    s_gate[tid] = ep_gate;
  }
  __syncthreads();  // all DMA landed and all fragment reads done before LDS holds the C tile

  // --- epilogue, in NCH passes of RCH tile rows ---
  // Lane holds output row wm0 + 32i + r32 and columns (within its 32-block) 8(e/4) + 4gq + e%4.
#pragma unroll
  for (int ch = 0; ch < C::NCH; ++ch) {
    const int r_lo = ch * C::RCH;
    if (ch > 0) __syncthreads();  // previous pass's reads of the C tile are done
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
      if (loader) break;  // loader waves only help with the stores below
      const int row = wm0 + 32 * i + r32 - r_lo;  // row within this pass
      if (wm0 + 32 * i < r_lo || wm0 + 32 * i >= r_lo + C::RCH) continue;
      if (C::SWIGLU_FWD) {
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
              v[e] = zg * swiglu_sigmoid(zg) * zu;
            }
            // (the training form's three conversions per element round in integer arithmetic:
            // the conversion instruction made its register allocation spill; same bits)
            const auto pk = [](float a, float b) {
              return EPI == EPI_SWIGLU_SAVE ? pack_bf16x2_int(a, b) : pack_bf16x2(a, b);
            };
            u32x2 w2;
            w2[0] = pk(v[0], v[1]);
            w2[1] = pk(v[2], v[3]);
            uint16_t *t = lds + row * C::CS + colblk + 8 * q4 + 4 * gq;
            *(u32x2 *)t = w2;
            if (EPI == EPI_SWIGLU_SAVE) {  // zg and zu beside g in the tile
              w2[0] = pk(acc[i][2 * p][4 * q4], acc[i][2 * p][4 * q4 + 1]);
              w2[1] = pk(acc[i][2 * p][4 * q4 + 2], acc[i][2 * p][4 * q4 + 3]);
              *(u32x2 *)(t + C::BN_OUT) = w2;
              w2[0] = pk(acc[i][2 * p + 1][4 * q4], acc[i][2 * p + 1][4 * q4 + 1]);
              w2[1] = pk(acc[i][2 * p + 1][4 * q4 + 2], acc[i][2 * p + 1][4 * q4 + 3]);
              *(u32x2 *)(t + 2 * C::BN_OUT) = w2;
            }
          }
        }
      } else if (C::F32_TILE) {
        float *lf = (float *)lds;
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            f32x4 v4;
            v4[0] = acc[i][j][4 * q4];
            v4[1] = acc[i][j][4 * q4 + 1];
            v4[2] = acc[i][j][4 * q4 + 2];
            v4[3] = acc[i][j][4 * q4 + 3];
            *(f32x4 *)(lf + row * C::CS + wn0 + 32 * j + 8 * q4 + 4 * gq) = v4;
          }
      } else {
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int q4 = 0; q4 < 4; ++q4) {
            u32x2 w2;
            w2[0] = pack_bf16x2(acc[i][j][4 * q4 + 0], acc[i][j][4 * q4 + 1]);
            w2[1] = pack_bf16x2(acc[i][j][4 * q4 + 2], acc[i][j][4 * q4 + 3]);
            *(u32x2 *)(lds + row * C::CS + wn0 + 32 * j + 8 * q4 + 4 * gq) = w2;
          }
      }
    }
    __syncthreads();

    // LDS C rows -> global, 8 columns per thread per step
    constexpr int CPO = C::BN_OUT / 8;                                // chunks per output row
    constexpr int CPRO = (EPI == EPI_SWIGLU_SAVE ? 3 : 1) * CPO;      // chunks per tile row
    constexpr int CHUNKS = C::RCH * CPRO;
#pragma unroll 4
    for (int id = tid; id < CHUNKS; id += C::NT) {
      const int r = id / CPRO, cc = id % CPRO;
      const int part = EPI == EPI_SWIGLU_SAVE ? cc / CPO : 0;  // g, zg, zu
      const int m = m0 + r_lo + r, n = n0 + (cc - part * CPO) * 8;
      if (m >= M || n >= n_out) continue;
      if (EPI == EPI_RESIDUAL) {
        const float *lf = (const float *)lds + r * C::CS + cc * 8;
        const f32x4 f0 = *(const f32x4 *)lf, f1 = *(const f32x4 *)(lf + 4);
        const int64_t xrow = s_xrow[r_lo + r];
        uint16_t *xp = g.x + xrow * g.ldc + n;
        f32x4 a0 = {0.f, 0.f, 0.f, 0.f}, a1 = {0.f, 0.f, 0.f, 0.f};  // no a: a = 0
        if (g.a) {
          const float *ap = g.a + (size_t)m * g.ldc + n;
          a0 = *(const f32x4 *)ap;
          a1 = *(const f32x4 *)(ap + 4);
        }
        const u32x4 xv = *(const u32x4 *)xp;
        const bool mod = g.gate && g.residual_form == 1;
        const float gg = s_gate[r_lo + r];
        u32x4 yv;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          const float xlo = __uint_as_float(xv[h] << 16);
          const float xhi = __uint_as_float(xv[h] & 0xFFFF0000u);
          const float alo = h < 2 ? a0[2 * h] : a1[2 * h - 4];
          const float ahi = h < 2 ? a0[2 * h + 1] : a1[2 * h - 3];
          const float flo = h < 2 ? f0[2 * h] : f1[2 * h - 4];
          const float fhi = h < 2 ? f0[2 * h + 1] : f1[2 * h - 3];
          const float ylo = !g.gate ? dense_residual(xlo, alo, flo)
                            : mod ? mod_residual(xlo, gg, alo, flo) : gated_residual(xlo, gg, alo, flo);
          const float yhi = !g.gate ? dense_residual(xhi, ahi, fhi)
                            : mod ? mod_residual(xhi, gg, ahi, fhi) : gated_residual(xhi, gg, ahi, fhi);
          yv[h] = pack_bf16x2(ylo, yhi);
        }
        *(u32x4 *)xp = yv;
        if (g.fsave) {
          float *fp = g.fsave + (size_t)m * g.ldc + n;
          *(f32x4 *)fp = f0;
          *(f32x4 *)(fp + 4) = f1;
        }
      } else if (EPI == EPI_STORE_F32) {
        const float *lf = (const float *)lds + r * C::CS + cc * 8;
        float *cp = g.M1 > 0 && m >= g.M1 ? g.Cf2 + (size_t)(m - g.M1) * g.ldc + n
                                          : g.Cf + (size_t)m * g.ldc + n;
        *(f32x4 *)cp = *(const f32x4 *)lf;
        *(f32x4 *)(cp + 4) = *(const f32x4 *)(lf + 4);
      } else if (EPI == EPI_SWIGLU_BWD) {
        // dg -> dzg = dg zu SiLU'(zg), dzu = dg SiLU(zg), with SiLU'(z) = s(z)(1 + z(1 - s(z)))
        const float *lf = (const float *)lds + r * C::CS + cc * 8;
        const f32x4 d0 = *(const f32x4 *)lf, d1 = *(const f32x4 *)(lf + 4);
        const uint16_t *zp = g.Z + (size_t)m * g.ldz + n;
        float zg[8], zu[8], dg[8], og[8], ou[8];
        unpack8(*(const uint4 *)zp, zg);
        unpack8(*(const uint4 *)(zp + g.N), zu);
#pragma unroll
        for (int e = 0; e < 4; ++e) { dg[e] = d0[e]; dg[4 + e] = d1[e]; }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float sg = swiglu_sigmoid(zg[e]);
          ou[e] = dg[e] * (zg[e] * sg);
          og[e] = dg[e] * zu[e] * (sg * (1.0f + zg[e] * (1.0f - sg)));
        }
        uint16_t *cp = g.C + (size_t)m * g.ldc + n;
        *(uint4 *)cp = pack8(og);
        *(uint4 *)(cp + g.N) = pack8(ou);
      } else if (EPI == EPI_SWIGLU_SAVE) {
        const u32x4 v = *(const u32x4 *)(lds + r * C::CS + cc * 8);
        uint16_t *dst = part == 0 ? g.C + (size_t)m * g.ldc + n
                                  : g.Z + (size_t)m * g.ldz + (part - 1) * g.N + n;
        *(u32x4 *)dst = v;
      } else {
        *(u32x4 *)(g.C + (size_t)m * g.ldc + n) = *(const u32x4 *)(lds + r * C::CS + cc * 8);
      }
    }
  }
  }  // tile loop
  // PF: the last tile's surplus copies (clamped to its last k-tile) and its unused fragment
  // reads complete before the workgroup gives up its LDS
  if (PF) __builtin_amdgcn_s_waitcnt((0) | (7 << 4) | (0 << 8) | (0 << 14));
}

template <int BM, int BN, int WM, int WN, int BK, int NS, int EPI, int LAY = LAY_NT, int NL = 0,
          int SCHED = 0>
static hipError_t run_gemm(const GemmArgs &g, hipStream_t s) {
  using C = GemmCfg<BM, BN, WM, WN, BK, NS, EPI, LAY, NL>;
  const int tiles_m = (g.M + BM - 1) / BM;
  const int tiles_n = (g.N + C::BN_OUT - 1) / C::BN_OUT;
  // device-side row count: a CU-sized grid walks the tiles (g.M is only the bound)
  const int tiles = tiles_m * tiles_n;
  const int wgs_per_cu = C::WAVES_PER_EU * 4 / (C::NW + NL);  // resident workgroups per CU
  const int grid = g.map.n_dev || SCHED == 2 ? min(tiles, 256 * wgs_per_cu) : tiles;
  hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, BK, NS, EPI, LAY, NL, SCHED>), dim3(grid),
                     dim3(C::NT), 0, s, g);
  return hipGetLastError();
}

// Tile choice (measured on the projections of the X-MoD layer at 4096 routed rows):
//  * SwiGLU with at least two waves of 256x256 tiles: 256x256 (eight waves of 128x64, two per
//    SIMD, BK = 32, four-stage ring, each wave copying its share): the halved epilogue per flop
//    and the second wave per SIMD beat 256x128 by ~5 %. One workgroup per CU walks its tiles
//    with the ring running across tile boundaries (SCHED 2): no tile waits for its first
//    k-tile (8192 x 14336 x 4096: 1541 -> 1511 us; 4096 x 5632 x 2048: 179 -> 171 us).
//  * other products with at least two waves of 256x256 tiles: the same tile with the two wave
//    groups alternating between load and compute phases (8192 rows, d = 4096: QKV 346 -> 339 us,
//    O 254 -> 243, down 872 -> 840; identical results). For SwiGLU the alternation gained
//    < 1 %, and the 256x128 tile below stays ahead on smaller grids.
//  * otherwise 256x128 (four compute waves of 64x128 plus four loader waves, BK = 64,
//    three-stage ring) when the grid gives at least 5/8 of the 256 CUs a tile, else 128x128
//    (four compute waves of 64x64 plus four loader waves), or, when 128x128 tiles would give
//    at most half of the CUs one, 64x64 (four compute waves of 32x32 plus four loader waves):
//    at 1024 routed rows and d = 1024 the O and down products go from 64 to 256 tiles
//    (11.7 -> 9.2 us and 24.8 -> 16.2 us; at 192 tiles of 128x128 the larger tiles win).
//    Loader waves took 8 % off the down projection and 1-3 % off the others; a 64x128 wave
//    tile (two activation by four
//    weight fragments per k-step) sustains more MFMA work per LDS read than 128x64 with one
//    wave per SIMD (1.72 against 1.48 PFLOP/s in a register-fed probe).
constexpr int GEMM_CUS = 256;

template <int EPI, int LAY = LAY_NT>
static hipError_t dispatch(const GemmArgs &g, hipStream_t s) {
  constexpr bool swiglu = EPI == EPI_SWIGLU || EPI == EPI_SWIGLU_SAVE;
  const int half = swiglu ? 2 : 1;
  const long tm = (g.M + 255) / 256;
  if constexpr (swiglu) {
    const long t_256 = tm * ((g.N + 256 / half - 1) / (256 / half));
    if (t_256 >= 2 * GEMM_CUS) {
      if (EPI == EPI_SWIGLU && g.K / 32 >= 4)
        return run_gemm<256, 256, 128, 64, 32, 4, EPI_SWIGLU, LAY, 0, 2>(g, s);
      return run_gemm<256, 256, 128, 64, 32, 4, EPI, LAY>(g, s);
    }
  }
  if constexpr (LAY == LAY_NT && !swiglu) {
    // at least two waves of 256x256 tiles: 256x256, the two wave groups alternating
    const long t_256 = tm * ((g.N + 255) / 256);
    if (t_256 >= 2 * GEMM_CUS) return run_gemm<256, 256, 128, 64, 32, 4, EPI, LAY, 0, 1>(g, s);
  }
  const long t_big = tm * ((g.N + 128 / half - 1) / (128 / half));
  if (t_big >= GEMM_CUS * 5 / 8) return run_gemm<256, 128, 64, 128, 64, 3, EPI, LAY, 4>(g, s);
  if constexpr (LAY == LAY_NT && !swiglu) {
    // a grid of at most half a wave of 128x128 tiles: 64x64 tiles (four times as many)
    const long t_128 = ((g.M + 127) / 128) * ((g.N + 127) / 128);
    if (t_128 <= GEMM_CUS / 2) return run_gemm<64, 64, 32, 32, 64, 3, EPI, LAY, 4>(g, s);
  }
  return run_gemm<128, 128, 64, 64, 64, 3, EPI, LAY, 4>(g, s);
}

hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, hipStream_t s) {
  return launch_gemm(g, epi, LAY_NT, s);
}

hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, GemmLayout lay, hipStream_t s) {
  if (lay == LAY_NN) {
    switch (epi) {
      case EPI_STORE: return dispatch<EPI_STORE, LAY_NN>(g, s);
      case EPI_STORE_F32: return dispatch<EPI_STORE_F32, LAY_NN>(g, s);
      case EPI_SWIGLU_BWD: return dispatch<EPI_SWIGLU_BWD, LAY_NN>(g, s);
      default: return hipErrorInvalidValue;
    }
  }
  if (lay == LAY_TN) {
    if (epi == EPI_STORE_F32) return dispatch<EPI_STORE_F32, LAY_TN>(g, s);
    return hipErrorInvalidValue;
  }
  switch (epi) {
    case EPI_STORE: return dispatch<EPI_STORE>(g, s);
    case EPI_STORE_F32: return dispatch<EPI_STORE_F32>(g, s);
    case EPI_SWIGLU: return dispatch<EPI_SWIGLU>(g, s);
    case EPI_SWIGLU_SAVE: return dispatch<EPI_SWIGLU_SAVE>(g, s);
    case EPI_RESIDUAL: return dispatch<EPI_RESIDUAL>(g, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace xmod
