// Causal attention over the packed selected rows of each sequence (gfx950, MFMA bf16).
//
// The X-MoD review's Table 7 gives a sparse layer's KV context as the selected subset: packed
// row j of a sequence attends to packed rows 0..j only. Query head h reads KV head
// floor(h * Hkv / Hq) (the grouped-query mapping of the MoDA notes' section 2.1, written
// 0-based). Softmax uses the scale 1/sqrt(head_dim) and the usual online recurrence (running
// max, rescaled running sum and output), so the k x k score matrix is never stored.
//
// Work split: NW = 8 (or 4) waves per workgroup, 32 query rows per wave, key/value tiles of 64
// rows (128 for sequences of 2048 packed rows or more) shared by the workgroup. The register
// footprint allows two waves per SIMD. Two ways of
// giving a workgroup its 32 NW query rows, chosen at launch:
//  * one q-tile of 32 NW packed rows, last tile first in dispatch order: every wave stays busy
//    to the last key tiles, so each SIMD keeps two waves whose MFMA and softmax work overlap.
//    Used when the grid holds more workgroups than there are CUs.
//  * a pair of q-tiles of 16 NW rows (tile nqt-1-p for the first half of the waves, tile p for
//    the second): every workgroup has the same causal work, and the earlier tile's key/value
//    tiles are a prefix of the later one's. Used when each CU gets at most one workgroup: the
//    longest workgroup then holds half as many long rows. Grids of at most half a wave of
//    256-row tiles take four-wave workgroups, so that twice as many CUs share the work.
//
//  * K and V tiles are copied global -> LDS by the DMA form of the load (no staging registers)
//    into a two-stage ring: tile j+1 is in flight while tile j is used. Both stay row-major
//    ([key][hd]) with their 16-byte chunks XOR-swizzled per row.
//  * Scores are computed transposed, S^T = K Q^T (K fragment first), so each lane holds one
//    query's scores: lane l owns query l % 32 and keys 8(e/4) + 4(l/32) + e%4 of each 32-key
//    block. The same lane then holds query l % 32 of O^T = V^T P^T, so the softmax statistics
//    never leave the lane pair (l, l ^ 32).
//  * The P fragment is the second MFMA operand, in the key order the score accumulator already
//    has. The V^T fragment (hd rows, 8 keys per lane in that same order) comes straight from
//    the row-major V tile through the transposing LDS read (ds_read_b64_tr_b16): within each
//    16-lane group, lane 4a+b receives element b of the 8-byte reads of lanes 4e+a, e = 0..3,
//    so lanes that address 4 consecutive keys at 4 consecutive hd offsets hand every lane 4
//    keys of one hd column.
#include "common.h"
#include "wave.h"

namespace xmod {


__device__ __forceinline__ void attn_dma16(const void *gsrc, uint16_t *lds_block) {
  __builtin_amdgcn_global_load_lds(gsrc, (__attribute__((address_space(3))) void *)lds_block, 16,
                                   0, 0);
}

template <int HD, int NW_, int BKV_>
struct AttnCfg {
  // NW waves of 32 query rows: a q-tile of 32 NW rows, or a pair of q-tiles of 16 NW rows;
  // key/value tiles of BKV rows
  static constexpr int NW = NW_, BQ = 32 * NW, BQP = 16 * NW, BKV = BKV_, NT = 64 * NW;
  static constexpr int CPR = HD / 8;              // 16-byte chunks per row
  static constexpr int RPB = 64 / CPR;            // rows per 1 KB DMA block
  static constexpr int TILE = BKV * HD;           // elements of one K (or V) tile
  static constexpr int STAGE = 2 * TILE;          // K then V
  static constexpr int NBLK = 2 * TILE * 2 / 1024;  // 1 KB DMA blocks per stage (K and V)
  static constexpr int NDMA = NBLK / NW;          // per wave
  static_assert(NBLK % NW == 0, "DMA blocks split over the waves");
  // K: 32 consecutive rows read one logical chunk (ds_read_b128), 16 lanes per LDS pass
  // must hit distinct 16-byte bank groups.
  static __device__ __forceinline__ int kswz(int r) {
    return HD == 128 ? (r & 15) : ((r >> 1) & 7);
  }
  // V: a transposing read touches rows base..base+7 and 4 consecutive chunks 4t..4t+3;
  // moving the chunk's upper bits with the row spreads the 32 (row, chunk) pairs evenly over
  // the 64 banks.
  static __device__ __forceinline__ int vswz(int r) {
    return HD == 128 ? 4 * (r & 3) : 4 * ((r >> 1) & 1);
  }
};

// Keys and values of the whole sequence for the Selected-Q/full-KV control: kv rows b*T + j
// hold [K heads | V heads] (leading dimension ldkv); qpos[b*k + q] is the original position of
// packed query q; query q sees keys j <= qpos.
struct FullKV {
  const uint16_t *kv = nullptr;
  int ldkv = 0;
  const int32_t *qpos = nullptr;
  int T = 0;
};

template <int HD, bool FULLKV, int NW, int BKV_ = 64>
__global__ __launch_bounds__(64 * NW, 2) void attn_kernel(const uint16_t *__restrict__ qkv, int ldq,
                                                      uint16_t *__restrict__ o, int ldo,
                                                      int k_fixed, int Hq, int Hkv,
                                                      float scale_log2,
                                                      const int32_t *__restrict__ seq_off,
                                                      const int32_t *__restrict__ seq_len,
                                                      FullKV fkv, float *__restrict__ lse,
                                                      int paired) {
  using C = AttnCfg<HD, NW, BKV_>;
  constexpr int NB = BKV_ / 32;  // 32-key blocks per tile
  constexpr int BQ = C::BQ, BQP = C::BQP, BKV = C::BKV, KS = HD / 16, NT_HD = HD / 32;
  // Lazy rescaling: the reference maximum M of a lane moves only when a tile's maximum exceeds
  // it by more than 2^RESCALE_LOG2 (log2 units), so weights exp2(x - M) stay below 2^8 and most
  // tiles skip the rescale of the running sum and output.
  constexpr float RESCALE_LOG2 = 8.0f;
  __shared__ __attribute__((aligned(1024))) uint16_t lds[2 * C::STAGE];

  const int h = blockIdx.x, b = blockIdx.y;
  // sequence length and first packed row: fixed, or per sequence (the grid covers the longest)
  const int k = seq_len ? seq_len[b] : k_fixed;
  const int64_t row0 = seq_len ? (int64_t)seq_off[b] : (int64_t)b * k_fixed;
  const int nqt = paired ? (k + BQP - 1) / BQP : (k + BQ - 1) / BQ;
  const int n_units = paired ? (nqt + 1) / 2 : nqt;  // q-tile pairs or q-tiles
  // units in a grid-stride loop: one per workgroup when the grid covers the sequence's units,
  // several when it was sized below the longest possible sequence (per-sequence lengths)
  for (int it = blockIdx.z; it < n_units; it += gridDim.z) {
  if (it != (int)blockIdx.z) __syncthreads();  // the previous unit's epilogue is done with LDS
  const int gkv = (h * Hkv) / Hq;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int gq = lane >> 5, r32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(wid);
  // this wave's first packed query, whether it has a share, and the end of the workgroup's
  // query rows (its last key)
  int q_row0, q_end;
  bool active;
  if (paired) {
    const int qt_hi = nqt - 1 - it;
    const bool later = wid < NW / 2;
    q_row0 = (later ? qt_hi : it) * BQP + (wid % (NW / 2)) * 32;
    active = later || it != qt_hi;  // the middle tile of an odd count: the first half only
    q_end = min(qt_hi * BQP + BQP, k);
  } else {
    const int qt = nqt - 1 - it;
    q_row0 = qt * BQ + wid * 32;
    active = true;
    q_end = min(qt * BQ + BQ, k);
  }
  active = active && q_row0 < k;  // a ragged last tile leaves later waves empty
  const int q_pos = q_row0 + r32;  // packed query index
  // key positions: the packed rows themselves, or (full KV) every position of the sequence,
  // a query at original position qpos seeing keys <= qpos
  const int kvlen = FULLKV ? fkv.T : k;
  auto pos_of = [&](int q) -> int {  // position of packed query q (< k) among the keys
    return FULLKV ? fkv.qpos[(int64_t)b * k_fixed + q] : q;
  };
  const int q_key = FULLKV ? pos_of(min(q_pos, k - 1)) : q_pos;  // this lane's query position
  // first and last query positions of this wave (last = -1: nothing to do)
  const int q_first_wave = FULLKV ? pos_of(min(q_row0, k - 1)) : q_row0;
  const int q_last_wave = !active ? -1
                          : FULLKV ? pos_of(min(q_row0 + 31, k - 1)) : q_row0 + 31;

  const int key_hi = FULLKV ? pos_of(q_end - 1) + 1 : q_end;
  const int n_kv = (key_hi + BKV - 1) / BKV;
  const int ldk = FULLKV ? fkv.ldkv : ldq;
  const char *kbase = FULLKV ? (const char *)(fkv.kv + (int64_t)b * fkv.T * fkv.ldkv + gkv * HD)
                             : (const char *)(qkv + row0 * ldq + Hq * HD + gkv * HD);
  const char *vbase = kbase + (size_t)Hkv * HD * 2;

  // DMA: block i of a stage (i < NBLK/2: K, else V) is filled by wave i % 4; lane l lands at
  // byte 16 l, i.e. row RPB * (i mod NBLK/2) + l / CPR, physical chunk l % CPR. The byte
  // offset of a lane's source within a tile is fixed; tiles advance by BKV rows.
  auto dma_row = [&](int n) {
    const int i = C::NW * n + wv;
    const int blk = i >= C::NBLK / 2 ? i - C::NBLK / 2 : i;
    return C::RPB * blk + lane / C::CPR;
  };
  auto dma_lc = [&](int n) {
    const int i = C::NW * n + wv, row = dma_row(n);
    return (lane % C::CPR) ^ (i >= C::NBLK / 2 ? C::vswz(row) : C::kswz(row));
  };
  auto issue_tile = [&](int jt, int stage) {
    const size_t tile_bytes = (size_t)jt * BKV * ldk * 2;
    const bool ragged = jt * BKV + BKV > kvlen;  // rows past the sequence read its last row
#pragma unroll
    for (int n = 0; n < C::NDMA; ++n) {
      const int i = C::NW * n + wv;
      const bool is_v = i >= C::NBLK / 2;
      const int blk = is_v ? i - C::NBLK / 2 : i;
      int row = dma_row(n);
      if (ragged) row = min(row, kvlen - 1 - jt * BKV);
      const uint32_t off = (uint32_t)row * (uint32_t)ldk * 2u + (uint32_t)dma_lc(n) * 16u;
      attn_dma16((is_v ? vbase : kbase) + tile_bytes + off,
                 lds + stage + (is_v ? C::TILE : 0) + C::RPB * blk * HD);
    }
  };

  issue_tile(0, 0);

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
  float m_ref = -INFINITY, l_run = 0.f;  // m_ref in log2 units (score * scale_log2)

  // K fragment offsets (elements, within a stage): row t*32 + r32, logical chunk 2s + gq
  int k_off[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) k_off[s] = r32 * HD + (((2 * s + gq) ^ C::kswz(r32)) * 8);
  // Transposing-read byte offsets (within a stage's V tile): this lane, as the source of an
  // 8-byte read, addresses key row 16 s + 4 (g >> 1) + e (+ 8 for keys 4..7) and hd column
  // 32 t + 16 (g & 1) + 4 a, g = lane / 16, e = lane / 4 % 4, a = lane % 4. The swizzle of
  // those rows depends on the lane only, so (s, half) go into the instruction's offset.
  const int tg = lane >> 4, te = (lane >> 2) & 3, ta = lane & 3;
  const int v_row = 4 * (tg >> 1) + te;
  const uint32_t lds_base =
      (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint16_t *)lds;
  uint32_t v_off[NT_HD];
#pragma unroll
  for (int t = 0; t < NT_HD; ++t) {
    const int col = 32 * t + 16 * (tg & 1) + 4 * ta;
    v_off[t] = 2u * (uint32_t)(C::TILE + v_row * HD + ((col >> 3) ^ C::vswz(v_row)) * 8 + (col & 7));
  }
  static_assert(HD == 128 || HD == 64, "swizzle of V rows depends on row % 4 (HD 128) or row % 4 / 2 (HD 64)");

  __builtin_amdgcn_s_waitcnt(0);  // tile 0 and the Q fragments
  __syncthreads();

#pragma unroll 1
  for (int jt = 0; jt < n_kv; ++jt) {
    const int st = (jt & 1) * C::STAGE;
    if (jt + 1 < n_kv) issue_tile(jt + 1, C::STAGE - st);
    const uint16_t *Ks = lds + st;
    const int key0 = jt * BKV;
    // a tile that starts after this wave's last query contributes nothing to it
    if (key0 <= q_last_wave) {
      // S^T[key, query] for 64 keys x this wave's 32 queries. The K fragments of the second
      // 32-key block are read while the first block's MFMAs run.
      f32x16 sacc[NB];
      bf16x8 kf[KS];
#pragma unroll
      for (int s = 0; s < KS; ++s) kf[s] = *(const bf16x8 *)(Ks + k_off[s]);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < NB; ++t) {
#pragma unroll
        for (int e = 0; e < 16; ++e) sacc[t][e] = 0.f;
#pragma unroll
        for (int s = 0; s < KS; ++s) {
          sacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[s], qf[s], sacc[t], 0, 0, 0);
          if (t + 1 < NB) kf[s] = *(const bf16x8 *)(Ks + (t + 1) * 32 * HD + k_off[s]);
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      // The first 16-key step's V fragments are read while the softmax runs.
      u32x2 vr[2][NT_HD][2];
      const uint32_t v_st = lds_base + 2u * (uint32_t)st;
      auto issue_v = [&](int s, int buf) {
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                       : "=v"(vr[buf][t][0])
                       : "v"(v_st + v_off[t]), "i"(2 * 16 * HD * s));
          asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2"
                       : "=v"(vr[buf][t][1])
                       : "v"(v_st + v_off[t]), "i"(2 * (16 * s + 8) * HD));
        }
      };
      issue_v(0, 0);

      // causal mask only where the tile reaches past the wave's first query or the sequence
      if (key0 + BKV - 1 > q_first_wave || key0 + BKV > kvlen) {
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = key0 + t * 32 + 8 * (e >> 2) + 4 * gq + (e & 3);
            if (key > q_key || key >= kvlen) sacc[t][e] = -INFINITY;
          }
      }
      // online softmax in log2 units (statistics shared by lanes l and l^32)
      float mt = -INFINITY;
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) mt = fmaxf(mt, sacc[t][e]);
      mt = max_with_xor32(mt) * scale_log2;
      if (__builtin_amdgcn_ballot_w64(mt > m_ref + RESCALE_LOG2)) {
        const float m_new = fmaxf(m_ref, mt);
        const float corr = __builtin_amdgcn_exp2f(m_ref - m_new);  // exp2(-inf) = 0
        l_run *= corr;
#pragma unroll
        for (int t = 0; t < NT_HD; ++t)
#pragma unroll
          for (int e = 0; e < 16; ++e) oacc[t][e] *= corr;
        m_ref = m_new;
      }
      float psum = 0.f;
#pragma unroll
      for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sacc[t][e], scale_log2, -m_ref));
          sacc[t][e] = p;
          psum += p;
        }
      l_run += psum;

      // O^T[hd, query] += V^T[hd, key] P^T[key, query], 16 keys per MFMA. The transposing
      // reads are issued as inline assembly, one 16-key step ahead of their MFMAs, and waited
      // for explicitly: the compiler's own form of this read is ordered behind every pending
      // DMA copy, which would stall the wave on the next tile's copies here.
#pragma unroll
      for (int s = 0; s < BKV / 16; ++s) {
        const int buf = s & 1;
        if (s + 1 < BKV / 16) {
          issue_v(s + 1, buf ^ 1);
          // all but the 2 * NT_HD reads just issued have completed
          if (NT_HD == 4)
            asm volatile("s_waitcnt lgkmcnt(8)"
                         : "+v"(vr[buf][0][0]), "+v"(vr[buf][0][1]), "+v"(vr[buf][1][0]),
                           "+v"(vr[buf][1][1]), "+v"(vr[buf][2 % NT_HD][0]),
                           "+v"(vr[buf][2 % NT_HD][1]), "+v"(vr[buf][3 % NT_HD][0]),
                           "+v"(vr[buf][3 % NT_HD][1]));
          else
            asm volatile("s_waitcnt lgkmcnt(4)"
                         : "+v"(vr[buf][0][0]), "+v"(vr[buf][0][1]), "+v"(vr[buf][1][0]),
                           "+v"(vr[buf][1][1]));
        } else {
          if (NT_HD == 4)
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(vr[buf][0][0]), "+v"(vr[buf][0][1]), "+v"(vr[buf][1][0]),
                           "+v"(vr[buf][1][1]), "+v"(vr[buf][2 % NT_HD][0]),
                           "+v"(vr[buf][2 % NT_HD][1]), "+v"(vr[buf][3 % NT_HD][0]),
                           "+v"(vr[buf][3 % NT_HD][1]));
          else
            asm volatile("s_waitcnt lgkmcnt(0)"
                         : "+v"(vr[buf][0][0]), "+v"(vr[buf][0][1]), "+v"(vr[buf][1][0]),
                           "+v"(vr[buf][1][1]));
        }
        bf16x8 pf;
#pragma unroll
        for (int j = 0; j < 8; ++j) pf[j] = (__bf16)sacc[s >> 1][8 * (s & 1) + j];
#pragma unroll
        for (int t = 0; t < NT_HD; ++t) {
          bf16x8 vf;
          __builtin_memcpy(&vf, &vr[buf][t][0], 8);
          __builtin_memcpy((char *)&vf + 8, &vr[buf][t][1], 8);
          oacc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf, oacc[t], 0, 0, 0);
        }
      }
    }
    // the next tile's copies (this wave's) have landed; then every wave's have, and every wave
    // is done reading this stage before it is refilled
    __builtin_amdgcn_s_waitcnt((0 & 15) | (7 << 4) | (15 << 8));
    __syncthreads();
  }

  // Epilogue: O = O^T / l, staged through LDS (the ring is free after the last barrier; each
  // wave owns 32 rows x HD, 16-byte chunks XOR-swizzled by row) so that global stores are
  // whole row segments. Written straight from the MFMA layout, every store instruction would
  // touch 32 rows with 16 bytes each, which the memory system handles far below its rate.
  const float l_tot = sum_with_xor32(l_run);
  const float inv = 1.0f / l_tot;
  // log2 of the softmax normaliser in the weights' units: P = exp2(score * scale_log2 - lse)
  if (lse && active && gq == 0 && q_pos < k)
    lse[(row0 + q_pos) * Hq + h] = m_ref + __builtin_amdgcn_logf(l_tot);  // v_log_f32: log2
  if (active) {
    // The epilogue's lane-dependent addresses are derived from an opaque copy of the lane id,
    // so the compiler forms them here instead of keeping them live across the key loop.
    int lane_e = lane;
    asm volatile("" : "+v"(lane_e));
    const int r32e = lane_e & 31, gqe = lane_e >> 5;
    uint16_t *ow = lds + wid * 32 * HD;
#pragma unroll
    for (int t = 0; t < NT_HD; ++t)
#pragma unroll
      for (int q4 = 0; q4 < 4; ++q4) {
        const int c = 4 * t + q4;  // 16-byte chunk of hd 32t + 8q4 .. +7
        *(uint2 *)(ow + r32e * HD + ((c ^ (r32e & (C::CPR - 1))) * 8) + 4 * gqe) =
            make_uint2(pack_bf16x2(oacc[t][4 * q4] * inv, oacc[t][4 * q4 + 1] * inv),
                       pack_bf16x2(oacc[t][4 * q4 + 2] * inv, oacc[t][4 * q4 + 3] * inv));
      }
    // the same wave reads back: LDS operations of one wave complete in order
    constexpr int RPI = 64 / C::CPR;  // rows per store instruction
    const int q0 = q_row0;
#pragma unroll
    for (int i = 0; i < 32 / RPI; ++i) {
      const int r = RPI * i + lane_e / C::CPR, c = lane_e % C::CPR;
      const uint4 v = *(const uint4 *)(ow + r * HD + ((c ^ (r & (C::CPR - 1))) * 8));
      if (q0 + r < k) *(uint4 *)(o + (row0 + q0 + r) * ldo + h * HD + c * 8) = v;
    }
  }
  }  // unit loop
}

constexpr int ATTN_CUS = 256;  // MI355X

template <int HD, bool FULLKV, int NW, int BKV>
static void launch_nw(dim3 grid, hipStream_t s, const uint16_t *qkv, int ld_qkv, uint16_t *o,
                      int ld_o, int k, int Hq, int Hkv, float scale_log2, const int32_t *seq_off,
                      const int32_t *seq_len, const FullKV &fkv, float *lse, int paired) {
  hipLaunchKernelGGL((attn_kernel<HD, FULLKV, NW, BKV>), grid, dim3(64 * NW), 0, s, qkv, ld_qkv, o,
                     ld_o, k, Hq, Hkv, scale_log2, seq_off, seq_len, fkv, lse, paired);
}

// Key tiles of 128 rows for sequences of at least this many packed rows (half the barriers
// and per-tile softmax bookkeeping of 64-row tiles: 1 x 8192 rows, 32/8 heads 536 -> 517 us,
// 1 x 16384, 16/4 heads 1058 -> 1017 us, 2 x 4100, 32/8 heads 298 -> 291 us; at 8 x 512 rows
// they were 5 % slower). Chosen by the sequence length alone, so that a sequence's result
// does not depend on the batch it runs in. The Selected-Q/full-KV form keeps 64-row tiles (at
// 128 its register allocation spills), and so do per-sequence lengths (the host knows only
// their bound).
constexpr int ATTN_LONG_KEYS = 2048;

template <bool FULLKV>
static void launch_attn(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, int B, int k,
                        int Hq, int Hkv, int hd, const int32_t *seq_off, const int32_t *seq_len,
                        const FullKV &fkv, hipStream_t s, float *lse = nullptr) {
  // (head, sequence, unit): the unit index is the slowest, so in the one-tile split every
  // head's and sequence's longest tiles are dispatched first. Per-sequence lengths (k is then
  // only their bound): a quarter of the units of a longest sequence per (head, sequence), each
  // workgroup looping over its share.
  const long hb = (long)Hq * B;
  const long t256 = hb * ((k + 255) / 256);
  int nw = 8, paired = t256 <= ATTN_CUS;
  // At most half a wave of 256-row tiles: four-wave workgroups (pairs of 64-row q-tiles), twice
  // as many of them on the CUs. 1024 routed rows, 8 heads: 15.1 -> 12.3 us; 2048 rows, 12 heads
  // 20.9 -> 18.8 us; identical results (each wave's rows see the same key tiles in the same
  // order). At 256 workgroups of eight waves (4096 rows, 16 heads) it gains nothing.
  // fixed-length sequences of at least ATTN_LONG_KEYS rows take 128-row key tiles (with
  // per-sequence lengths k is only their bound, and the tiles stay 64 rows)
  const bool long_keys = !FULLKV && !seq_len && k >= ATTN_LONG_KEYS;
  if (t256 <= 128 && !long_keys) nw = 4;
  const int bq = 32 * nw;
  const int units = paired ? ((k + bq / 2 - 1) / (bq / 2) + 1) / 2 : (k + bq - 1) / bq;
  const dim3 grid((unsigned)Hq, (unsigned)B, (unsigned)(seq_len ? (units + 3) / 4 : units));
  const float scale_log2 = 1.4426950408889634f / sqrtf((float)hd);
#define XMOD_ATTN_NW(HD_, NW_, BKV_)                                                          \
  launch_nw<HD_, FULLKV, NW_, BKV_>(grid, s, qkv, ld_qkv, o, ld_o, k, Hq, Hkv, scale_log2,    \
                                    seq_off, seq_len, fkv, lse, paired)
  if constexpr (!FULLKV) {
    if (long_keys) {  // eight-wave workgroups only (the wave count does not change the bits)
      if (hd == 128) XMOD_ATTN_NW(128, 8, 128);
      else XMOD_ATTN_NW(64, 8, 128);
      return;
    }
  }
  if (hd == 128) {
    if (nw == 8) XMOD_ATTN_NW(128, 8, 64);
    else XMOD_ATTN_NW(128, 4, 64);
  } else {
    if (nw == 8) XMOD_ATTN_NW(64, 8, 64);
    else XMOD_ATTN_NW(64, 4, 64);
  }
#undef XMOD_ATTN_NW
}

hipError_t launch_attention(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, int B, int k,
                            int Hq, int Hkv, int hd, const int32_t *seq_off,
                            const int32_t *seq_len, hipStream_t s) {
  launch_attn<false>(qkv, ld_qkv, o, ld_o, B, k, Hq, Hkv, hd, seq_off, seq_len, FullKV{}, s);
  return hipGetLastError();
}

hipError_t launch_attention_lse(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, float *lse,
                                int B, int k, int Hq, int Hkv, int hd, hipStream_t s) {
  launch_attn<false>(qkv, ld_qkv, o, ld_o, B, k, Hq, Hkv, hd, nullptr, nullptr, FullKV{}, s, lse);
  return hipGetLastError();
}

hipError_t launch_attention_fullkv(const uint16_t *q, int ld_q, const uint16_t *kv, int ld_kv,
                                   const int32_t *qpos, uint16_t *o, int ld_o, int B, int k,
                                   int T, int Hq, int Hkv, int hd, hipStream_t s) {
  FullKV f;
  f.kv = kv; f.ldkv = ld_kv; f.qpos = qpos; f.T = T;
  launch_attn<true>(q, ld_q, o, ld_o, B, k, Hq, Hkv, hd, nullptr, nullptr, f, s);
  return hipGetLastError();
}

}  // namespace xmod
