// Router GEMV and per-sequence top-k of the X-MoD sparse layer (gfx950, wave64).
//
// Router: the scalar Linear(d, 1) score of the "Mixture-of-Depths explained" page ("basic
// architecture"), adjusted by the carried per-token bias of the X-MoD review's Eq. (8):
// ell_t = (w_r . x_t + beta_r) - tau * b_t, in fp32. One wave reduces one row; each wave keeps
// several rows' loads in flight, which is what an HBM-bound pass over all B*T rows needs.
//
// Top-k: the X-MoD review's training-time rule (section "training-time top-k") keeps the
// top-1/K share of each sequence, non-causally. One workgroup of 1024 threads owns one
// sequence: 4 radix passes of 8 bits over order-preserving uint32 keys find the k-th largest
// key, then a block-wide prefix sum over positions writes the winners in ascending position
// order. Ties at the threshold go to the lowest positions; -0 equals +0; NaN ranks lowest.
// All counting is integer, so the result does not depend on thread scheduling.
#include "common.h"
#include "wave.h"

namespace xmod {

// ---- router ---------------------------------------------------------------------------------

template <int NI, int R>
__global__ __launch_bounds__(256) void router_kernel(const uint16_t *__restrict__ x,
                                                     const uint16_t *__restrict__ w, float beta,
                                                     const float *__restrict__ bias, float tau,
                                                     float *__restrict__ logits, int64_t rows,
                                                     int d, float *__restrict__ s_out) {
  const int lane = threadIdx.x & 63;
  const int nch = d >> 3;  // 8-element chunks per row
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * R;
  if (row0 >= rows) return;

  float wf[NI][8];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int c = lane + 64 * i;
    if (c < nch) {
      unpack8(*(const uint4 *)(w + (size_t)c * 8), wf[i]);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) wf[i][e] = 0.f;
    }
  }
  uint4 xv[R][NI];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int64_t row = row0 + r < rows ? row0 + r : rows - 1;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int c = lane + 64 * i;
      xv[r][i] = c < nch ? *(const uint4 *)(x + row * d + (size_t)c * 8) : make_uint4(0, 0, 0, 0);
    }
  }
  float acc[R];
#pragma unroll
  for (int r = 0; r < R; ++r) {
    float a = 0.f;
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      float xf[8];
      unpack8(xv[r][i], xf);
#pragma unroll
      for (int e = 0; e < 8; ++e) a = fmaf(xf[e], wf[i][e], a);
    }
    acc[r] = wave_total(a);
  }
  if (lane == 0) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const int64_t row = row0 + r;
      if (row < rows) {
        const float s = __fadd_rn(acc[r], beta);
        const float tb = bias ? __fmul_rn(tau, bias[row]) : 0.f;
        logits[row] = __fsub_rn(s, tb);
        if (s_out) s_out[row] = s;
      }
    }
  }
}

template <int NI>
static hipError_t router_ni(const uint16_t *x, const uint16_t *w, float beta, const float *bias,
                            float tau, float *logits, int64_t rows, int d, hipStream_t s,
                            float *s_out) {
  // rows per wave (at d = 2048, NI = 4, two rows per wave measured ~4 % faster than four)
  constexpr int R = NI <= 2 ? 8 : (NI <= 8 ? 2 : 1);
  const int64_t waves = (rows + R - 1) / R;
  const int64_t blocks = (waves + 3) / 4;
  hipLaunchKernelGGL((router_kernel<NI, R>), dim3((unsigned)blocks), dim3(256), 0, s, x, w, beta,
                     bias, tau, logits, rows, d, s_out);
  return hipGetLastError();
}

hipError_t launch_router(const uint16_t *x, const uint16_t *w, float beta, const float *bias,
                         float tau, float *logits, int64_t rows, int d, hipStream_t s,
                         float *s_out) {
  const int ni = ((d >> 3) + 63) / 64;
  switch (ni) {
    case 1: return router_ni<1>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    case 2: return router_ni<2>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    case 3: return router_ni<3>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    case 4: return router_ni<4>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    case 5: case 6: return router_ni<6>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    case 7: case 8: return router_ni<8>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
    default: return router_ni<16>(x, w, beta, bias, tau, logits, rows, d, s, s_out);
  }
}

// ---- top-k ----------------------------------------------------------------------------------

// Order-preserving map of fp32 to uint32: a > b (as floats) iff key(a) > key(b).
__device__ __forceinline__ uint32_t order_key(float v) {
  uint32_t u = __float_as_uint(v);
  const uint32_t mag = u & 0x7FFFFFFFu;
  if (mag > 0x7F800000u) return 0u;  // NaN ranks lowest
  if (mag == 0u) u = 0u;             // -0 == +0
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Histogram copies of the first pass: that pass sees the top byte of every key (the sign and
// the high exponent bits, shared by all values of similar magnitude), so a wave's lanes pile
// onto a few bins; LDS atomics to one address within an instruction are serialised, and
// spreading the lanes over 4 copies (by lane % 4) cuts that serialisation fourfold. Later
// passes see spread digits of fewer candidates and use one copy.
constexpr int TOPK_COPIES0 = 4;

// Key ownership: with up to 4 keys per thread, thread t owns the consecutive positions
// 4t .. 4t+3 (one 16-byte span per lane, so every access is coalesced anyway). With 8 or
// more, thread t owns positions t, t + 1024, t + 2048, ... ("rows" of 1024 positions): a
// consecutive span per thread would make every load and store instruction touch 64 cache
// lines, which took most of the kernel's time (32768 positions: 68 -> 37 us per call;
// 65536: 148 -> 97 us, where 64 keys per thread spill registers either way).
template <int KPT>
__global__ __launch_bounds__(1024) void topk_kernel(const float *__restrict__ logits, int T, int k,
                                                    int32_t *__restrict__ idx,
                                                    float *__restrict__ gate,
                                                    float *__restrict__ bias, float delta) {
  constexpr bool STRIDED = KPT >= 8;
  // pass 0: TOPK_COPIES0 copies; passes 1-3: one each (a single barrier per pass)
  __shared__ uint32_t hist[(TOPK_COPIES0 + 3) * 256];
  __shared__ uint32_t s_wave_gt[16], s_wave_eq[16];
  // strided ownership: per (row, wave) counts of keys above / equal to the threshold, then
  // their exclusive prefix in position order
  __shared__ uint32_t s_tab_gt[STRIDED ? KPT * 16 : 1], s_tab_eq[STRIDED ? KPT * 16 : 1];

  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const float *L = logits + (int64_t)b * T;
  const int p0 = tid * KPT;
  auto pos_of = [&](int j) { return STRIDED ? j * 1024 + tid : p0 + j; };

  for (int i = tid; i < (TOPK_COPIES0 + 3) * 256; i += 1024) hist[i] = 0u;
  // The logits (for the gate) and, with consecutive ownership, the carried bias values of this
  // thread's positions are loaded up front, so the output phase waits on no global read.
  float* const Bi = bias ? bias + (int64_t)b * T : nullptr;
  // (with strided ownership only the keys stay in registers; the logits and bias values are
  // read again, coalesced, a batch of rows at a time, when the output is written)
  uint32_t key[KPT];
  float lv[STRIDED ? 1 : KPT], bv[STRIDED ? 1 : KPT];
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    const int p = pos_of(j);
    const float l = p < T ? L[p] : 0.f;
    if (!STRIDED) {
      lv[j] = l;
      bv[j] = (Bi && p < T) ? Bi[p] : 0.f;
    }
    key[j] = p < T ? order_key(l) : 0u;
  }
  __syncthreads();

  // Radix select of the k-th largest key, 8 bits per pass from the top. After each pass's
  // barrier every wave scans that pass's histogram itself (no broadcast, no second barrier).
  uint32_t prefix = 0u, pmask = 0u, remaining = (uint32_t)k;
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int shift = 24 - 8 * pass;
    const int ncopy = pass == 0 ? TOPK_COPIES0 : 1;
    uint32_t *h = hist + (pass == 0 ? 0 : (TOPK_COPIES0 + pass - 1) * 256);
    uint32_t *hc = h + (pass == 0 ? (lane % TOPK_COPIES0) * 256 : 0);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const bool cand = (pos_of(j) < T) && ((key[j] & pmask) == prefix);
      if (cand) atomicAdd(&hc[(key[j] >> shift) & 255u], 1u);
    }
    __syncthreads();
    // lane l owns bins 255-4l .. 252-4l, scanned from the top (largest digit first)
    uint32_t c[4], tot = 0;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      c[q] = 0u;
      for (int cp = 0; cp < ncopy; ++cp) c[q] += h[cp * 256 + 255 - 4 * lane - q];
      tot += c[q];
    }
    const uint32_t incl = wave_incl_scan(tot);
    const uint32_t excl = incl - tot;
    // exactly one lane holds the bin where the running count reaches `remaining`
    uint32_t digit = 0u, rem_new = 0u;
    const bool mine = excl < remaining && remaining <= incl;
    if (mine) {
      uint32_t above = excl;
      bool found = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!found && remaining <= above + c[q]) {
          digit = 255u - 4u * lane - q;
          rem_new = remaining - above;
          found = true;
        }
        if (!found) above += c[q];
      }
    }
    const int src = __ffsll((unsigned long long)__ballot(mine)) - 1;  // wave-uniform
    digit = (uint32_t)__builtin_amdgcn_readlane((int)digit, src);
    remaining = (uint32_t)__builtin_amdgcn_readlane((int)rem_new, src);
    prefix |= digit << shift;
    pmask |= 255u << shift;
  }
  const uint32_t thr = prefix;     // key of the k-th largest
  const uint32_t need = remaining; // how many keys equal to thr are taken (lowest positions)

  int32_t *I = idx + (int64_t)b * k;
  float *G = gate ? gate + (int64_t)b * k : nullptr;
  // The selected keys: all above the threshold key, plus the first `need` equal to it in
  // position order. Output slot of a selected key = the number of selected keys before it.
  if (!STRIDED) {
    // Block-wide exclusive prefix over (count > thr, count == thr) in position order.
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      if (p0 + j < T) {
        gt += key[j] > thr;
        eq += key[j] == thr;
      }
    }
    const uint32_t gt_incl = wave_incl_scan(gt), eq_incl = wave_incl_scan(eq);
    if (lane == 63) {
      s_wave_gt[wid] = gt_incl;
      s_wave_eq[wid] = eq_incl;
    }
    __syncthreads();
    uint32_t gt_base = 0, eq_base = 0;
    for (int w2 = 0; w2 < wid; ++w2) {
      gt_base += s_wave_gt[w2];
      eq_base += s_wave_eq[w2];
    }
    const uint32_t gt_before = gt_base + gt_incl - gt;
    uint32_t eq_seen = eq_base + eq_incl - eq;
    uint32_t pos = gt_before + (eq_seen < need ? eq_seen : need);
#pragma unroll
    for (int j = 0; j < KPT; ++j) {
      const int p = p0 + j;
      if (p < T) {
        bool sel = key[j] > thr;
        if (key[j] == thr) {
          sel = eq_seen < need;
          ++eq_seen;
        }
        // Exactly k keys of the sequence pass, so pos < k; the bound is a cheap guarantee that
        // idx is never overrun, not a selection rule.
        if (sel && pos < (uint32_t)k) {
          I[pos] = p;
          if (G) G[pos] = 1.0f / (1.0f + expf(-lv[j]));
          if (Bi) Bi[p] = __fadd_rn(bv[j], delta);
          ++pos;
        }
      }
    }
    return;
  }

  // Strided ownership: position order is (row j, wave, lane), and each lane holds one key
  // per row, so a row's counts in a wave are ballot popcounts and a lane's offset within them
  // is the number of set ballot bits below it. The (row, wave) totals get one block-wide
  // exclusive scan.
  auto row_masks = [&](int j, unsigned long long &gm, unsigned long long &em) {
    const bool valid = pos_of(j) < T;
    gm = __ballot(valid && key[j] > thr);
    em = __ballot(valid && key[j] == thr);
  };
  auto below = [&](unsigned long long m) {  // set bits of m in lanes below this one
    return (uint32_t)__builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32),
                                              __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
  };
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    unsigned long long gm, em;
    row_masks(j, gm, em);
    if (lane == 0) {
      s_tab_gt[j * 16 + wid] = (uint32_t)__popcll(gm);
      s_tab_eq[j * 16 + wid] = (uint32_t)__popcll(em);
    }
  }
  __syncthreads();
  {
    // entry e = (row e / 16, wave e % 16), KPT * 16 <= 1024 entries, one per thread
    const bool has = tid < KPT * 16;
    const uint32_t g = has ? s_tab_gt[tid] : 0u, q = has ? s_tab_eq[tid] : 0u;
    const uint32_t g_incl = wave_incl_scan(g), q_incl = wave_incl_scan(q);
    if (lane == 63) {
      s_wave_gt[wid] = g_incl;
      s_wave_eq[wid] = q_incl;
    }
    __syncthreads();
    uint32_t g_base = 0, q_base = 0;
    for (int w2 = 0; w2 < wid; ++w2) {
      g_base += s_wave_gt[w2];
      q_base += s_wave_eq[w2];
    }
    if (has) {  // each thread rewrites only the entry it read above
      s_tab_gt[tid] = g_base + g_incl - g;
      s_tab_eq[tid] = q_base + q_incl - q;
    }
  }
  __syncthreads();
  // Output, 8 rows at a time: the rows' logits (for the gate) and bias values are read first
  // (coalesced, every position), so a batch waits for one round trip rather than one per row.
  constexpr int RB = KPT < 8 ? KPT : 8;
#pragma unroll
  for (int j0 = 0; j0 < KPT; j0 += RB) {
    float lc[RB], bc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int p = pos_of(j0 + r);
      lc[r] = p < T ? L[p] : 0.f;
      bc[r] = (Bi && p < T) ? Bi[p] : 0.f;
    }
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int j = j0 + r, p = pos_of(j);
      unsigned long long gm, em;
      row_masks(j, gm, em);
      const uint32_t gt_before = s_tab_gt[j * 16 + wid] + below(gm);
      const uint32_t eq_before = s_tab_eq[j * 16 + wid] + below(em);
      const bool sel = p < T && (key[j] > thr || (key[j] == thr && eq_before < need));
      const uint32_t pos = gt_before + (eq_before < need ? eq_before : need);
      if (sel && pos < (uint32_t)k) {  // pos < k always holds; the bound only guards idx
        I[pos] = p;
        if (G) G[pos] = 1.0f / (1.0f + expf(-lc[r]));
        if (Bi) Bi[p] = __fadd_rn(bc[r], delta);
      }
    }
  }
}

hipError_t launch_topk(const float *logits, int B, int T, int k, int32_t *idx, float *gate,
                       float *bias, float delta, hipStream_t s) {
  const int need = (T + 1023) / 1024;
#define XMOD_TOPK(KPT_)                                                                         \
  hipLaunchKernelGGL((topk_kernel<KPT_>), dim3(B), dim3(1024), 0, s, logits, T, k, idx, gate, \
                     bias, delta)
  if (need <= 1) XMOD_TOPK(1);
  else if (need <= 2) XMOD_TOPK(2);
  else if (need <= 4) XMOD_TOPK(4);
  else if (need <= 8) XMOD_TOPK(8);
  else if (need <= 16) XMOD_TOPK(16);
  else if (need <= 32) XMOD_TOPK(32);
  else XMOD_TOPK(64);
#undef XMOD_TOPK
  return hipGetLastError();
}

// ---- eval-time causal threshold routing -------------------------------------------------------
//
// The X-MoD review's section "training-time top-k, eval-time causal threshold": at evaluation
// a token enters the sparse layer when its routing probability is at least 1/2, which for the
// gate sigmoid(ell) of Eq. (8) means ell >= 0 (-0 included, NaN excluded). Each sequence routes
// its own number of tokens; the selected rows are listed flat, sequence after sequence, in
// ascending position. Two kernels: the per-sequence counts, then (each sequence adding up the
// counts before it) the positions, gates and bias updates.

__device__ __forceinline__ uint32_t block_sum_1024(uint32_t v, uint32_t *s_part) {
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  if (lane == 0) s_part[wid] = v;
  __syncthreads();
  uint32_t t = 0;
  for (int w = 0; w < (int)(blockDim.x >> 6); ++w) t += s_part[w];
  return t;
}

__global__ __launch_bounds__(1024) void threshold_count_kernel(const float *__restrict__ logits,
                                                               int T, int32_t *__restrict__ counts) {
  __shared__ uint32_t s_part[16];
  const int b = blockIdx.x;
  const float *L = logits + (int64_t)b * T;
  uint32_t c = 0;
  for (int p = threadIdx.x; p < T; p += 1024) c += L[p] >= 0.f;
  const uint32_t tot = block_sum_1024(c, s_part);
  if (threadIdx.x == 0) counts[b] = (int32_t)tot;
}

template <int KPT>
__global__ __launch_bounds__(1024) void threshold_write_kernel(
    const float *__restrict__ logits, int B, int T, const int32_t *__restrict__ counts,
    int32_t *__restrict__ offsets, int32_t *__restrict__ src, float *__restrict__ gate,
    int32_t *__restrict__ n_total, float *__restrict__ bias, float delta) {
  __shared__ uint32_t s_part[16];
  __shared__ uint32_t s_wave_tot[16];
  const int b = blockIdx.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  // first flat row of this sequence: the counts of the sequences before it
  uint32_t before = 0;
  for (int q = tid; q < b; q += 1024) before += (uint32_t)counts[q];
  const uint32_t off = block_sum_1024(before, s_part);

  const float *L = logits + (int64_t)b * T;
  const int p0 = tid * KPT;
  float lv[KPT];
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    lv[j] = p0 + j < T ? L[p0 + j] : -1.f;
    mine += lv[j] >= 0.f;
  }
  // block-wide exclusive prefix of the selected counts, in position order
  uint32_t incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, 64);
    if (lane >= o) incl += t;
  }
  if (lane == 63) s_wave_tot[wid] = incl;
  __syncthreads();
  uint32_t base = 0;
  for (int w = 0; w < wid; ++w) base += s_wave_tot[w];
  uint32_t pos = off + base + incl - mine;
  float *Bi = bias ? bias + (int64_t)b * T : nullptr;
#pragma unroll
  for (int j = 0; j < KPT; ++j) {
    if (lv[j] >= 0.f) {
      const int p = p0 + j;
      src[pos] = (int32_t)((int64_t)b * T + p);
      if (gate) gate[pos] = 1.0f / (1.0f + expf(-lv[j]));
      if (Bi) Bi[p] = __fadd_rn(Bi[p], delta);
      ++pos;
    }
  }
  if (tid == 0) {
    offsets[b] = (int32_t)off;
    if (b == B - 1) *n_total = (int32_t)(off + (uint32_t)counts[b]);
  }
}

hipError_t launch_threshold_select(const float *logits, int B, int T, int32_t *counts,
                                   int32_t *offsets, int32_t *src, float *gate, int32_t *n_total,
                                   float *bias, float delta, hipStream_t s) {
  hipLaunchKernelGGL(threshold_count_kernel, dim3(B), dim3(1024), 0, s, logits, T, counts);
  const int need = (T + 1023) / 1024;
#define XMOD_THR(KPT_)                                                                         \
  hipLaunchKernelGGL((threshold_write_kernel<KPT_>), dim3(B), dim3(1024), 0, s, logits, B, T, \
                     counts, offsets, src, gate, n_total, bias, delta)
  if (need <= 1) XMOD_THR(1);
  else if (need <= 2) XMOD_THR(2);
  else if (need <= 4) XMOD_THR(4);
  else if (need <= 8) XMOD_THR(8);
  else if (need <= 16) XMOD_THR(16);
  else if (need <= 32) XMOD_THR(32);
  else XMOD_THR(64);
#undef XMOD_THR
  return hipGetLastError();
}

// ---- top-k / threshold mask agreement ([XMOD] "routing diagnostics", Table 10) -----------------

__global__ __launch_bounds__(1024) void mask_agreement_kernel(const float *__restrict__ logits,
                                                              const int32_t *__restrict__ idx,
                                                              int T, int k,
                                                              uint32_t *__restrict__ agree) {
  __shared__ uint32_t bits[65536 / 32];
  __shared__ uint32_t s_part[16];
  const int b = blockIdx.x;
  const int nw = (T + 31) / 32;
  for (int i = threadIdx.x; i < nw; i += 1024) bits[i] = 0u;
  __syncthreads();
  for (int j = threadIdx.x; j < k; j += 1024) {
    const int p = min(max(idx[(int64_t)b * k + j], 0), T - 1);
    atomicOr(&bits[p >> 5], 1u << (p & 31));
  }
  __syncthreads();
  const float *L = logits + (int64_t)b * T;
  uint32_t c = 0;
  for (int p = threadIdx.x; p < T; p += 1024) {
    const bool top = (bits[p >> 5] >> (p & 31)) & 1u;
    c += top == (L[p] >= 0.f);
  }
  const uint32_t tot = block_sum_1024(c, s_part);
  if (threadIdx.x == 0) atomicAdd(agree, tot);
}

hipError_t launch_mask_agreement(const float *logits, const int32_t *idx, int B, int T, int k,
                                 uint32_t *agree, hipStream_t s) {
  hipLaunchKernelGGL(mask_agreement_kernel, dim3(B), dim3(1024), 0, s, logits, idx, T, k, agree);
  return hipGetLastError();
}

}  // namespace xmod

