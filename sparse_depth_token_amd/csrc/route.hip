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

// The value of a key: the logit itself for every non-NaN logit (-0 comes back as +0, which
// the gate cannot tell apart), a NaN for NaN. The output phases take the gate's logit from
// here rather than loading the logits a second time.
__device__ __forceinline__ float key_value(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
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
  // (positions past T load position T-1 and are masked afterwards: a load behind a branch
  // makes the compiler wait for it before the next one is issued)
  // Loaded 16 at a time: all of a batch is in flight at once, and the batches are kept apart
  // so that the loads' registers stay bounded.
  uint32_t key[KPT];
  float bv[STRIDED ? 1 : KPT];
  constexpr int LB = KPT < 16 ? KPT : 16;
#pragma unroll
  for (int j0 = 0; j0 < KPT; j0 += LB) {
    float lraw[LB];
#pragma unroll
    for (int i = 0; i < LB; ++i) {
      const int p = pos_of(j0 + i);
      lraw[i] = L[p < T ? p : T - 1];
      if (!STRIDED) bv[j0 + i] = Bi ? Bi[p < T ? p : T - 1] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < LB; ++i) key[j0 + i] = pos_of(j0 + i) < T ? order_key(lraw[i]) : 0u;
    asm volatile("" ::: "memory");
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
          if (G) G[pos] = 1.0f / (1.0f + expf(-key_value(key[j])));
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
    uint32_t t = thr;  // opaque: the output phase recomputes the masks instead of keeping them
    asm volatile("" : "+s"(t));
    gm = __ballot(valid && key[j] > t);
    em = __ballot(valid && key[j] == t);
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
  // Output, 8 rows at a time: the rows' bias values are read first (coalesced, every
  // position), so a batch waits for one round trip rather than one per row.
  constexpr int RB = KPT < 8 ? KPT : 8;
#pragma unroll
  for (int j0 = 0; j0 < KPT; j0 += RB) {
    float bc[RB];
#pragma unroll
    for (int r = 0; r < RB; ++r) {
      const int p = pos_of(j0 + r);
      bc[r] = Bi ? Bi[p < T ? p : T - 1] : 0.f;
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
        if (G) G[pos] = 1.0f / (1.0f + expf(-key_value(key[j])));
        if (Bi) Bi[p] = __fadd_rn(bc[r], delta);
      }
    }
  }
}

// ---- top-k over several workgroups per sequence ----------------------------------------------
//
// The one-workgroup select above runs a sequence on one CU: with few, long sequences (one
// sequence of 32768 tokens) that CU issues every instruction of the select while the rest of
// the GPU idles. The chunked select cuts each sequence into chunks of 4096 positions and
// splits the work over three kernels:
//   1. one workgroup per chunk: for each value of the top 11 key bits (2048 buckets), the
//      number of the chunk's keys in that bucket or above, stored as is (no atomics across
//      workgroups, no counters to clear);
//   2. one workgroup per sequence: the sum of its chunks' counts gives the bucket of the k-th
//      largest key (the highest bucket whose count reaches k). Only the keys in that bucket (a
//      few percent of the sequence for spread-out logits) are gathered into LDS; two passes
//      over them (bits 20..10, 9..0) pin the k-th largest key exactly. Each chunk's count of
//      keys above it is its count for the bucket above plus its gathered keys above it; those
//      counts (and the counts of keys equal to it) become the number of each before every
//      chunk. When the bucket holds more keys than LDS takes (heavy ties), the two passes and
//      the counts run over all keys, held in registers.
//   3. one workgroup per chunk: its selected positions, at output slot = number of selected
//      keys before them (keys above the threshold, plus the first `need` equal keys).
// The threshold key, the tie rule and the output slots are those of the one-workgroup select,
// so both paths write identical results.

constexpr int TOPK_CHUNK = 4096;
constexpr int TOPK_CAND = 8192;  // gathered keys held in LDS (32 KiB)

struct TopkScratch {
  uint32_t *hist;      // [B][P][2048] per chunk: keys whose top 11 bits are >= the bucket
  uint32_t *base;      // [B][P][2] selected keys above / equal to the threshold before chunk c
  uint32_t *thr_need;  // [B][2] threshold key, number of keys equal to it that are selected
};

__host__ __device__ inline int64_t topk_chunks(int T) { return (T + TOPK_CHUNK - 1) / TOPK_CHUNK; }

static TopkScratch topk_scratch(void *ws, int B, int T) {
  const size_t P = (size_t)topk_chunks(T);
  char *c = (char *)ws;
  TopkScratch t;
  t.hist = (uint32_t *)c;
  t.base = (uint32_t *)(c + (size_t)B * P * 2048 * 4);
  t.thr_need = (uint32_t *)(c + (size_t)B * P * 2048 * 4 + (size_t)B * P * 8);
  return t;
}

// Thread t of a chunk's workgroup owns its positions 4t .. 4t+3 (positions past T load
// position T-1 and are masked).
__device__ __forceinline__ void chunk_keys(const float *__restrict__ L, int T, int p0,
                                           uint32_t (&key)[4], bool (&valid)[4]) {
  float l[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) l[i] = L[p0 + i < T ? p0 + i : T - 1];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    valid[i] = p0 + i < T;
    key[i] = valid[i] ? order_key(l[i]) : 0u;
  }
}

__global__ __launch_bounds__(1024) void topk_chunk_hist_kernel(const float *__restrict__ logits,
                                                               int T,
                                                               uint32_t *__restrict__ hist) {
  __shared__ uint2 h2[1024];  // 2048 buckets
  __shared__ uint32_t s_w[16];
  uint32_t *h = (uint32_t *)h2;
  const int c = blockIdx.x, b = blockIdx.y, P = gridDim.x, tid = threadIdx.x;
  const int lane = tid & 63, wid = tid >> 6;
  uint32_t key[4];
  bool valid[4];
  chunk_keys(logits + (int64_t)b * T, T, c * TOPK_CHUNK + 4 * tid, key, valid);
  h2[tid] = make_uint2(0u, 0u);
  __syncthreads();
#pragma unroll
  for (int i = 0; i < 4; ++i)
    if (valid[i]) atomicAdd(&h[key[i] >> 21], 1u);
  __syncthreads();
  // counts from the top bucket down: thread t holds buckets 2047-2t (.y) and 2046-2t (.x)
  const uint2 v = h2[1023 - tid];
  const uint32_t tot = v.x + v.y, incl = wave_incl_scan(tot);
  if (lane == 63) s_w[wid] = incl;
  __syncthreads();
  uint32_t above = incl - tot;
  for (int w = 0; w < wid; ++w) above += s_w[w];
  ((uint2 *)(hist + ((int64_t)b * P + c) * 2048))[1023 - tid] =
      make_uint2(above + v.y + v.x, above + v.y);
}

// The bucket holding the `remaining`-th largest key of a histogram whose bins thread t holds
// in descending digit order (bins nb-1-BPT*t-q, q = 0..BPT-1, in c[q]; threads past the bins
// pass 0): its digit and the rank of the wanted key within it. 1 <= remaining <= the
// histogram's total, so exactly one thread finds the bucket. Two barriers; s_w and s_pick are
// free again when it returns.
template <int BPT>
__device__ __forceinline__ void block_pick(const uint32_t (&c)[BPT], uint32_t remaining, int nb,
                                           uint32_t *s_w, uint32_t *s_pick, uint32_t &digit,
                                           uint32_t &rem_out) {
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  uint32_t tot = 0;
#pragma unroll
  for (int q = 0; q < BPT; ++q) tot += c[q];
  const uint32_t incl_w = wave_incl_scan(tot);
  if (lane == 63) s_w[wid] = incl_w;
  __syncthreads();
  uint32_t before = 0;
  for (int w = 0; w < wid; ++w) before += s_w[w];
  const uint32_t incl = before + incl_w, excl = incl - tot;
  if (excl < remaining && remaining <= incl) {
    uint32_t above = excl;
    bool found = false;
#pragma unroll
    for (int q = 0; q < BPT; ++q) {
      if (!found && remaining <= above + c[q]) {
        s_pick[0] = (uint32_t)(nb - 1 - BPT * tid - q);
        s_pick[1] = remaining - above;
        found = true;
      }
      if (!found) above += c[q];
    }
  }
  __syncthreads();
  digit = s_pick[0];
  rem_out = s_pick[1];
}

// R: rows of 1024 positions per thread (thread t holds positions t, t + 1024, ...), at least
// T / 1024; chunk c is rows 4c .. 4c+3. Every key of the sequence is loaded once, up front
// (all loads in flight together), and kept in registers.
template <int R>
__global__ __launch_bounds__(1024) void topk_threshold_kernel(const float *__restrict__ logits,
                                                              int T, int k, TopkScratch sc) {
  __shared__ uint32_t pool[TOPK_CAND];  // gathered keys, or the (row, wave) count tables
  __shared__ uint32_t h2[2048], h3[1024];
  __shared__ uint32_t s_w[16], s_w2[16], s_pick[2];
  __shared__ uint32_t s_cgt[16], s_ceq[16];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int P = (int)topk_chunks(T);  // <= 16
  const float *L = logits + (int64_t)b * T;
  // the chunks' counts summed: thread t holds those of buckets 2047-2t (C_hi) and 2046-2t (C_lo)
  const uint2 *H = (const uint2 *)(sc.hist + (int64_t)b * P * 2048);
  uint32_t C_hi = 0, C_lo = 0;
  auto sum_counts = [&]() {
    uint2 hv[16];
#pragma unroll
    for (int ch = 0; ch < 16; ++ch) hv[ch] = H[(ch < P ? ch : P - 1) * 1024 + 1023 - tid];
#pragma unroll
    for (int ch = 0; ch < 16; ++ch) {
      if (ch < P) {
        C_hi += hv[ch].y;
        C_lo += hv[ch].x;
      }
    }
  };
  // (with 64 rows of keys the counts are summed first, so that their loads and the keys'
  // are not in flight, in registers, together)
  if (R > 32) {
    sum_counts();
    asm volatile("" ::: "memory");
  }
  // the keys, 32 rows in flight at a time
  uint32_t key[R];
  constexpr int KB = R < 32 ? R : 32;
#pragma unroll
  for (int j0 = 0; j0 < R; j0 += KB) {
    float lraw[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) {
      const int p = (j0 + i) * 1024 + tid;  // p >= T for every row past the last
      lraw[i] = L[p < T ? p : T - 1];
    }
    if (R <= 32) sum_counts();
#pragma unroll
    for (int i = 0; i < KB; ++i)
      key[j0 + i] = (j0 + i) * 1024 + tid < T ? order_key(lraw[i]) : 0u;
    if (R > 32) asm volatile("" ::: "memory");
  }
  h2[2047 - 2 * tid] = C_hi;
  h2[2046 - 2 * tid] = C_lo;
  if (tid < 16) {
    s_cgt[tid] = 0u;
    s_ceq[tid] = 0u;
  }
  __syncthreads();
  // the bucket of the k-th largest key: the highest bucket whose count reaches k (the counts
  // do not increase with the bucket, the lowest is T >= k and the one above the top is 0)
  const uint32_t above_hi = tid == 0 ? 0u : h2[2048 - 2 * tid];
  const uint32_t ku = (uint32_t)k;
  if (C_hi >= ku && above_hi < ku) {
    s_pick[0] = 2047u - 2u * tid;
    s_pick[1] = ku - above_hi;
  }
  if (C_lo >= ku && C_hi < ku) {
    s_pick[0] = 2046u - 2u * tid;
    s_pick[1] = ku - C_hi;
  }
  __syncthreads();
  const uint32_t d0 = s_pick[0];
  uint32_t rem = s_pick[1];
  h2[tid] = 0u;  // (every thread has read h2 before the barrier above)
  h2[tid + 1024] = 0u;
  h3[tid] = 0u;
  // each chunk's keys in buckets above d0
  uint32_t g_above = 0;
  if (tid < P && d0 < 2047u) g_above = sc.hist[((int64_t)b * P + tid) * 2048 + d0 + 1];

  // the keys in bucket d0: this thread's count, then its offset among all of them. (Each loop
  // over the rows tests a position's range from an opaque copy of the thread id, so that the
  // compiler recomputes the tests rather than keeping one lane mask per row live throughout.)
  auto opaque_tid = [&]() {
    int t = tid;
    asm volatile("" : "+v"(t));
    return t;
  };
  uint32_t n = 0;
  {
    const int t = opaque_tid();
#pragma unroll
    for (int j = 0; j < R; ++j) n += (j * 1024 + t < T && (key[j] >> 21) == d0) ? 1u : 0u;
  }
  const uint32_t n_incl = wave_incl_scan(n);
  if (lane == 63) s_w2[wid] = n_incl;
  __syncthreads();
  uint32_t off = n_incl - n, total = 0;
  for (int w = 0; w < 16; ++w) {
    const uint32_t v = s_w2[w];
    off += w < wid ? v : 0u;
    total += v;
  }

  uint32_t thr, need;
  if (total <= (uint32_t)TOPK_CAND) {
    // gathered entry: chunk << 21 | the key's low 21 bits (its top 11 bits are d0)
    const int t = opaque_tid();
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j * 1024 + t < T && (key[j] >> 21) == d0)
        pool[off++] = ((uint32_t)(j >> 2) << 21) | (key[j] & 0x1FFFFFu);
    __syncthreads();
    for (uint32_t i = tid; i < total; i += 1024) atomicAdd(&h2[(pool[i] >> 10) & 2047u], 1u);
    __syncthreads();
    uint32_t c2[2] = {h2[2047 - 2 * tid], h2[2046 - 2 * tid]};
    uint32_t d1;
    block_pick<2>(c2, rem, 2048, s_w, s_pick, d1, rem);
    for (uint32_t i = tid; i < total; i += 1024) {
      const uint32_t e = pool[i];
      if (((e >> 10) & 2047u) == d1) atomicAdd(&h3[e & 1023u], 1u);
    }
    __syncthreads();
    uint32_t c3[1] = {h3[1023 - tid]};
    uint32_t d2;
    block_pick<1>(c3, rem, 1024, s_w, s_pick, d2, rem);
    const uint32_t tl = (d1 << 10) | d2;
    thr = (d0 << 21) | tl;
    need = rem;
    for (uint32_t i = tid; i < total; i += 1024) {
      const uint32_t e = pool[i], lo = e & 0x1FFFFFu, ch = e >> 21;
      if (lo > tl) atomicAdd(&s_cgt[ch], 1u);
      else if (lo == tl) atomicAdd(&s_ceq[ch], 1u);
    }
    __syncthreads();
    if (wid == 0) {  // lanes 0..15: chunk counts, exclusive prefix over the chunks
      uint32_t g = 0, q = 0;
      if (lane < P) {
        g = g_above + s_cgt[lane];
        q = s_ceq[lane];
      }
      const uint32_t g_incl = wave_incl_scan(g), q_incl = wave_incl_scan(q);
      if (lane < P) {
        uint32_t *B2 = sc.base + ((int64_t)b * P + lane) * 2;
        B2[0] = g_incl - g;
        B2[1] = q_incl - q;
      }
    }
  } else {
    // heavy ties: the two passes and the counts over every key in registers
    int t = opaque_tid();
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j * 1024 + t < T && (key[j] >> 21) == d0) atomicAdd(&h2[(key[j] >> 10) & 2047u], 1u);
    __syncthreads();
    uint32_t c2[2] = {h2[2047 - 2 * tid], h2[2046 - 2 * tid]};
    uint32_t d1;
    block_pick<2>(c2, rem, 2048, s_w, s_pick, d1, rem);
    const uint32_t pre = (d0 << 11) | d1;  // key >> 10 of the k-th largest
    t = opaque_tid();
#pragma unroll
    for (int j = 0; j < R; ++j)
      if (j * 1024 + t < T && (key[j] >> 10) == pre) atomicAdd(&h3[key[j] & 1023u], 1u);
    __syncthreads();
    uint32_t c3[1] = {h3[1023 - tid]};
    uint32_t d2;
    block_pick<1>(c3, rem, 1024, s_w, s_pick, d2, rem);
    thr = (pre << 10) | d2;
    need = rem;
    // per (row, wave) counts of keys above and equal to the threshold: pool[e], pool[1024 + e]
    t = opaque_tid();
#pragma unroll
    for (int j = 0; j < R; ++j) {
      const bool valid = j * 1024 + t < T;
      uint32_t th = thr;  // opaque, so that the row masks are not all kept live together
      asm volatile("" : "+v"(th));
      const unsigned long long gm = __ballot(valid && key[j] > th);
      const unsigned long long em = __ballot(valid && key[j] == th);
      if (lane == 0) {
        pool[j * 16 + wid] = (uint32_t)__popcll(gm);
        pool[1024 + j * 16 + wid] = (uint32_t)__popcll(em);
      }
    }
    __syncthreads();
    // exclusive prefix over the entries (row, wave) in position order; entry (4c, 0), held by
    // thread 64c, is the count before chunk c
    const int rows = (T + 1023) / 1024;
    const bool has = tid < rows * 16;
    const uint32_t g = has ? pool[tid] : 0u, q = has ? pool[1024 + tid] : 0u;
    const uint32_t g_incl = wave_incl_scan(g), q_incl = wave_incl_scan(q);
    if (lane == 63) {
      s_w[wid] = g_incl;
      s_w2[wid] = q_incl;
    }
    __syncthreads();
    uint32_t g_base = 0, q_base = 0;
    for (int w = 0; w < wid; ++w) {
      g_base += s_w[w];
      q_base += s_w2[w];
    }
    if (has && lane == 0) {
      uint32_t *B2 = sc.base + ((int64_t)b * P + wid) * 2;
      B2[0] = g_base + g_incl - g;
      B2[1] = q_base + q_incl - q;
    }
  }
  if (tid == 0) {
    sc.thr_need[2 * b] = thr;
    sc.thr_need[2 * b + 1] = need;
  }
}

__global__ __launch_bounds__(1024) void topk_emit_kernel(const float *__restrict__ logits, int T,
                                                         int k, TopkScratch sc,
                                                         int32_t *__restrict__ idx,
                                                         float *__restrict__ gate,
                                                         float *__restrict__ bias, float delta) {
  __shared__ uint32_t s_gt[16], s_eq[16];
  const int c = blockIdx.x, b = blockIdx.y, P = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, wid = tid >> 6;
  const int p0 = c * TOPK_CHUNK + 4 * tid;
  uint32_t key[4];
  bool valid[4];
  chunk_keys(logits + (int64_t)b * T, T, p0, key, valid);
  float *const Bi = bias ? bias + (int64_t)b * T : nullptr;
  float bv[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) bv[i] = Bi ? Bi[p0 + i < T ? p0 + i : T - 1] : 0.f;
  const uint32_t thr = sc.thr_need[2 * b], need = sc.thr_need[2 * b + 1];
  const uint32_t *B2 = sc.base + ((int64_t)b * P + c) * 2;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    gt += valid[i] && key[i] > thr;
    eq += valid[i] && key[i] == thr;
  }
  const uint32_t gt_incl = wave_incl_scan(gt), eq_incl = wave_incl_scan(eq);
  if (lane == 63) {
    s_gt[wid] = gt_incl;
    s_eq[wid] = eq_incl;
  }
  __syncthreads();
  uint32_t gb = B2[0], eb = B2[1];
  for (int w = 0; w < wid; ++w) {
    gb += s_gt[w];
    eb += s_eq[w];
  }
  const uint32_t gt_before = gb + gt_incl - gt;
  uint32_t eq_seen = eb + eq_incl - eq;
  uint32_t pos = gt_before + (eq_seen < need ? eq_seen : need);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (!valid[i]) continue;
    bool sel = key[i] > thr;
    if (key[i] == thr) {
      sel = eq_seen < need;
      ++eq_seen;
    }
    if (sel && pos < (uint32_t)k) {  // pos < k always holds; the bound only guards idx
      idx[(int64_t)b * k + pos] = p0 + i;
      if (gate) gate[(int64_t)b * k + pos] = 1.0f / (1.0f + expf(-key_value(key[i])));
      if (Bi) Bi[p0 + i] = __fadd_rn(bv[i], delta);
      ++pos;
    }
  }
}

// Whether sequences of T positions take the chunked select: longer than 8192 positions (shorter
// ones finish on one workgroup about as fast as three launches take). Large batches run in
// groups of at most 4096 chunks (32 MiB of counts), one group after another on the stream,
// reusing the scratch.
static bool topk_chunked(int T) { return T > 8192 && T <= 65536; }

static int topk_group(int B, int T) {
  const int g = (int)(4096 / topk_chunks(T));
  return B < g ? B : g;
}

size_t topk_scratch_bytes(int B, int T) {
  if (B < 1 || T < 1 || !topk_chunked(T)) return 0;
  const size_t P = (size_t)topk_chunks(T), G = (size_t)topk_group(B, T);
  return G * P * 2048 * 4 + G * P * 8 + G * 8;
}

hipError_t launch_topk(const float *logits, int B, int T, int k, int32_t *idx, float *gate,
                       float *bias, float delta, hipStream_t s, void *scratch) {
  if (scratch && topk_chunked(T)) {
    const int G = topk_group(B, T);
    const TopkScratch sc = topk_scratch(scratch, G, T);
    const int rows = (T + 1023) / 1024;
    for (int b0 = 0; b0 < B; b0 += G) {
      const int nb = B - b0 < G ? B - b0 : G;
      const float *lg = logits + (int64_t)b0 * T;
      int32_t *ix = idx + (int64_t)b0 * k;
      float *gt = gate ? gate + (int64_t)b0 * k : nullptr;
      float *bs = bias ? bias + (int64_t)b0 * T : nullptr;
      const dim3 grid((unsigned)topk_chunks(T), (unsigned)nb);
      hipLaunchKernelGGL(topk_chunk_hist_kernel, grid, dim3(1024), 0, s, lg, T, sc.hist);
      if (rows <= 16)
        hipLaunchKernelGGL(topk_threshold_kernel<16>, dim3(nb), dim3(1024), 0, s, lg, T, k, sc);
      else if (rows <= 32)
        hipLaunchKernelGGL(topk_threshold_kernel<32>, dim3(nb), dim3(1024), 0, s, lg, T, k, sc);
      else
        hipLaunchKernelGGL(topk_threshold_kernel<64>, dim3(nb), dim3(1024), 0, s, lg, T, k, sc);
      hipLaunchKernelGGL(topk_emit_kernel, grid, dim3(1024), 0, s, lg, T, k, sc, ix, gt, bs,
                         delta);
    }
    return hipGetLastError();
  }
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

