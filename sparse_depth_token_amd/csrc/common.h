// Device helpers and internal launcher declarations shared by the HIP sources of the X-MoD
// layer library (gfx950, wave64). Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>


namespace xmod {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// bf16 <-> fp32. Widening is exact; narrowing rounds to nearest even.
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
// gfx950 converts in hardware (v_cvt_pk_bf16_f32: round to nearest even, two values at once).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, (__bf16)f);
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}
// The same rounding in integer arithmetic (identical bits for finite inputs), for code whose
// register allocation the conversion instruction's pairing upsets.
__device__ __forceinline__ uint32_t pack_bf16x2_int(float lo, float hi) {
  uint32_t a = __float_as_uint(lo), b = __float_as_uint(hi);
  a += 0x7FFFu + ((a >> 16) & 1u);
  b += 0x7FFFu + ((b >> 16) & 1u);
  return (a >> 16) | (b & 0xFFFF0000u);
}
// Unpack 8 bf16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8(const uint4 &v, float *f) {
  f[0] = __uint_as_float(v.x << 16); f[1] = __uint_as_float(v.x & 0xFFFF0000u);
  f[2] = __uint_as_float(v.y << 16); f[3] = __uint_as_float(v.y & 0xFFFF0000u);
  f[4] = __uint_as_float(v.z << 16); f[5] = __uint_as_float(v.z & 0xFFFF0000u);
  f[6] = __uint_as_float(v.w << 16); f[7] = __uint_as_float(v.w & 0xFFFF0000u);
}
__device__ __forceinline__ uint4 pack8(const float *f) {
  return make_uint4(pack_bf16x2(f[0], f[1]), pack_bf16x2(f[2], f[3]),
                    pack_bf16x2(f[4], f[5]), pack_bf16x2(f[6], f[7]));
}
__device__ __forceinline__ uint4 pack8_int(const float *f) {
  return make_uint4(pack_bf16x2_int(f[0], f[1]), pack_bf16x2_int(f[2], f[3]),
                    pack_bf16x2_int(f[4], f[5]), pack_bf16x2_int(f[6], f[7]));
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}

// Gated residual of one element, in the fixed order g = varsigma*r, t = a + f, p = g*t,
// y = X + p, each rounded in fp32 (no contraction). Shared by the standalone scatter and the
// fused down-projection epilogue so both give identical bits.
__device__ __forceinline__ float gated_residual(float X, float g, float a, float f) {
  const float t = __fadd_rn(a, f);
  const float p = __fmul_rn(g, t);
  return __fadd_rn(X, p);
}
// Dense residual: y = X + (a + f).
__device__ __forceinline__ float dense_residual(float X, float a, float f) {
  return __fadd_rn(X, __fadd_rn(a, f));
}
// MoD's residual of a routed token: the attention output enters ungated, the FFN output gated
// by the router score r: y = (X + a) + r*f, each operation rounded in fp32.
__device__ __forceinline__ float mod_residual(float X, float r, float a, float f) {
  return __fadd_rn(__fadd_rn(X, a), __fmul_rn(r, f));
}

}  // namespace xmod

// ---- packed-row map -------------------------------------------------------------------------
namespace xmod {

// Packed row m of a layer -> row of the hidden state x, viewed as [B*T, d]:
//  * src != nullptr: x row src[m] (eval-time threshold routing: sequences route different
//    numbers of tokens, so rows are listed flat and their count n_dev lives on the device);
//  * idx != nullptr: x row (m / k) * T + idx[m] (top-k routing, k rows per sequence);
//  * otherwise m (dense layer: every row).
// Rows outside [0, x_rows) (a caller error) are clamped so that no access leaves x.
struct RowMap {
  const int32_t *idx = nullptr;
  const int32_t *src = nullptr;
  const int32_t *n_dev = nullptr;  // device-side number of packed rows, or nullptr
  int T = 0, k = 0;
  int64_t x_rows = 0;
};

__device__ __forceinline__ int64_t rowmap_x(const RowMap &r, int64_t m) {
  int64_t row;
  if (r.src) row = r.src[m];
  else if (r.idx) row = (m / r.k) * r.T + min(max(r.idx[m], 0), r.T - 1);
  else row = m;
  return min(max(row, (int64_t)0), r.x_rows - 1);
}
// Number of packed rows: the device count when there is one (never above the launch bound).
__device__ __forceinline__ int64_t rowmap_count(const RowMap &r, int64_t bound) {
  return r.n_dev ? min((int64_t)*r.n_dev, bound) : bound;
}

}  // namespace xmod

// ---- launchers (host side, defined in the .hip files) ---------------------------------------
namespace xmod {

// logits = s - tau*b in fp32; s_out (optional) receives s = w.x + beta itself.
hipError_t launch_router(const uint16_t *x, const uint16_t *w, float beta, const float *bias,
                         float tau, float *logits, int64_t rows, int d, hipStream_t s,
                         float *s_out = nullptr);

// Top-k of each sequence's logits (ascending positions, ties to the lower position). With
// scratch (topk_scratch_bytes(B, T) bytes; 0 means none is used) long sequences are split over
// several workgroups; the result is the same either way.
hipError_t launch_topk(const float *logits, int B, int T, int k, int32_t *idx, float *gate,
                       float *bias, float delta, hipStream_t s, void *scratch = nullptr);
size_t topk_scratch_bytes(int B, int T);

// Eval-time threshold routing: per sequence the tokens with logit >= 0, packed flat in
// sequence order (counts[b], offsets[b], src[m] = b*T + t, gate[m] = sigmoid(logit)), the
// total in *n_total, and bias[b*T + t] += delta for every selected token.
hipError_t launch_threshold_select(const float *logits, int B, int T, int32_t *counts,
                                   int32_t *offsets, int32_t *src, float *gate, int32_t *n_total,
                                   float *bias, float delta, hipStream_t s);

// Adds to *agree the number of positions where the top-k mask (idx [B, k]) and the threshold
// mask (logit >= 0) take the same decision.
hipError_t launch_mask_agreement(const float *logits, const int32_t *idx, int B, int T, int k,
                                 uint32_t *agree, hipStream_t s);

// Gather rows (via the row map) and optionally RMSNorm them. rows: launch bound. With
// normalize, xraw (optional) also receives the gathered rows themselves.
hipError_t launch_gather_rows(const uint16_t *x, const RowMap &map, const uint16_t *gain,
                              float eps, bool normalize, int64_t rows, int d, uint16_t *out,
                              hipStream_t s, uint16_t *xraw = nullptr);

// v[m] = RMSNorm(X[m] + a[m]; gain), X gathered from x via the row map; a fp32.
hipError_t launch_residual_rmsnorm(const uint16_t *x, const RowMap &map, const float *a,
                                   const uint16_t *gain, float eps, int64_t rows, int d,
                                   uint16_t *v, hipStream_t s);

// Standalone gated scatter (gate != nullptr) or dense residual (gate == nullptr).
hipError_t launch_scatter(uint16_t *x, const RowMap &map, const float *gate, float varsigma,
                          const uint16_t *a, const uint16_t *f, int64_t rows, int d,
                          hipStream_t s);

// In place on the packed [Q | K | V] rows (row m of M, or of the device count): per-head RMSNorm
// of the queries (q_norm) and keys (k_norm), when given, then the rotary embedding at each
// row's original position (x row % T) when theta > 0. V is untouched.
hipError_t launch_qk_form(uint16_t *qkv, int ld_qkv, const RowMap &map, int64_t rows, int Hq,
                          int Hkv, int hd, const uint16_t *q_norm, const uint16_t *k_norm,
                          float eps, float theta, hipStream_t s);

enum GemmEpilogue {
  EPI_STORE = 0, EPI_SWIGLU = 1, EPI_RESIDUAL = 2, EPI_STORE_F32 = 3,
  EPI_SWIGLU_SAVE = 4,  // EPI_SWIGLU that also stores the pre-activations [zg | zu] to Z
  EPI_SWIGLU_BWD = 5    // accumulator dg; reads Z = [zg | zu], writes C = [dzg | dzu]
};

// Operand layouts: A is [M, K] (k-contiguous rows) or, k-major, [K, M]; B is [N, K] or,
// k-major, [K, N]. NT: both k-contiguous; NN: B k-major; TN: both k-major.
enum GemmLayout { LAY_NT = 0, LAY_NN = 1, LAY_TN = 2 };

struct GemmArgs {
  const uint16_t *A;  int lda;     // [M, K] activations
  const uint16_t *B;  int ldb;     // [N, K] weights (EPI_SWIGLU: gate weights, N = F)
  const uint16_t *B2;              // EPI_SWIGLU: up weights [N, K], same ldb
  uint16_t *C;        int ldc;     // EPI_STORE / EPI_SWIGLU bf16 output [M, N]
  float *Cf;                       // EPI_STORE_F32 fp32 output [M, N], same ldc
  int M, N, K;                     // M: rows, or their upper bound when map.n_dev is set
  // Rows: map.n_dev (when set) holds the actual row count on the device; the grid covers M
  // and workgroups past the actual tiles exit at once.
  // EPI_RESIDUAL: output row m is x row rowmap_x(map, m); the accumulator is f (kept fp32),
  // added as X + varsigma*gate[m]*(a + f), or X + (a + f) if gate == nullptr; a is fp32
  // [M, N] with leading dimension ldc, as is x, or nullptr for a = 0.
  RowMap map;
  uint16_t *x; const float *gate; float varsigma; const float *a;
  int residual_form;  // EPI_RESIDUAL with gate: 0 X + (varsigma*gate)*(a + f); 1 (X + a) + gate*f
  float *fsave;       // EPI_RESIDUAL: when set, f is also stored (fp32 [M, N], ldc)
  // k-major B (LAY_NN): k-rows >= K1 (when K1 > 0) are rows k - K1 of B2 (same ldb).
  int K1;
  // EPI_STORE_F32: output rows m >= M1 (when M1 > 0) go to row m - M1 of Cf2 (same ldc).
  float *Cf2; int M1;
  // EPI_SWIGLU_SAVE / EPI_SWIGLU_BWD: pre-activations, zg in columns [0, N), zu in [N, 2N).
  uint16_t *Z; int ldz;
};

hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, hipStream_t s);
// Layout-aware form: k-major operands need their M / N a multiple of 8 (at least 8) and K a
// multiple of 64; LAY_NN supports EPI_STORE, EPI_STORE_F32, EPI_SWIGLU_BWD; LAY_TN EPI_STORE_F32.
hipError_t launch_gemm(const GemmArgs &g, GemmEpilogue epi, GemmLayout lay, hipStream_t s);

// Causal attention over packed sequences: fixed length k (seq_len == nullptr, sequence b at
// rows b*k) or per-sequence lengths and first rows (seq_len[b], seq_off[b], each <= max_len).
hipError_t launch_attention(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, int B, int k,
                            int Hq, int Hkv, int hd, const int32_t *seq_off,
                            const int32_t *seq_len, hipStream_t s);

// launch_attention for fixed-length sequences that also stores lse[row * Hq + h], the log2 of
// each query's softmax normaliser in the units of the weights (P = exp2(score * scale_log2 - lse)).
hipError_t launch_attention_lse(const uint16_t *qkv, int ld_qkv, uint16_t *o, int ld_o, float *lse,
                                int B, int k, int Hq, int Hkv, int hd, hipStream_t s);

// Backward of launch_attention_lse for fixed-length sequences: D[row * Hq + h] (fp32 scratch)
// and dqkv = [dQ | dK | dV] bf16 rows (ld_dqkv), every column written.
hipError_t launch_attention_bwd(const uint16_t *qkv, int ld_qkv, const uint16_t *o, int ld_o,
                                const float *lse, const uint16_t *dO, int ld_do, float *D,
                                uint16_t *dqkv, int ld_dqkv, int B, int k, int Hq, int Hkv,
                                int hd, hipStream_t s);

// ---- backward row kernels (rows_bwd.hip) ----
hipError_t launch_zero(void *p, size_t bytes, hipStream_t s);          // bytes / 16 chunks
hipError_t launch_copy32(void *dst, const void *src, int64_t n_words, hipStream_t s);
int bwd_row_wgs();    // workgroups (= partial rows written) of the packed-row kernels
int bwd_route_wgs();  // workgroups (= partial rows written) of the every-token router kernel
// out[c] = scale * sum over p < n_part of part[p * n + c], in a fixed order; tmp: 16 * n floats.
struct ColsumJob {
  const float *part; int n_part; int n; float *out; float scale; float *tmp; int blk0;
};
struct ColsumJobs { ColsumJob job[6]; int n; };
hipError_t launch_colsum_multi(ColsumJobs jobs, hipStream_t s);
hipError_t launch_resid_bwd(const uint16_t *dy, const RowMap &map, const float *a, const float *f,
                            const float *gate, float varsigma, int d, int64_t M, int64_t M_pad,
                            uint16_t *dt, float *dell, float *dell_tok, uint8_t *q_tok,
                            float *vs_part, hipStream_t s);
hipError_t launch_rms2_bwd(const uint16_t *dy, const RowMap &map, const uint16_t *X,
                           const float *a, const float *dv, const uint16_t *gain, float eps,
                           const uint16_t *dt, int d, int64_t M, int64_t M_pad, uint16_t *da,
                           float *dXacc, float *g_part, hipStream_t s);
hipError_t launch_rms1_bwd(const uint16_t *X, const RowMap &map, const float *du,
                           const uint16_t *gain, float eps, const float *dXacc,
                           const float *s_tok, const float *dell, float coef_n,
                           const uint16_t *w_r, int d, int64_t M, uint16_t *dx, float *g_part,
                           float *wr_part, hipStream_t s);
hipError_t launch_route_bwd(const uint16_t *x, const uint16_t *dy, const float *s_tok,
                            const float *dell_tok, const uint8_t *q_tok, float coef_n,
                            const uint16_t *w_r, int d, int64_t rows, uint16_t *dx,
                            float *wr_part, float *beta_part, float *loss_part, hipStream_t s);

// Selected-Q/full-KV attention: queries q [B*k, ld_q] (packed, Hq heads), keys and values of
// every position kv [B*T, ld_kv] ([K heads | V heads]); packed query b*k + j sits at original
// position qpos[b*k + j] and sees keys at positions <= it.
hipError_t launch_attention_fullkv(const uint16_t *q, int ld_q, const uint16_t *kv, int ld_kv,
                                   const int32_t *qpos, uint16_t *o, int ld_o, int B, int k,
                                   int T, int Hq, int Hkv, int hd, hipStream_t s);

}  // namespace xmod
