// C ABI of the X-MoD sparse-depth layer library: argument validation, workspace planning and
// the order in which the kernels of one layer, or of a stack of layers, are enqueued.
// Semantics of every entry point are documented in include/xmod.h.
#include <math.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <vector>

#include "xmod.h"
#include "common.h"

using namespace xmod;

namespace {

thread_local int32_t g_last_hip = 0;

#define XMOD_HIP(expr)                 \
  do {                                 \
    hipError_t e_ = (expr);            \
    if (e_ != hipSuccess) {            \
      g_last_hip = (int32_t)e_;        \
      return XMOD_ERR_HIP;             \
    }                                  \
  } while (0)

// ---- measurement hook: events between kernels (see xmod_phase_timing_enable) ----
// Boundary b of a call lies after kernel slot first_slot + b - 1 and before slot first_slot + b;
// an event is recorded there when either neighbouring slot is selected by the mask.
struct PhaseCall {
  int first_slot = 0, n_bound = 0;
  std::vector<std::pair<int, size_t>> ev;  // (boundary, event index)
};
struct PhaseLog {
  bool on = false;
  uint32_t mask = 0xFFFFFFFFu;
  std::vector<hipEvent_t> pool;
  size_t used = 0;
  std::vector<PhaseCall> calls;
};
PhaseLog g_phase;

void phase_mark(hipStream_t s) {
  if (!g_phase.on || g_phase.calls.empty()) return;
  PhaseCall &c = g_phase.calls.back();
  const int b = c.n_bound++;
  auto sel = [](int slot) { return slot >= 0 && slot < 32 && ((g_phase.mask >> slot) & 1u); };
  if (!sel(c.first_slot + b - 1) && !sel(c.first_slot + b)) return;
  if (g_phase.used == g_phase.pool.size()) {
    hipEvent_t e;
    // timing only: no system-scope fence (its cache write-back would stall the next kernel)
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return;
    g_phase.pool.push_back(e);
  }
  if (hipEventRecord(g_phase.pool[g_phase.used], s) != hipSuccess) return;
  c.ev.emplace_back(b, g_phase.used);
  ++g_phase.used;
}
void phase_begin(hipStream_t s, int first_slot) {
  if (!g_phase.on) return;
  g_phase.calls.emplace_back();
  g_phase.calls.back().first_slot = first_slot;
  phase_mark(s);
}

constexpr size_t kAlign = 256;
size_t align_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

xmod_status check_dims(const xmod_dims *dm) {
  if (!dm) return XMOD_ERR_INVALID_ARG;
  if (dm->B < 1 || dm->T < 1 || dm->d < 1 || dm->n_q_heads < 1 || dm->n_kv_heads < 1 ||
      dm->head_dim < 1 || dm->ffn_hidden < 1)
    return XMOD_ERR_INVALID_ARG;
  if (dm->n_q_heads % dm->n_kv_heads != 0) return XMOD_ERR_INVALID_ARG;
  if (!(dm->rms_eps >= 0.f) || !isfinite(dm->rms_eps)) return XMOD_ERR_INVALID_ARG;
  if (dm->head_dim != 64 && dm->head_dim != 128) return XMOD_ERR_UNSUPPORTED;
  if (dm->d % 64 != 0 || dm->ffn_hidden % 64 != 0 || dm->d > 8192) return XMOD_ERR_UNSUPPORTED;
  if (dm->T > 65536) return XMOD_ERR_UNSUPPORTED;
  return XMOD_OK;
}

// The GEMMs address their operands with 32-bit byte offsets (one buffer resource per
// operand), so every matrix a layer multiplies must hold fewer than 2^31 elements: the
// activations of M rows ([M, d], [M, dq + 2 dkv], [M, dq], and [M, 2F] for the training
// forward's saved pre-activations, M padded to 64 for the weight gradients) and the weights.
xmod_status check_rows(const xmod_dims *dm, int64_t M) {
  const int64_t lim = (int64_t)1 << 31;
  const int64_t dq = (int64_t)dm->n_q_heads * dm->head_dim;
  const int64_t nqkv = dq + 2LL * dm->n_kv_heads * dm->head_dim;
  const int64_t width = std::max({(int64_t)dm->d, nqkv, (int64_t)2 * dm->ffn_hidden});
  if ((M + 64) * width >= lim) return XMOD_ERR_UNSUPPORTED;
  if (nqkv * dm->d >= lim || dq * dm->d >= lim || (int64_t)dm->ffn_hidden * dm->d >= lim)
    return XMOD_ERR_UNSUPPORTED;
  return XMOD_OK;
}

bool layer_ok(const xmod_layer *L, bool sparse) {
  if (!L) return false;
  if (sparse && !L->w_router) return false;
  if (!L->g_attn || !L->w_qkv || !L->w_o || !L->g_ffn || !L->w_gate || !L->w_up || !L->w_down)
    return false;
  if (!isfinite(L->router_bias) || !isfinite(L->varsigma)) return false;
  if (L->residual != 0 && L->residual != 1) return false;
  if (!(L->rope_theta >= 0.f) || !isfinite(L->rope_theta)) return false;
  return true;
}

struct Plan {
  size_t logits = 0, idx = 0, gate = 0, u = 0, qkv = 0, o = 0, a = 0, g = 0, total = 0;
  size_t topk = 0;                               // scratch of the chunked top-k (may be empty)
  size_t counts = 0, offsets = 0, n_total = 0;  // threshold routing
};

// Workspace layout of one layer with (at most) M routed rows (offsets 256-byte aligned).
Plan plan_layer(const xmod_dims *dm, int64_t M, bool sparse, bool threshold = false) {
  Plan p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  const int64_t dq = (int64_t)dm->n_q_heads * dm->head_dim;
  const int64_t nqkv = dq + 2LL * dm->n_kv_heads * dm->head_dim;
  if (sparse) {
    p.logits = take((size_t)dm->B * dm->T * 4);
    p.idx = take((size_t)M * 4);
    p.gate = take((size_t)M * 4);
    if (!threshold) p.topk = take(topk_scratch_bytes(dm->B, dm->T));
  }
  if (threshold) {
    p.counts = take((size_t)dm->B * 4);
    p.offsets = take((size_t)dm->B * 4);
    p.n_total = take(4);
  }
  p.u = take((size_t)M * dm->d * 2);
  p.qkv = take((size_t)M * nqkv * 2);
  p.o = take((size_t)M * dq * 2);
  p.a = take((size_t)M * dm->d * 4);
  p.g = take((size_t)M * dm->ffn_hidden * 2);
  p.total = off;
  return p;
}

template <typename T>
T *at(void *ws, size_t off) { return reinterpret_cast<T *>(static_cast<char *>(ws) + off); }

// Attention, FFN and the residual write-back for the packed rows of the row map (M rows, or
// at most M with a device-side count): the attention sees sequences of k rows each, or of
// seq_len[b] rows from seq_off[b] (at most k). gate == nullptr selects the dense residual
// y = x + (a + f).
xmod_status run_body(uint16_t *x, const RowMap &map, int64_t M, const int32_t *seq_off,
                     const int32_t *seq_len, const float *gate, const xmod_layer *L,
                     const xmod_dims *dm, int k, const Plan &p, void *ws, hipStream_t s) {
  const int B = dm->B, d = dm->d;
  const int dq = dm->n_q_heads * dm->head_dim;
  const int nqkv = dq + 2 * dm->n_kv_heads * dm->head_dim;
  uint16_t *u = at<uint16_t>(ws, p.u), *qkv = at<uint16_t>(ws, p.qkv), *o = at<uint16_t>(ws, p.o);
  float *a = at<float>(ws, p.a);
  uint16_t *gbuf = at<uint16_t>(ws, p.g);

  XMOD_HIP(launch_gather_rows(x, map, (const uint16_t *)L->g_attn, dm->rms_eps, true, M, d, u, s));
  phase_mark(s);
  GemmArgs g{};
  g.map = map;
  g.A = u; g.lda = d; g.B = (const uint16_t *)L->w_qkv; g.ldb = d; g.C = qkv; g.ldc = nqkv;
  g.M = (int)M; g.N = nqkv; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, s));
  phase_mark(s);
  // optional QK-norm / rotary embedding (timed with the attention slot)
  XMOD_HIP(launch_qk_form(qkv, nqkv, map, M, dm->n_q_heads, dm->n_kv_heads, dm->head_dim,
                          (const uint16_t *)L->q_norm, (const uint16_t *)L->k_norm, dm->rms_eps,
                          L->rope_theta, s));
  XMOD_HIP(launch_attention(qkv, nqkv, o, dq, B, k, dm->n_q_heads, dm->n_kv_heads, dm->head_dim,
                            seq_off, seq_len, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = o; g.lda = dq; g.B = (const uint16_t *)L->w_o; g.ldb = dq; g.Cf = a; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = dq;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, s));
  phase_mark(s);
  XMOD_HIP(launch_residual_rmsnorm(x, map, a, (const uint16_t *)L->g_ffn, dm->rms_eps, M, d, u, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = u; g.lda = d; g.B = (const uint16_t *)L->w_gate; g.B2 = (const uint16_t *)L->w_up;
  g.ldb = d; g.C = gbuf; g.ldc = dm->ffn_hidden; g.M = (int)M; g.N = dm->ffn_hidden; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_SWIGLU, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = gbuf; g.lda = dm->ffn_hidden; g.B = (const uint16_t *)L->w_down; g.ldb = dm->ffn_hidden;
  g.ldc = d; g.M = (int)M; g.N = d; g.K = dm->ffn_hidden;
  g.x = x; g.gate = gate; g.varsigma = L->varsigma; g.a = a; g.residual_form = L->residual;
  XMOD_HIP(launch_gemm(g, EPI_RESIDUAL, s));
  phase_mark(s);
  return XMOD_OK;
}

RowMap topk_map(const int32_t *idx, const xmod_dims *dm, int k) {
  RowMap m;
  m.idx = idx; m.T = dm->T; m.k = k; m.x_rows = (int64_t)dm->B * dm->T;
  return m;
}

xmod_status sparse_layer(void *x, const xmod_layer *L, const xmod_dims *dm, int32_t K,
                         float *bias, float tau, float delta, int32_t *idx_out, float *gate_out,
                         void *ws, hipStream_t s) {
  const int k = dm->T / K;
  const int64_t M = (int64_t)dm->B * k;
  const Plan p = plan_layer(dm, M, true);
  float *logits = at<float>(ws, p.logits);
  int32_t *idx = idx_out ? idx_out : at<int32_t>(ws, p.idx);
  float *gate = gate_out ? gate_out : at<float>(ws, p.gate);
  phase_begin(s, 0);
  XMOD_HIP(launch_router((const uint16_t *)x, (const uint16_t *)L->w_router, L->router_bias, bias,
                         tau, logits, (int64_t)dm->B * dm->T, dm->d, s));
  phase_mark(s);
  XMOD_HIP(launch_topk(logits, dm->B, dm->T, k, idx, gate, bias, delta, s, at<void>(ws, p.topk)));
  phase_mark(s);
  return run_body((uint16_t *)x, topk_map(idx, dm, k), M, nullptr, nullptr, gate, L, dm, k, p,
                  ws, s);
}

// Eval-time causal threshold routing: router, selection of every token with ell >= 0, then the
// same body over the flat list of selected rows (count known only on the device; the
// launches cover all B*T rows and surplus workgroups exit at once).
xmod_status sparse_layer_threshold(void *x, const xmod_layer *L, const xmod_dims *dm,
                                   float *bias, float tau, float delta, int32_t *src_out,
                                   int32_t *counts_out, int32_t *n_total_out, void *ws,
                                   hipStream_t s) {
  const int64_t M = (int64_t)dm->B * dm->T;
  const Plan p = plan_layer(dm, M, true, true);
  float *logits = at<float>(ws, p.logits);
  int32_t *src = src_out ? src_out : at<int32_t>(ws, p.idx);
  float *gate = at<float>(ws, p.gate);
  int32_t *counts = counts_out ? counts_out : at<int32_t>(ws, p.counts);
  int32_t *offsets = at<int32_t>(ws, p.offsets);
  int32_t *n_total = n_total_out ? n_total_out : at<int32_t>(ws, p.n_total);
  phase_begin(s, 0);
  XMOD_HIP(launch_router((const uint16_t *)x, (const uint16_t *)L->w_router, L->router_bias, bias,
                         tau, logits, M, dm->d, s));
  phase_mark(s);
  XMOD_HIP(launch_threshold_select(logits, dm->B, dm->T, counts, offsets, src, gate, n_total,
                                   bias, delta, s));
  phase_mark(s);
  RowMap map;
  map.src = src; map.n_dev = n_total; map.T = dm->T; map.x_rows = M;
  return run_body((uint16_t *)x, map, M, offsets, counts, gate, L, dm, dm->T, p, ws, s);
}

xmod_status dense_layer(void *x, const xmod_layer *L, const xmod_dims *dm, void *ws,
                        hipStream_t s) {
  const Plan p = plan_layer(dm, (int64_t)dm->B * dm->T, false);
  phase_begin(s, 2);
  RowMap map;
  map.T = dm->T; map.x_rows = (int64_t)dm->B * dm->T;
  return run_body((uint16_t *)x, map, (int64_t)dm->B * dm->T, nullptr, nullptr, nullptr, L, dm,
                  dm->T, p, ws, s);
}

__global__ void zero_f32_kernel(float *p, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

int block_sparse_per_block(float A, int32_t K, bool *ok) {
  const double ak = (double)A * (double)K;
  const double r = nearbyint(ak);
  *ok = isfinite(ak) && fabs(ak - r) <= 1e-6 && r >= 0 && r <= 1e6;
  return (int)r;
}

}  // namespace


// ---- mechanism controls of Table 7 ----------------------------------------------------------

namespace {

struct PlanMech {
  size_t logits = 0, idx = 0, gate = 0, u = 0, u2 = 0, qkv = 0, kv = 0, o = 0, a = 0, g = 0;
  size_t topk = 0, total = 0;
};

// kind 0: routed FFN refinement (M = B*k routed rows); 1: full-sequence attention block;
// 2: Selected-Q/full-KV layer (M routed rows, keys / values of all B*T rows).
PlanMech plan_mech(const xmod_dims *dm, int64_t M, int kind) {
  PlanMech p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  const int64_t BT = (int64_t)dm->B * dm->T;
  const int64_t dq = (int64_t)dm->n_q_heads * dm->head_dim;
  const int64_t dkv = (int64_t)dm->n_kv_heads * dm->head_dim;
  if (kind != 1) {
    p.logits = take((size_t)BT * 4);
    p.idx = take((size_t)M * 4);
    p.gate = take((size_t)M * 4);
    p.topk = take(topk_scratch_bytes(dm->B, dm->T));
  }
  if (kind == 0) {
    p.u = take((size_t)M * dm->d * 2);
    p.g = take((size_t)M * dm->ffn_hidden * 2);
  } else if (kind == 1) {
    p.u = take((size_t)BT * dm->d * 2);
    p.qkv = take((size_t)BT * (dq + 2 * dkv) * 2);
    p.o = take((size_t)BT * dq * 2);
  } else {
    p.u = take((size_t)BT * dm->d * 2);       // RMSNorm of every row
    p.kv = take((size_t)BT * 2 * dkv * 2);    // keys and values of every row
    p.u2 = take((size_t)M * dm->d * 2);       // selected rows of u, later v
    p.qkv = take((size_t)M * dq * 2);         // queries of the selected rows
    p.o = take((size_t)M * dq * 2);
    p.a = take((size_t)M * dm->d * 4);
    p.g = take((size_t)M * dm->ffn_hidden * 2);
  }
  p.total = off;
  return p;
}

xmod_status route_topk_into(const void *x, const xmod_layer *L, const xmod_dims *dm, int k,
                            float *bias, float tau, float delta, float *logits, int32_t *idx,
                            float *gate, void *topk_scratch, hipStream_t s) {
  XMOD_HIP(launch_router((const uint16_t *)x, (const uint16_t *)L->w_router, L->router_bias, bias,
                         tau, logits, (int64_t)dm->B * dm->T, dm->d, s));
  phase_mark(s);
  XMOD_HIP(launch_topk(logits, dm->B, dm->T, k, idx, gate, bias, delta, s, topk_scratch));
  phase_mark(s);
  return XMOD_OK;
}

}  // namespace

namespace xmod {
// ceiling probes (probe.hip)
hipError_t launch_probe_mfma(float *out, int iters, hipStream_t s);
hipError_t launch_probe_read_chunked(const void *src, size_t bytes, uint32_t *out, hipStream_t s);
hipError_t launch_probe_read(const void *src, size_t bytes, int depth, uint32_t *out,
                             hipStream_t s);
}  // namespace xmod

extern "C" {

size_t xmod_train_workspace_bytes(const xmod_dims *dims, int32_t K, int32_t entry);

size_t xmod_workspace_bytes(const xmod_dims *dims, int32_t K, int32_t entry_point) {
  if (check_dims(dims) != XMOD_OK) return 0;
  switch (entry_point) {
    case XMOD_WS_ROUTE_TOPK: return topk_scratch_bytes(dims->B, dims->T);
    case XMOD_WS_SPARSE_LAYER:
      if (K < 1 || dims->T / K < 1) return 0;
      return plan_layer(dims, (int64_t)dims->B * (dims->T / K), true).total;
    case XMOD_WS_DENSE_LAYER: return plan_layer(dims, (int64_t)dims->B * dims->T, false).total;
    case XMOD_WS_SPARSE_THRESHOLD:
      return plan_layer(dims, (int64_t)dims->B * dims->T, true, true).total;
    case XMOD_WS_ROUTED_FFN:
      if (K < 1 || dims->T / K < 1) return 0;
      return plan_mech(dims, (int64_t)dims->B * (dims->T / K), 0).total;
    case XMOD_WS_ATTN_LAYER: return plan_mech(dims, (int64_t)dims->B * dims->T, 1).total;
    case XMOD_WS_SPARSE_FULLKV:
      if (K < 1 || dims->T / K < 1) return 0;
      return plan_mech(dims, (int64_t)dims->B * (dims->T / K), 2).total;
    case XMOD_WS_TRAIN_SAVED:
    case XMOD_WS_BACKWARD:
      return xmod_train_workspace_bytes(dims, K, entry_point);
    case XMOD_WS_BLOCK: {
      const size_t dn = plan_layer(dims, (int64_t)dims->B * dims->T, false).total;
      if (K < 1 || dims->T / K < 1) return dn;
      const size_t sp = plan_layer(dims, (int64_t)dims->B * (dims->T / K), true).total;
      return dn > sp ? dn : sp;
    }
    default: return 0;
  }
}

xmod_status xmod_route_topk(const void *x, const void *w_router, float router_bias,
                            const float *bias, float tau, int32_t K, const xmod_dims *dims,
                            float *logits, int32_t *idx, float *gate, void *ws, size_t ws_bytes,
                            void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !w_router || !logits || !idx || !gate || K < 1 || dims->T / K < 1)
    return XMOD_ERR_INVALID_ARG;
  if (!isfinite(router_bias) || !isfinite(tau)) return XMOD_ERR_INVALID_ARG;
  const size_t need = topk_scratch_bytes(dims->B, dims->T);
  if (ws && ws_bytes < need) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  XMOD_HIP(launch_router((const uint16_t *)x, (const uint16_t *)w_router, router_bias, bias, tau,
                         logits, (int64_t)dims->B * dims->T, dims->d, s));
  XMOD_HIP(launch_topk(logits, dims->B, dims->T, dims->T / K, idx, gate, nullptr, 0.f, s,
                       need ? ws : nullptr));
  return XMOD_OK;
}

size_t xmod_topk_workspace_bytes(int32_t B, int32_t T) {
  if (B < 1 || T < 1 || T > 65536) return 0;
  return topk_scratch_bytes(B, T);
}

xmod_status xmod_topk_from_logits(const float *logits, int32_t B, int32_t T, int32_t k,
                                  int32_t *idx, float *gate, float *bias, float delta, void *ws,
                                  size_t ws_bytes, void *stream) {
  if (!logits || !idx || B < 1 || T < 1 || k < 1 || k > T) return XMOD_ERR_INVALID_ARG;
  if (T > 65536) return XMOD_ERR_UNSUPPORTED;
  if (!isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  const size_t need = topk_scratch_bytes(B, T);
  if (ws && ws_bytes < need) return XMOD_ERR_WORKSPACE;
  XMOD_HIP(launch_topk(logits, B, T, k, idx, gate, bias, delta, (hipStream_t)stream,
                       need ? ws : nullptr));
  return XMOD_OK;
}

xmod_status xmod_pack(const void *x, const int32_t *idx, int32_t B, int32_t T, int32_t d,
                      int32_t k, void *x_packed, void *stream) {
  if (!x || !idx || !x_packed || B < 1 || T < 1 || d < 1 || k < 1 || k > T)
    return XMOD_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > 8192) return XMOD_ERR_UNSUPPORTED;
  RowMap map;
  map.idx = idx; map.T = T; map.k = k; map.x_rows = (int64_t)B * T;
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, map, nullptr, 0.f, false, (int64_t)B * k, d,
                              (uint16_t *)x_packed, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_scatter_gated(void *x, const int32_t *idx, const float *gate, float varsigma,
                               const void *a_packed, const void *f_packed, int32_t B, int32_t T,
                               int32_t d, int32_t k, void *stream) {
  if (!x || !idx || !gate || !a_packed || !f_packed || B < 1 || T < 1 || d < 1 || k < 1 || k > T)
    return XMOD_ERR_INVALID_ARG;
  if (!isfinite(varsigma)) return XMOD_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > 8192) return XMOD_ERR_UNSUPPORTED;
  RowMap map;
  map.idx = idx; map.T = T; map.k = k; map.x_rows = (int64_t)B * T;
  XMOD_HIP(launch_scatter((uint16_t *)x, map, gate, varsigma, (const uint16_t *)a_packed,
                          (const uint16_t *)f_packed, (int64_t)B * k, d, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_sparse_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                  int32_t K, float *bias, float tau, float delta,
                                  int32_t *idx_out, float *gate_out, void *ws, size_t ws_bytes,
                                  void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, true) || K < 1 || dims->T / K < 1) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * (dims->T / K)) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  const size_t need = xmod_workspace_bytes(dims, K, XMOD_WS_SPARSE_LAYER);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  return sparse_layer(x, layer, dims, K, bias, tau, delta, idx_out, gate_out, ws,
                      (hipStream_t)stream);
}

}  // extern "C"

// ---- the allocation-free sparse layer: its workspace is a static device array ---------------
namespace {

// One copy per GPU, zero-initialised at load; every byte the layer reads is written by an
// earlier kernel of the same call, so nothing needs clearing between calls.
__device__ __align__(256) unsigned char scratch[XMOD_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the device of stream s, looked up once per device with that
// device current (the array's host-side name is not a device address).
xmod_status scratch_for_stream(hipStream_t s, void **out) {
  int dev = -1;
  if (s) {
    XMOD_HIP(hipStreamGetDevice(s, &dev));
  } else {
    XMOD_HIP(hipGetDevice(&dev));
  }
  if (dev < 0 || dev >= kMaxDevices) return XMOD_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    XMOD_HIP(hipGetDevice(&cur));
    if (cur != dev) XMOD_HIP(hipSetDevice(dev));
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (cur != dev) XMOD_HIP(hipSetDevice(cur));
    XMOD_HIP(e);
    if (!p) return XMOD_ERR_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return XMOD_OK;
}

}  // namespace

extern "C" {

xmod_status xmod_sparse_layer_fwd_noalloc(void *x, const xmod_layer *layer,
                                          const xmod_dims *dims, int32_t K, float *bias,
                                          float tau, float delta, int32_t *idx_out,
                                          float *gate_out, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, true) || K < 1 || dims->T / K < 1) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * (dims->T / K)) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  const size_t need = xmod_workspace_bytes(dims, K, XMOD_WS_SPARSE_LAYER);
  if (need > XMOD_NOALLOC_SCRATCH_BYTES) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void *ws = nullptr;
  const xmod_status sc = scratch_for_stream(s, &ws);
  if (sc != XMOD_OK) return sc;
  return sparse_layer(x, layer, dims, K, bias, tau, delta, idx_out, gate_out, ws, s);
}

xmod_status xmod_dense_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                 void *ws, size_t ws_bytes, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, false)) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  const size_t need = xmod_workspace_bytes(dims, 1, XMOD_WS_DENSE_LAYER);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  return dense_layer(x, layer, dims, ws, (hipStream_t)stream);
}

xmod_status xmod_block_fwd(void *x, const xmod_layer *layers, int32_t n_layers,
                           const xmod_dims *dims, int32_t N0, int32_t N1, float A, int32_t K,
                           float *bias, float tau, float delta, void *ws, size_t ws_bytes,
                           void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  bool ok = false;
  const int ak = block_sparse_per_block(A, K, &ok);
  if (!x || !layers || !bias || N0 < 0 || N1 < 0 || K < 1 || dims->T / K < 1 || !ok)
    return XMOD_ERR_INVALID_ARG;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  const int64_t expect = (int64_t)N0 + (int64_t)N1 * (ak + 1);
  if (expect != n_layers) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  for (int64_t i = 0; i < n_layers; ++i) {
    const bool sparse = i >= N0 && ((i - N0) % (ak + 1)) < ak;
    if (!layer_ok(&layers[i], sparse)) return XMOD_ERR_INVALID_ARG;
  }
  const size_t need = xmod_workspace_bytes(dims, K, XMOD_WS_BLOCK);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;

  hipStream_t s = (hipStream_t)stream;
  const int64_t nb = (int64_t)dims->B * dims->T;
  const unsigned zgrid = (unsigned)((nb + 255) / 256);
  for (int64_t i = 0; i < n_layers; ++i) {
    const bool in_prefix = i < N0;
    const int64_t pos = in_prefix ? 0 : (i - N0) % (ak + 1);
    if (!in_prefix && pos == 0) {  // start of a block: the carried bias restarts from zero
      hipLaunchKernelGGL(zero_f32_kernel, dim3(zgrid), dim3(256), 0, s, bias, nb);
      XMOD_HIP(hipGetLastError());
    }
    xmod_status r;
    if (!in_prefix && pos < ak)
      r = sparse_layer(x, &layers[i], dims, K, bias, tau, delta, nullptr, nullptr, ws, s);
    else
      r = dense_layer(x, &layers[i], dims, ws, s);
    if (r != XMOD_OK) return r;
  }
  return XMOD_OK;
}

xmod_status xmod_rmsnorm_rows(const void *x, const int32_t *idx, const void *gain, float eps,
                              int32_t B, int32_t T, int32_t d, int32_t k, void *out,
                              void *stream) {
  if (!x || !gain || !out || B < 1 || T < 1 || d < 1 || k < 1 || k > T)
    return XMOD_ERR_INVALID_ARG;
  if (!(eps >= 0.f) || !isfinite(eps)) return XMOD_ERR_INVALID_ARG;
  if (d % 64 != 0 || d > 8192) return XMOD_ERR_UNSUPPORTED;
  RowMap map;
  map.idx = idx; map.T = T; map.k = k; map.x_rows = (int64_t)B * T;
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, map, (const uint16_t *)gain, eps, true,
                              (int64_t)B * k, d, (uint16_t *)out, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_gemm_bf16_nt(const void *A, int32_t lda, const void *Bm, int32_t ldb, void *Cm,
                              int32_t ldc, int32_t M, int32_t N, int32_t K, void *stream) {
  if (!A || !Bm || !Cm || M < 1 || N < 1 || K < 1 || lda < K || ldb < K || ldc < N)
    return XMOD_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || ldc % 8 != 0)
    return XMOD_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;  // operands addressed by 32-bit byte offsets
  if ((int64_t)M * lda >= lim || (int64_t)N * ldb >= lim || (int64_t)M * ldc >= lim)
    return XMOD_ERR_UNSUPPORTED;
  GemmArgs g{};
  g.A = (const uint16_t *)A; g.lda = lda; g.B = (const uint16_t *)Bm; g.ldb = ldb;
  g.C = (uint16_t *)Cm; g.ldc = ldc; g.M = M; g.N = N; g.K = K;
  XMOD_HIP(launch_gemm(g, EPI_STORE, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_gemm_bf16(int32_t layout, const void *A, int32_t lda, const void *Bm, int32_t ldb,
                           void *Cm, int32_t ldc, int32_t out_f32, int32_t M, int32_t N,
                           int32_t K, void *stream) {
  if (layout < XMOD_GEMM_NT || layout > XMOD_GEMM_TN || !A || !Bm || !Cm || M < 1 || N < 1 ||
      K < 1 || ldc < N)
    return XMOD_ERR_INVALID_ARG;
  const bool a_km = layout == XMOD_GEMM_TN, b_km = layout != XMOD_GEMM_NT;
  if (lda < (a_km ? M : K) || ldb < (b_km ? N : K)) return XMOD_ERR_INVALID_ARG;
  if (K % 64 != 0 || N % 8 != 0 || lda % 8 != 0 || ldb % 8 != 0 || ldc % 8 != 0 ||
      (a_km && M % 8 != 0) || (layout == XMOD_GEMM_TN && !out_f32))
    return XMOD_ERR_UNSUPPORTED;
  const int64_t lim = (int64_t)1 << 31;
  if ((int64_t)(a_km ? K : M) * lda >= lim || (int64_t)(b_km ? K : N) * ldb >= lim ||
      (int64_t)M * ldc >= lim)
    return XMOD_ERR_UNSUPPORTED;
  GemmArgs g{};
  g.A = (const uint16_t *)A; g.lda = lda; g.B = (const uint16_t *)Bm; g.ldb = ldb;
  g.ldc = ldc; g.M = M; g.N = N; g.K = K;
  if (out_f32) g.Cf = (float *)Cm;
  else g.C = (uint16_t *)Cm;
  const GemmLayout lay = layout == XMOD_GEMM_NT ? LAY_NT : layout == XMOD_GEMM_NN ? LAY_NN : LAY_TN;
  XMOD_HIP(launch_gemm(g, out_f32 ? EPI_STORE_F32 : EPI_STORE, lay, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_attention_fwd(const void *qkv, int32_t ld_qkv, void *o, int32_t ld_o, int32_t B,
                               int32_t k, int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               void *stream) {
  if (!qkv || !o || B < 1 || k < 1 || n_q_heads < 1 || n_kv_heads < 1 ||
      n_q_heads % n_kv_heads != 0)
    return XMOD_ERR_INVALID_ARG;
  if (head_dim != 64 && head_dim != 128) return XMOD_ERR_UNSUPPORTED;
  const int32_t nqkv = (n_q_heads + 2 * n_kv_heads) * head_dim;
  if (ld_qkv < nqkv || ld_o < n_q_heads * head_dim || ld_qkv % 8 != 0 || ld_o % 8 != 0)
    return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_attention((const uint16_t *)qkv, ld_qkv, (uint16_t *)o, ld_o, B, k, n_q_heads,
                            n_kv_heads, head_dim, nullptr, nullptr, (hipStream_t)stream));
  return XMOD_OK;
}

static xmod_status attn_shape_ok(int32_t B, int32_t k, int32_t Hq, int32_t Hkv, int32_t hd) {
  if (B < 1 || k < 1 || Hq < 1 || Hkv < 1 || Hq % Hkv != 0) return XMOD_ERR_INVALID_ARG;
  if (hd != 64 && hd != 128) return XMOD_ERR_UNSUPPORTED;
  return XMOD_OK;
}

xmod_status xmod_attention_fwd_lse(const void *qkv, int32_t ld_qkv, void *o, int32_t ld_o,
                                   float *lse, int32_t B, int32_t k, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, void *stream) {
  if (!qkv || !o || !lse) return XMOD_ERR_INVALID_ARG;
  const xmod_status st = attn_shape_ok(B, k, n_q_heads, n_kv_heads, head_dim);
  if (st != XMOD_OK) return st;
  const int32_t nqkv = (n_q_heads + 2 * n_kv_heads) * head_dim;
  if (ld_qkv < nqkv || ld_o < n_q_heads * head_dim || ld_qkv % 8 != 0 || ld_o % 8 != 0)
    return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_attention_lse((const uint16_t *)qkv, ld_qkv, (uint16_t *)o, ld_o, lse, B, k,
                                n_q_heads, n_kv_heads, head_dim, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_attention_bwd(const void *qkv, int32_t ld_qkv, const void *o, int32_t ld_o,
                               const float *lse, const void *dO, int32_t ld_do, float *D,
                               void *dqkv, int32_t ld_dqkv, int32_t B, int32_t k,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               void *stream) {
  if (!qkv || !o || !lse || !dO || !D || !dqkv) return XMOD_ERR_INVALID_ARG;
  const xmod_status st = attn_shape_ok(B, k, n_q_heads, n_kv_heads, head_dim);
  if (st != XMOD_OK) return st;
  const int32_t dq = n_q_heads * head_dim, nqkv = (n_q_heads + 2 * n_kv_heads) * head_dim;
  if (ld_qkv < nqkv || ld_dqkv < nqkv || ld_o < dq || ld_do < dq || ld_qkv % 8 != 0 ||
      ld_dqkv % 8 != 0 || ld_o % 8 != 0 || ld_do % 8 != 0)
    return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_attention_bwd((const uint16_t *)qkv, ld_qkv, (const uint16_t *)o, ld_o, lse,
                                (const uint16_t *)dO, ld_do, D, (uint16_t *)dqkv, ld_dqkv, B, k,
                                n_q_heads, n_kv_heads, head_dim, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_probe_mfma(float *out, int32_t iters, void *stream) {
  if (!out || iters < 1 || iters > (1 << 18)) return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_probe_mfma(out, iters, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_probe_read(const void *src, size_t bytes, int32_t loads_in_flight,
                            uint32_t *out, void *stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return XMOD_ERR_INVALID_ARG;
  if (loads_in_flight != 4 && loads_in_flight != 8 && loads_in_flight != 16)
    return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_probe_read(src, bytes, loads_in_flight, out, (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_probe_read_chunked(const void *src, size_t bytes, uint32_t *out, void *stream) {
  if (!src || !out || bytes == 0 || bytes % 16 != 0 || (uintptr_t)src % 16 != 0)
    return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_probe_read_chunked(src, bytes, out, (hipStream_t)stream));
  return XMOD_OK;
}

void xmod_phase_timing_enable(int32_t on) {
  g_phase.on = on != 0;
  g_phase.used = 0;
  g_phase.calls.clear();
}

void xmod_phase_timing_slots(uint32_t mask) { g_phase.mask = mask; }

xmod_status xmod_phase_times(float *ms, int32_t n_slots, int32_t *n_calls) {
  if (!ms || n_slots < 1) return XMOD_ERR_INVALID_ARG;
  for (int i = 0; i < n_slots; ++i) ms[i] = 0.f;
  if (n_calls) *n_calls = (int32_t)g_phase.calls.size();
  if (g_phase.used > 0) XMOD_HIP(hipEventSynchronize(g_phase.pool[g_phase.used - 1]));
  for (const PhaseCall &c : g_phase.calls) {
    for (size_t i = 1; i < c.ev.size(); ++i) {
      if (c.ev[i].first != c.ev[i - 1].first + 1) continue;  // not the two ends of one slot
      const int slot = c.first_slot + c.ev[i - 1].first;
      float t = 0.f;
      XMOD_HIP(hipEventElapsedTime(&t, g_phase.pool[c.ev[i - 1].second],
                                   g_phase.pool[c.ev[i].second]));
      if (slot < n_slots) ms[slot] += t;
    }
  }
  g_phase.used = 0;
  g_phase.calls.clear();
  return XMOD_OK;
}

const char *xmod_status_string(xmod_status st) {
  switch (st) {
    case XMOD_OK: return "ok";
    case XMOD_ERR_INVALID_ARG: return "invalid argument";
    case XMOD_ERR_UNSUPPORTED: return "unsupported shape";
    case XMOD_ERR_WORKSPACE: return "workspace missing or too small";
    case XMOD_ERR_HIP: return "HIP launch error";
    default: return "unknown status";
  }
}

int32_t xmod_last_hip_error(void) { return g_last_hip; }

}  // extern "C"

xmod_status xmod_threshold_select(const float *logits, int32_t B, int32_t T, int32_t *counts,
                                  int32_t *offsets, int32_t *src, float *gate, int32_t *n_total,
                                  float *bias, float delta, void *stream) {
  if (!logits || !counts || !offsets || !src || !n_total || B < 1 || T < 1)
    return XMOD_ERR_INVALID_ARG;
  if ((int64_t)B * T > INT32_MAX) return XMOD_ERR_UNSUPPORTED;
  if (T > 65536) return XMOD_ERR_UNSUPPORTED;
  if (!isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  XMOD_HIP(launch_threshold_select(logits, B, T, counts, offsets, src, gate, n_total, bias, delta,
                                   (hipStream_t)stream));
  return XMOD_OK;
}

xmod_status xmod_sparse_layer_fwd_threshold(void *x, const xmod_layer *layer,
                                            const xmod_dims *dims, float *bias, float tau,
                                            float delta, int32_t *src_out, int32_t *counts_out,
                                            int32_t *n_total_out, void *ws, size_t ws_bytes,
                                            void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, true)) return XMOD_ERR_INVALID_ARG;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if ((int64_t)dims->B * dims->T > INT32_MAX) return XMOD_ERR_UNSUPPORTED;
  const size_t need = xmod_workspace_bytes(dims, 1, XMOD_WS_SPARSE_THRESHOLD);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  return sparse_layer_threshold(x, layer, dims, bias, tau, delta, src_out, counts_out,
                                n_total_out, ws, (hipStream_t)stream);
}

xmod_status xmod_mask_agreement(const float *logits, const int32_t *idx, int32_t B, int32_t T,
                                int32_t k, uint32_t *agree, void *stream) {
  if (!logits || !idx || !agree || B < 1 || T < 1 || k < 1 || k > T) return XMOD_ERR_INVALID_ARG;
  if (T > 65536) return XMOD_ERR_UNSUPPORTED;
  XMOD_HIP(launch_mask_agreement(logits, idx, B, T, k, agree, (hipStream_t)stream));
  return XMOD_OK;
}


xmod_status xmod_routed_ffn_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                int32_t K, float *bias, float tau, float delta,
                                int32_t *idx_out, float *gate_out, void *ws, size_t ws_bytes,
                                void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!x || !layer || !layer->w_router || !layer->g_ffn || !layer->w_gate || !layer->w_up ||
      !layer->w_down || K < 1 || dims->T / K < 1)
    return XMOD_ERR_INVALID_ARG;
  if (!isfinite(tau) || !isfinite(delta) || !isfinite(layer->router_bias) ||
      !isfinite(layer->varsigma))
    return XMOD_ERR_INVALID_ARG;
  const size_t need = xmod_workspace_bytes(dims, K, XMOD_WS_ROUTED_FFN);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int k = dims->T / K;
  const int64_t M = (int64_t)dims->B * k;
  const PlanMech p = plan_mech(dims, M, 0);
  int32_t *idx = idx_out ? idx_out : at<int32_t>(ws, p.idx);
  float *gate = gate_out ? gate_out : at<float>(ws, p.gate);
  uint16_t *u = at<uint16_t>(ws, p.u), *gbuf = at<uint16_t>(ws, p.g);
  phase_begin(s, 0);
  const xmod_status r = route_topk_into(x, layer, dims, k, bias, tau, delta, at<float>(ws, p.logits),
                                        idx, gate, at<void>(ws, p.topk), s);
  if (r != XMOD_OK) return r;
  const RowMap map = topk_map(idx, dims, k);
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, map, (const uint16_t *)layer->g_ffn,
                              dims->rms_eps, true, M, dims->d, u, s));
  phase_mark(s);
  GemmArgs g{};
  g.map = map;
  g.A = u; g.lda = dims->d; g.B = (const uint16_t *)layer->w_gate;
  g.B2 = (const uint16_t *)layer->w_up; g.ldb = dims->d; g.C = gbuf; g.ldc = dims->ffn_hidden;
  g.M = (int)M; g.N = dims->ffn_hidden; g.K = dims->d;
  XMOD_HIP(launch_gemm(g, EPI_SWIGLU, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = gbuf; g.lda = dims->ffn_hidden; g.B = (const uint16_t *)layer->w_down;
  g.ldb = dims->ffn_hidden; g.ldc = dims->d; g.M = (int)M; g.N = dims->d; g.K = dims->ffn_hidden;
  g.x = (uint16_t *)x; g.gate = gate; g.varsigma = layer->varsigma; g.a = nullptr;
  XMOD_HIP(launch_gemm(g, EPI_RESIDUAL, s));
  phase_mark(s);
  return XMOD_OK;
}

xmod_status xmod_attention_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                     void *ws, size_t ws_bytes, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!x || !layer || !layer->g_attn || !layer->w_qkv || !layer->w_o) return XMOD_ERR_INVALID_ARG;
  if (!(layer->rope_theta >= 0.f) || !isfinite(layer->rope_theta)) return XMOD_ERR_INVALID_ARG;
  const size_t need = xmod_workspace_bytes(dims, 1, XMOD_WS_ATTN_LAYER);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int64_t M = (int64_t)dims->B * dims->T;
  const PlanMech p = plan_mech(dims, M, 1);
  const int d = dims->d, dq = dims->n_q_heads * dims->head_dim;
  const int nqkv = dq + 2 * dims->n_kv_heads * dims->head_dim;
  uint16_t *u = at<uint16_t>(ws, p.u), *qkv = at<uint16_t>(ws, p.qkv), *o = at<uint16_t>(ws, p.o);
  RowMap map;
  map.T = dims->T; map.x_rows = M;
  phase_begin(s, 2);
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, map, (const uint16_t *)layer->g_attn,
                              dims->rms_eps, true, M, d, u, s));
  phase_mark(s);
  GemmArgs g{};
  g.map = map;
  g.A = u; g.lda = d; g.B = (const uint16_t *)layer->w_qkv; g.ldb = d; g.C = qkv; g.ldc = nqkv;
  g.M = (int)M; g.N = nqkv; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, s));
  phase_mark(s);
  XMOD_HIP(launch_qk_form(qkv, nqkv, map, M, dims->n_q_heads, dims->n_kv_heads, dims->head_dim,
                          (const uint16_t *)layer->q_norm, (const uint16_t *)layer->k_norm,
                          dims->rms_eps, layer->rope_theta, s));
  XMOD_HIP(launch_attention(qkv, nqkv, o, dq, dims->B, dims->T, dims->n_q_heads,
                            dims->n_kv_heads, dims->head_dim, nullptr, nullptr, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = o; g.lda = dq; g.B = (const uint16_t *)layer->w_o; g.ldb = dq; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = dq;
  g.x = (uint16_t *)x; g.gate = nullptr; g.a = nullptr;  // y = x + O W_o^T
  XMOD_HIP(launch_gemm(g, EPI_RESIDUAL, s));
  phase_mark(s);
  return XMOD_OK;
}

xmod_status xmod_sparse_layer_fwd_fullkv(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                         int32_t K, float *bias, float tau, float delta,
                                         int32_t *idx_out, float *gate_out, void *ws,
                                         size_t ws_bytes, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, true) || K < 1 || dims->T / K < 1) return XMOD_ERR_INVALID_ARG;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * dims->T) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  const size_t need = xmod_workspace_bytes(dims, K, XMOD_WS_SPARSE_FULLKV);
  if (!ws || ws_bytes < need) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int B = dims->B, T = dims->T, d = dims->d, k = T / K;
  const int64_t M = (int64_t)B * k, BT = (int64_t)B * T;
  const int Hq = dims->n_q_heads, Hkv = dims->n_kv_heads, hd = dims->head_dim;
  const int dq = Hq * hd, dkv = Hkv * hd;
  const PlanMech p = plan_mech(dims, M, 2);
  int32_t *idx = idx_out ? idx_out : at<int32_t>(ws, p.idx);
  float *gate = gate_out ? gate_out : at<float>(ws, p.gate);
  uint16_t *u = at<uint16_t>(ws, p.u), *kv = at<uint16_t>(ws, p.kv), *u2 = at<uint16_t>(ws, p.u2);
  uint16_t *q = at<uint16_t>(ws, p.qkv), *o = at<uint16_t>(ws, p.o), *gbuf = at<uint16_t>(ws, p.g);
  float *a = at<float>(ws, p.a);
  phase_begin(s, 0);
  const xmod_status r = route_topk_into(x, layer, dims, k, bias, tau, delta,
                                        at<float>(ws, p.logits), idx, gate, at<void>(ws, p.topk), s);
  if (r != XMOD_OK) return r;
  RowMap all;
  all.T = T; all.x_rows = BT;
  const RowMap map = topk_map(idx, dims, k);
  // RMSNorm of every row; keys and values of every row; queries of the selected rows
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, all, (const uint16_t *)layer->g_attn,
                              dims->rms_eps, true, BT, d, u, s));
  XMOD_HIP(launch_gather_rows(u, map, nullptr, 0.f, false, M, d, u2, s));
  phase_mark(s);
  GemmArgs g{};
  g.map = all;
  g.A = u; g.lda = d; g.B = (const uint16_t *)layer->w_qkv + (size_t)dq * d; g.ldb = d;
  g.C = kv; g.ldc = 2 * dkv; g.M = (int)BT; g.N = 2 * dkv; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, s));
  g = GemmArgs{};
  g.map = map;
  g.A = u2; g.lda = d; g.B = (const uint16_t *)layer->w_qkv; g.ldb = d; g.C = q; g.ldc = dq;
  g.M = (int)M; g.N = dq; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, s));
  phase_mark(s);
  // optional QK-norm / rotary embedding: queries at their original positions, keys at theirs
  XMOD_HIP(launch_qk_form(q, dq, map, M, Hq, 0, hd, (const uint16_t *)layer->q_norm, nullptr,
                          dims->rms_eps, layer->rope_theta, s));
  XMOD_HIP(launch_qk_form(kv, 2 * dkv, all, BT, 0, Hkv, hd, nullptr,
                          (const uint16_t *)layer->k_norm, dims->rms_eps, layer->rope_theta, s));
  XMOD_HIP(launch_attention_fullkv(q, dq, kv, 2 * dkv, idx, o, dq, B, k, T, Hq, Hkv, hd, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = o; g.lda = dq; g.B = (const uint16_t *)layer->w_o; g.ldb = dq; g.Cf = a; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = dq;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, s));
  phase_mark(s);
  XMOD_HIP(launch_residual_rmsnorm((const uint16_t *)x, map, a, (const uint16_t *)layer->g_ffn,
                                   dims->rms_eps, M, d, u2, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = u2; g.lda = d; g.B = (const uint16_t *)layer->w_gate; g.B2 = (const uint16_t *)layer->w_up;
  g.ldb = d; g.C = gbuf; g.ldc = dims->ffn_hidden; g.M = (int)M; g.N = dims->ffn_hidden; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_SWIGLU, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = gbuf; g.lda = dims->ffn_hidden; g.B = (const uint16_t *)layer->w_down;
  g.ldb = dims->ffn_hidden; g.ldc = d; g.M = (int)M; g.N = d; g.K = dims->ffn_hidden;
  g.x = (uint16_t *)x; g.gate = gate; g.varsigma = layer->varsigma; g.a = a;
  g.residual_form = layer->residual;
  XMOD_HIP(launch_gemm(g, EPI_RESIDUAL, s));
  phase_mark(s);
  return XMOD_OK;
}

// ---- training: forward that keeps what the backward reads, and the backward -------------------

namespace {

// Packed rows are padded to a multiple of 64 for the weight-gradient products (sums over the
// rows); padding rows of their operands are zero.
int64_t pad_rows(int64_t M) { return (M + 63) / 64 * 64; }

struct PlanTrain {
  size_t s = 0, logits = 0, idx = 0, gate = 0, topk = 0, X = 0, u = 0, qkv = 0, o = 0, lse = 0;
  size_t a = 0;
  size_t v = 0, g = 0, z = 0, f = 0, total = 0;
};

PlanTrain plan_train(const xmod_dims *dm, int64_t M) {
  PlanTrain p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  const int64_t BT = (int64_t)dm->B * dm->T, Mp = pad_rows(M), d = dm->d, F = dm->ffn_hidden;
  const int64_t dq = (int64_t)dm->n_q_heads * dm->head_dim;
  const int64_t nqkv = dq + 2LL * dm->n_kv_heads * dm->head_dim;
  p.s = take(BT * 4);
  p.logits = take(BT * 4);
  p.idx = take(M * 4);
  p.gate = take(M * 4);
  p.topk = take(topk_scratch_bytes(dm->B, dm->T));
  p.X = take(Mp * d * 2);
  p.u = take(Mp * d * 2);
  p.qkv = take(Mp * nqkv * 2);
  p.o = take(Mp * dq * 2);
  p.lse = take(M * dm->n_q_heads * 4);
  p.a = take(M * d * 4);
  p.v = take(Mp * d * 2);
  p.g = take(Mp * F * 2);
  p.z = take(Mp * 2 * F * 2);
  p.f = take(M * d * 4);
  p.total = off;
  return p;
}

struct PlanBwd {
  size_t dt = 0, dz = 0, dv = 0, da = 0, dxacc = 0, dO = 0, D = 0, dqkv = 0, dell = 0;
  size_t dell_tok = 0, q_tok = 0, part_g2 = 0, part_g1 = 0, part_wr = 0, spart = 0, tmp = 0;
  size_t total = 0;
};

PlanBwd plan_bwd(const xmod_dims *dm, int64_t M) {
  PlanBwd p;
  size_t off = 0;
  auto take = [&](size_t bytes) { size_t at = off; off += align_up(bytes); return at; };
  const int64_t BT = (int64_t)dm->B * dm->T, Mp = pad_rows(M), d = dm->d, F = dm->ffn_hidden;
  const int64_t dq = (int64_t)dm->n_q_heads * dm->head_dim;
  const int64_t nqkv = dq + 2LL * dm->n_kv_heads * dm->head_dim;
  const int64_t R = bwd_row_wgs(), RT = bwd_route_wgs();
  p.dt = take(Mp * d * 2);
  p.dz = take(Mp * 2 * F * 2);
  p.dv = take(M * d * 4);       // dv, later du
  p.da = take(Mp * d * 2);
  p.dxacc = take(M * d * 4);
  p.dO = take(M * dq * 2);
  p.D = take(M * dm->n_q_heads * 4);
  p.dqkv = take(Mp * nqkv * 2);
  p.dell = take(M * 4);
  p.dell_tok = take(BT * 4);   // dell_tok and q_tok are adjacent: one zero fill
  p.q_tok = take(BT);
  p.part_g2 = take(R * d * 4);
  p.part_g1 = take(R * d * 4);
  p.part_wr = take((R + RT) * d * 4);
  p.spart = take((R + 2 * RT) * 4);
  p.tmp = take(16 * (3 * d + 3) * 4);
  p.total = off;
  return p;
}

bool core_form(const xmod_layer *L) {
  return L->residual == 0 && !L->q_norm && !L->k_norm && L->rope_theta == 0.f;
}

// zero rows [M, Mp) of a row-major bf16 buffer with `width` columns
xmod_status zero_pad_rows(uint16_t *buf, int64_t M, int64_t Mp, int64_t width, hipStream_t s) {
  if (Mp > M) XMOD_HIP(launch_zero(buf + M * width, (size_t)((Mp - M) * width * 2), s));
  return XMOD_OK;
}

}  // namespace

size_t xmod_train_workspace_bytes(const xmod_dims *dims, int32_t K, int32_t entry) {
  if (check_dims(dims) != XMOD_OK || K < 1 || dims->T / K < 1) return 0;
  const int64_t M = (int64_t)dims->B * (dims->T / K);
  return entry == XMOD_WS_TRAIN_SAVED ? plan_train(dims, M).total : plan_bwd(dims, M).total;
}

xmod_status xmod_sparse_layer_fwd_train(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                        int32_t K, float *bias, float tau, float delta,
                                        int32_t *idx_out, float *gate_out, void *saved,
                                        size_t saved_bytes, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !layer_ok(layer, true) || K < 1 || dims->T / K < 1) return XMOD_ERR_INVALID_ARG;
  if (!isfinite(tau) || !isfinite(delta)) return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * (dims->T / K)) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!core_form(layer)) return XMOD_ERR_UNSUPPORTED;
  const int k = dims->T / K;
  const int64_t M = (int64_t)dims->B * k, Mp = pad_rows(M), BT = (int64_t)dims->B * dims->T;
  const PlanTrain p = plan_train(dims, M);
  if (!saved || saved_bytes < p.total) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  const int d = dims->d, F = dims->ffn_hidden, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads;
  const int hd = dims->head_dim, dq = Hq * hd, nqkv = dq + 2 * Hkv * hd;
  float *sv = at<float>(saved, p.s), *logits = at<float>(saved, p.logits);
  int32_t *idx = at<int32_t>(saved, p.idx);
  float *gate = at<float>(saved, p.gate), *lse = at<float>(saved, p.lse);
  uint16_t *Xs = at<uint16_t>(saved, p.X), *u = at<uint16_t>(saved, p.u);
  uint16_t *qkv = at<uint16_t>(saved, p.qkv), *o = at<uint16_t>(saved, p.o);
  uint16_t *v = at<uint16_t>(saved, p.v), *gb = at<uint16_t>(saved, p.g);
  uint16_t *z = at<uint16_t>(saved, p.z);
  float *a = at<float>(saved, p.a), *f = at<float>(saved, p.f);

  phase_begin(s, 0);
  XMOD_HIP(launch_router((const uint16_t *)x, (const uint16_t *)layer->w_router,
                         layer->router_bias, bias, tau, logits, BT, d, s, sv));
  phase_mark(s);
  XMOD_HIP(launch_topk(logits, dims->B, dims->T, k, idx, gate, bias, delta, s,
                       at<void>(saved, p.topk)));
  if (idx_out) XMOD_HIP(launch_copy32(idx_out, idx, M, s));
  if (gate_out) XMOD_HIP(launch_copy32(gate_out, gate, M, s));
  phase_mark(s);
  const RowMap map = topk_map(idx, dims, k);
  XMOD_HIP(launch_gather_rows((const uint16_t *)x, map, (const uint16_t *)layer->g_attn,
                              dims->rms_eps, true, M, d, u, s, Xs));
  phase_mark(s);
  GemmArgs g{};
  g.A = u; g.lda = d; g.B = (const uint16_t *)layer->w_qkv; g.ldb = d; g.C = qkv; g.ldc = nqkv;
  g.M = (int)M; g.N = nqkv; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, s));
  phase_mark(s);
  XMOD_HIP(launch_attention_lse(qkv, nqkv, o, dq, lse, dims->B, k, Hq, Hkv, hd, s));
  phase_mark(s);
  g = GemmArgs{};
  g.A = o; g.lda = dq; g.B = (const uint16_t *)layer->w_o; g.ldb = dq; g.Cf = a; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = dq;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, s));
  phase_mark(s);
  XMOD_HIP(launch_residual_rmsnorm((const uint16_t *)x, map, a, (const uint16_t *)layer->g_ffn,
                                   dims->rms_eps, M, d, v, s));
  phase_mark(s);
  g = GemmArgs{};
  g.A = v; g.lda = d; g.B = (const uint16_t *)layer->w_gate; g.B2 = (const uint16_t *)layer->w_up;
  g.ldb = d; g.C = gb; g.ldc = F; g.Z = z; g.ldz = 2 * F; g.M = (int)M; g.N = F; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_SWIGLU_SAVE, s));
  phase_mark(s);
  g = GemmArgs{};
  g.map = map;
  g.A = gb; g.lda = F; g.B = (const uint16_t *)layer->w_down; g.ldb = F; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = F;
  g.x = (uint16_t *)x; g.gate = gate; g.varsigma = layer->varsigma; g.a = a; g.fsave = f;
  XMOD_HIP(launch_gemm(g, EPI_RESIDUAL, s));
  // padding rows of the operands the weight-gradient products read
  if (zero_pad_rows(u, M, Mp, d, s) != XMOD_OK || zero_pad_rows(o, M, Mp, dq, s) != XMOD_OK ||
      zero_pad_rows(v, M, Mp, d, s) != XMOD_OK || zero_pad_rows(gb, M, Mp, F, s) != XMOD_OK)
    return XMOD_ERR_HIP;
  phase_mark(s);
  return XMOD_OK;
}

xmod_status xmod_sparse_layer_bwd(const void *x, const void *dy, void *dx,
                                  const xmod_layer *layer, const xmod_dims *dims, int32_t K,
                                  float route_coef, const void *saved, size_t saved_bytes,
                                  const xmod_layer_grads *gr, float *loss_route, void *ws,
                                  size_t ws_bytes, void *stream) {
  const xmod_status st = check_dims(dims);
  if (st != XMOD_OK) return st;
  if (!x || !dy || !dx || !saved || !gr || !layer_ok(layer, true) || K < 1 || dims->T / K < 1)
    return XMOD_ERR_INVALID_ARG;
  if (check_rows(dims, (int64_t)dims->B * (dims->T / K)) != XMOD_OK) return XMOD_ERR_UNSUPPORTED;
  if (!gr->w_router || !gr->router_bias || !gr->varsigma || !gr->g_attn || !gr->w_qkv ||
      !gr->w_o || !gr->g_ffn || !gr->w_gate || !gr->w_up || !gr->w_down)
    return XMOD_ERR_INVALID_ARG;
  if (!isfinite(route_coef)) return XMOD_ERR_INVALID_ARG;
  if (!core_form(layer)) return XMOD_ERR_UNSUPPORTED;
  const int k = dims->T / K;
  const int64_t M = (int64_t)dims->B * k, Mp = pad_rows(M), BT = (int64_t)dims->B * dims->T;
  const PlanTrain p = plan_train(dims, M);
  const PlanBwd q = plan_bwd(dims, M);
  if (saved_bytes < p.total || !ws || ws_bytes < q.total) return XMOD_ERR_WORKSPACE;
  hipStream_t s = (hipStream_t)stream;
  void *sv_ = const_cast<void *>(saved);
  const int d = dims->d, F = dims->ffn_hidden, Hq = dims->n_q_heads, Hkv = dims->n_kv_heads;
  const int hd = dims->head_dim, dq = Hq * hd, nqkv = dq + 2 * Hkv * hd;
  const float eps = dims->rms_eps;
  const float coef_n = (float)((double)route_coef / (double)BT);
  const int R = bwd_row_wgs(), RT = bwd_route_wgs();
  // saved by the forward
  const float *s_tok = at<float>(sv_, p.s), *gate = at<float>(sv_, p.gate);
  const int32_t *idx = at<int32_t>(sv_, p.idx);
  const uint16_t *Xs = at<uint16_t>(sv_, p.X), *u = at<uint16_t>(sv_, p.u);
  const uint16_t *qkv = at<uint16_t>(sv_, p.qkv), *o = at<uint16_t>(sv_, p.o);
  const uint16_t *v = at<uint16_t>(sv_, p.v), *gb = at<uint16_t>(sv_, p.g);
  uint16_t *z = at<uint16_t>(sv_, p.z);
  const float *lse = at<float>(sv_, p.lse), *a = at<float>(sv_, p.a), *f = at<float>(sv_, p.f);
  // workspace
  uint16_t *dt = at<uint16_t>(ws, q.dt), *dz = at<uint16_t>(ws, q.dz), *da = at<uint16_t>(ws, q.da);
  uint16_t *dO = at<uint16_t>(ws, q.dO), *dqkv = at<uint16_t>(ws, q.dqkv);
  float *dv = at<float>(ws, q.dv), *dxacc = at<float>(ws, q.dxacc), *D = at<float>(ws, q.D);
  float *dell = at<float>(ws, q.dell), *dell_tok = at<float>(ws, q.dell_tok);
  uint8_t *q_tok = at<uint8_t>(ws, q.q_tok);
  float *part_g2 = at<float>(ws, q.part_g2), *part_g1 = at<float>(ws, q.part_g1);
  float *part_wr = at<float>(ws, q.part_wr), *spart = at<float>(ws, q.spart);
  float *tmp = at<float>(ws, q.tmp);
  float *vs_part = spart, *beta_part = spart + R, *loss_part = spart + R + RT;
  const RowMap map = topk_map(idx, dims, k);

  // gated residual: dt, the gate's gradient, d varsigma partials; selection marks per token
  phase_begin(s, 9);
  XMOD_HIP(launch_zero(dell_tok, align_up((size_t)BT * 4) + align_up((size_t)BT), s));
  XMOD_HIP(launch_resid_bwd((const uint16_t *)dy, map, a, f, gate, layer->varsigma, d, M, Mp, dt,
                            dell, dell_tok, q_tok, vs_part, s));
  phase_mark(s);
  // FFN: dg = dt W_down (SwiGLU backward in the epilogue), dW_down = dt^T g
  GemmArgs g{};
  g.A = dt; g.lda = d; g.B = (const uint16_t *)layer->w_down; g.ldb = F; g.C = dz; g.ldc = 2 * F;
  g.Z = z; g.ldz = 2 * F; g.M = (int)M; g.N = F; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_SWIGLU_BWD, LAY_NN, s));
  if (zero_pad_rows(dz, M, Mp, 2 * F, s) != XMOD_OK) return XMOD_ERR_HIP;
  phase_mark(s);
  g = GemmArgs{};
  g.A = dt; g.lda = d; g.B = gb; g.ldb = F; g.Cf = gr->w_down; g.ldc = F;
  g.M = d; g.N = F; g.K = (int)Mp;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_TN, s));
  phase_mark(s);
  // dv = dzg W_gate + dzu W_up; [dW_gate; dW_up] = [dzg | dzu]^T v
  g = GemmArgs{};
  g.A = dz; g.lda = 2 * F; g.B = (const uint16_t *)layer->w_gate; g.B2 = (const uint16_t *)layer->w_up;
  g.K1 = F; g.ldb = d; g.Cf = dv; g.ldc = d; g.M = (int)M; g.N = d; g.K = 2 * F;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_NN, s));
  phase_mark(s);
  g = GemmArgs{};
  g.A = dz; g.lda = 2 * F; g.B = v; g.ldb = d; g.Cf = gr->w_gate; g.Cf2 = gr->w_up; g.M1 = F;
  g.ldc = d; g.M = 2 * F; g.N = d; g.K = (int)Mp;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_TN, s));
  phase_mark(s);
  // RMSNorm before the FFN: da = dt + dh, dX so far = dy + dh, d g_ffn
  XMOD_HIP(launch_rms2_bwd((const uint16_t *)dy, map, Xs, a, dv, (const uint16_t *)layer->g_ffn,
                           eps, dt, d, M, Mp, da, dxacc, part_g2, s));
  phase_mark(s);
  // O projection: dO = da W_o, dW_o = da^T O
  g = GemmArgs{};
  g.A = da; g.lda = d; g.B = (const uint16_t *)layer->w_o; g.ldb = dq; g.C = dO; g.ldc = dq;
  g.M = (int)M; g.N = dq; g.K = d;
  XMOD_HIP(launch_gemm(g, EPI_STORE, LAY_NN, s));
  phase_mark(s);
  g = GemmArgs{};
  g.A = da; g.lda = d; g.B = o; g.ldb = dq; g.Cf = gr->w_o; g.ldc = dq;
  g.M = d; g.N = dq; g.K = (int)Mp;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_TN, s));
  phase_mark(s);
  // attention
  XMOD_HIP(launch_attention_bwd(qkv, nqkv, o, dq, lse, dO, dq, D, dqkv, nqkv, dims->B, k, Hq, Hkv,
                                hd, s));
  if (zero_pad_rows(dqkv, M, Mp, nqkv, s) != XMOD_OK) return XMOD_ERR_HIP;
  phase_mark(s);
  // QKV projection: du = dqkv W_qkv (into dv's buffer), dW_qkv = dqkv^T u
  g = GemmArgs{};
  g.A = dqkv; g.lda = nqkv; g.B = (const uint16_t *)layer->w_qkv; g.ldb = d; g.Cf = dv; g.ldc = d;
  g.M = (int)M; g.N = d; g.K = nqkv;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_NN, s));
  phase_mark(s);
  g = GemmArgs{};
  g.A = dqkv; g.lda = nqkv; g.B = u; g.ldb = d; g.Cf = gr->w_qkv; g.ldc = d;
  g.M = nqkv; g.N = d; g.K = (int)Mp;
  XMOD_HIP(launch_gemm(g, EPI_STORE_F32, LAY_TN, s));
  phase_mark(s);
  // RMSNorm before attention: dx of the selected rows, d g_attn, router terms of those rows
  XMOD_HIP(launch_rms1_bwd(Xs, map, dv, (const uint16_t *)layer->g_attn, eps, dxacc, s_tok, dell,
                           coef_n, (const uint16_t *)layer->w_router, d, M, (uint16_t *)dx,
                           part_g1, part_wr, s));
  phase_mark(s);
  // router and routing loss over every token: dx of the other rows, d w_r, d beta, L_route
  XMOD_HIP(launch_route_bwd((const uint16_t *)x, (const uint16_t *)dy, s_tok, dell_tok, q_tok,
                            coef_n, (const uint16_t *)layer->w_router, d, BT, (uint16_t *)dx,
                            part_wr + (size_t)R * d, beta_part, loss_part, s));
  phase_mark(s);
  // every column and scalar sum of partial rows, in one pair of launches
  ColsumJobs J{};
  auto job = [&](const float *part, int n_part, int n, float *out, float scale) {
    ColsumJob &j = J.job[J.n];
    j.part = part; j.n_part = n_part; j.n = n; j.out = out; j.scale = scale;
    j.tmp = tmp + (size_t)16 * (J.n < 3 ? J.n * d : 3 * d + (J.n - 3));
    ++J.n;
  };
  job(part_g2, R, d, gr->g_ffn, 1.0f);
  job(part_g1, R, d, gr->g_attn, 1.0f);
  job(part_wr, R + RT, d, gr->w_router, 1.0f);
  job(beta_part, RT, 1, gr->router_bias, 1.0f);
  job(vs_part, R, 1, gr->varsigma, 1.0f);
  if (loss_route) job(loss_part, RT, 1, loss_route, (float)(1.0 / (double)BT));
  XMOD_HIP(launch_colsum_multi(J, s));
  phase_mark(s);
  return XMOD_OK;
}
