/*
 * xmod.h - C ABI of the X-MoD sparse-depth layer forward on AMD MI355X (gfx950).
 *
 * What is computed (sources are cited by page title and section / equation):
 *   [XMOD] "X-MoD: Practical Scaling Laws for Sparse-Depth Routing Beyond Mixture-of-Depths"
 *          (close-reading page): Fig. 1(b) and Eq. (7) (gated residual of a sparse layer),
 *          Eq. (8) (router logit adjusted by a carried per-token bias), section "training-time
 *          top-k" (non-causal top-1/K selection per sequence), Eq. (3) (the stack
 *          [Dense]xN0 + ([Sparse(K)]xAK + [Dense])xN1 and the bias reset at each anchor),
 *          Table 7 (a sparse layer attends over the selected subset only).
 *   [MOD]  "Mixture-of-Depths explained" (blog page), section "basic architecture": scalar
 *          Linear(d, 1) router, top-k of floor(T * capacity) tokens, RMSNorm before attention
 *          and before the FFN, unselected rows passed through.
 *   [MOE]  "Beyond dense Transformers: MoE, SSMs and hybrids", bias-free SwiGLU FFN.
 *   [MODA] "Mixture-of-Depths Attention" reading notes, section 2.1: GQA head mapping.
 *   [XMOD] section "mechanism controls" (Table 7): the Routed-FFN and Selected-Q/full-KV
 *          counterfactuals.
 *   [XMOD] section "training-time top-k, eval-time causal threshold": at evaluation a token
 *          enters a sparse layer when its routing probability is at least 1/2; section
 *          "routing diagnostics", Table 10: agreement of the top-k and threshold masks.
 *
 * One Sparse(K) layer, per sequence b of length T:
 *   s_t   = w_r . x_t + beta_r                      (fp32 accumulate)
 *   ell_t = s_t - tau * b_t                          (fp32, product rounded then difference)
 *   S     = the k = floor(T/K) largest ell, ties to the lower position, packed ascending
 *   r     = sigmoid(ell_S)                           (uses b before this layer's update)
 *   X = x_S;  u = RMSNorm(X; g_attn);  [Q|K|V] = u W_qkv^T
 *   O     = causal softmax(Q K^T / sqrt(hd)) V over the packed rows; query head h reads
 *           KV head floor(h * Hkv / Hq)
 *   a = O W_o^T;  v = RMSNorm(X + a; g_ffn);  f = (SiLU(v W_gate^T) * (v W_up^T)) W_down^T
 *   y_S   = X + (varsigma * r) * (a + f)  written in place into x; unselected rows untouched
 *   b_S  += delta                                     (fp32, when a bias buffer is given)
 * A dense layer is the same with S = every position, no gate and no varsigma:
 *   y = x + (a + f).
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned (allocated by the caller, e.g. through PyTorch). The
 *     library never allocates or frees device memory. Scratch space comes from a caller
 *     workspace of at least xmod_workspace_bytes() bytes, 256-byte aligned.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL is the null stream) and
 *     returns without synchronising. Pointers must stay valid until that work completes.
 *     Calls are stateless; concurrent calls must not share output or workspace buffers.
 *   - bf16 tensors are raw 16-bit bfloat16 arrays; fp32 tensors are float arrays.
 *   - Activations are row-major [B, T, d]. Weights use the [out, in] layout of a Linear layer.
 *     W_qkv rows are: Hq query heads, then Hkv key heads, then Hkv value heads, each head_dim
 *     rows. idx lists positions within a sequence, ascending, [B, k]; packed row m = b*k + j.
 *   - Arguments are validated before the first launch; on an error status nothing is written.
 *     XMOD_ERR_INVALID_ARG: NULL required pointer, non-positive size, K < 1, floor(T/K) < 1,
 *       Hq % Hkv != 0, A*K not an integer, wrong number of layers.
 *     XMOD_ERR_UNSUPPORTED: head_dim not 64 or 128, d or ffn_hidden not a multiple of 64,
 *       T > 65536 (the selection kernels hold one sequence's keys or decisions in one
 *       workgroup's registers or LDS at some stage), d > 8192, or a matrix of 2^31 elements or
 *       more for the projections (they address operands by 32-bit byte offsets): with M the
 *       routed rows (B*floor(T/K) for the top-k layer entry points, B*T for the dense, block,
 *       threshold and mechanism-control entry points), (M + 64) * max(d, dq + 2 dkv,
 *       2 ffn_hidden) and each weight matrix must stay below 2^31 elements.
 *     XMOD_ERR_WORKSPACE: workspace NULL or smaller than xmod_workspace_bytes().
 *     XMOD_ERR_HIP: a kernel launch failed; xmod_last_hip_error() returns the hipError_t
 *       (kept per calling thread). Faults inside kernels surface at the caller's next sync.
 */
#ifndef XMOD_H
#define XMOD_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  XMOD_OK = 0,
  XMOD_ERR_INVALID_ARG = 1,
  XMOD_ERR_UNSUPPORTED = 2,
  XMOD_ERR_WORKSPACE = 3,
  XMOD_ERR_HIP = 4
} xmod_status;

/* Shapes shared by the layers of one model. */
typedef struct {
  int32_t B;            /* sequences */
  int32_t T;            /* tokens per sequence */
  int32_t d;            /* model width */
  int32_t n_q_heads;    /* Hq */
  int32_t n_kv_heads;   /* Hkv, divides Hq */
  int32_t head_dim;     /* 64 or 128 */
  int32_t ffn_hidden;   /* F */
  float rms_eps;        /* RMSNorm epsilon */
} xmod_dims;

/* Weights of one layer: device pointers to bf16 arrays, plus host scalars. */
typedef struct {
  const void *w_router;  /* [d]; unused by dense layers */
  float router_bias;     /* beta_r (host scalar) */
  float varsigma;        /* per-layer scale of the gated residual, Eq. (7) (host scalar) */
  const void *g_attn;    /* [d] RMSNorm gain before attention */
  const void *w_qkv;     /* [Hq*hd + 2*Hkv*hd, d] */
  const void *w_o;       /* [d, Hq*hd] */
  const void *g_ffn;     /* [d] RMSNorm gain before the FFN */
  const void *w_gate;    /* [F, d] */
  const void *w_up;      /* [F, d] */
  const void *w_down;    /* [d, F] */
  /* Layer-form options; zero / NULL gives the layer described at the top of this file. */
  int32_t residual;      /* 0: X-MoD, y = X + (varsigma*r)*(a + f), Eq. (7); 1: MoD,
                            y = (X + a) + r*f, [XMOD] Eq. (6) (varsigma unused). Sparse layers. */
  const void *q_norm;    /* [head_dim] bf16 or NULL: RMSNorm of every query head (QK-norm) */
  const void *k_norm;    /* [head_dim] bf16 or NULL: RMSNorm of every key head */
  float rope_theta;      /* > 0: rotary embedding of queries and keys at the tokens' original
                            positions, pairs (i, i + hd/2) rotated by pos * theta^(-2i/hd),
                            after the QK-norm; 0: none. (The page's backbones follow the Qwen3
                            structure, [XMOD] "backbone configuration"; the pages do not list
                            these parts, so they are options.) */
} xmod_layer;

/* Entry-point ids for xmod_workspace_bytes(). */
enum {
  XMOD_WS_ROUTE_TOPK = 0,
  XMOD_WS_SPARSE_LAYER = 1,
  XMOD_WS_DENSE_LAYER = 2,
  XMOD_WS_BLOCK = 3,
  XMOD_WS_SPARSE_THRESHOLD = 4,
  XMOD_WS_ROUTED_FFN = 5,
  XMOD_WS_ATTN_LAYER = 6,
  XMOD_WS_SPARSE_FULLKV = 7,
  XMOD_WS_TRAIN_SAVED = 8,  /* what xmod_sparse_layer_fwd_train keeps for the backward */
  XMOD_WS_BACKWARD = 9      /* workspace of xmod_sparse_layer_bwd */
};

/* Workspace bytes an entry point needs for these shapes (0 if none). K is ignored for the
 * dense layer. Returns 0 for invalid shapes as well; the entry point then reports the error. */
size_t xmod_workspace_bytes(const xmod_dims *dims, int32_t K, int32_t entry_point);

/* Router and top-k of one sparse layer ([XMOD] Eq. (8), "training-time top-k"; [MOD]).
 *   x [B,T,d] bf16; w_router [d] bf16; bias [B,T] fp32 or NULL (zeros), read only.
 *   logits [B,T] fp32 out: ell. idx [B,k] int32 out, ascending. gate [B,k] fp32 out:
 *   sigmoid(ell) at idx. k = floor(T/K). ws: xmod_workspace_bytes(dims, K, XMOD_WS_ROUTE_TOPK)
 *   bytes (0 for most shapes), or NULL; see xmod_topk_from_logits. */
xmod_status xmod_route_topk(const void *x, const void *w_router, float router_bias,
                            const float *bias, float tau, int32_t K, const xmod_dims *dims,
                            float *logits, int32_t *idx, float *gate, void *ws, size_t ws_bytes,
                            void *stream);

/* Top-k of given fp32 logits [B,T] ([XMOD] "training-time top-k": the top-1/K tokens of each
 * sequence; [MOD] "basic architecture": top-k of the router scores): idx [B,k] int32 ascending;
 * ties to the lower position (the MoE/SSM chapter's routing checklist asks for the tie rule to
 * be declared), -0 equals +0, NaN ranks lowest. gate [B,k] fp32 = sigmoid(logit) at idx
 * ([XMOD] Eq. (8)), or NULL. If bias is non-NULL, bias[b, idx] += delta (fp32): the carried
 * bias grows for every selected token ([XMOD] "three stabilisers").
 * ws: xmod_topk_workspace_bytes(B, T) bytes of device memory, or NULL. The size is nonzero for
 * sequences longer than 8192 positions (at most 32 MiB: large batches run in groups); with it
 * each sequence is split over several workgroups, without it each sequence runs on one
 * workgroup. Both write identical results. A ws smaller than needed: XMOD_ERR_WORKSPACE. */
size_t xmod_topk_workspace_bytes(int32_t B, int32_t T);
xmod_status xmod_topk_from_logits(const float *logits, int32_t B, int32_t T, int32_t k,
                                  int32_t *idx, float *gate, float *bias, float delta, void *ws,
                                  size_t ws_bytes, void *stream);

/* Gather the selected rows: x_packed[b*k + j] = x[b, idx[b,j]] (bit copy). x [B,T,d] bf16,
 * x_packed [B*k, d] bf16 out. ([MOD] "basic architecture": gather of the chosen tokens.) */
xmod_status xmod_pack(const void *x, const int32_t *idx, int32_t B, int32_t T, int32_t d,
                      int32_t k, void *x_packed, void *stream);

/* Gated scatter of [XMOD] Eq. (7), in place: for every packed row m = b*k + j,
 *   x[b, idx[b,j]] = bf16_rne(X + (varsigma * gate[m]) * (a[m] + f[m])), X = x[b, idx[b,j]],
 * each operation rounded in fp32 in that order (no fused multiply-add). Other rows of x are
 * not touched. a_packed, f_packed [B*k, d] bf16; gate [B*k] fp32. */
xmod_status xmod_scatter_gated(void *x, const int32_t *idx, const float *gate, float varsigma,
                               const void *a_packed, const void *f_packed, int32_t B, int32_t T,
                               int32_t d, int32_t k, void *stream);

/* Forward of one Sparse(K) layer ([XMOD] Fig. 1(b), Eqs. (7)-(8); Table 7), in place on x.
 *   bias [B,T] fp32 in/out or NULL: read for ell, then bias[idx] += delta.
 *   idx_out [B,k] int32 and gate_out [B,k] fp32: optional copies of the selection. */
xmod_status xmod_sparse_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                  int32_t K, float *bias, float tau, float delta,
                                  int32_t *idx_out, float *gate_out, void *ws, size_t ws_bytes,
                                  void *stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc): xmod_sparse_layer_fwd without a caller workspace.
 * The workspace is a static device array of XMOD_NOALLOC_SCRATCH_BYTES owned by the library,
 * one per GPU, held until the process ends; this call allocates nothing. Arguments and
 * results are those of xmod_sparse_layer_fwd (bit for bit: the same kernels run) minus
 * ws / ws_bytes. Returns XMOD_ERR_WORKSPACE, before any launch, when the layer needs more than
 * the array (xmod_workspace_bytes(dims, K, XMOD_WS_SPARSE_LAYER) > XMOD_NOALLOC_SCRATCH_BYTES;
 * e.g. 4 x 4096 tokens at d 1536, K 8 fit, 8 x 4096 at d 2048 do not). The kernels run on the
 * device of `stream` (the current device for the null stream). Every call on one GPU uses
 * that GPU's one array and leaves its contents behind: calls that may overlap on one GPU (on
 * different streams, or from host threads without ordering between them) race. */
#define XMOD_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
xmod_status xmod_sparse_layer_fwd_noalloc(void *x, const xmod_layer *layer,
                                          const xmod_dims *dims, int32_t K, float *bias,
                                          float tau, float delta, int32_t *idx_out,
                                          float *gate_out, void *stream);

/* Eval-time causal threshold routing of given fp32 logits [B,T] ([XMOD] "training-time top-k,
 * eval-time causal threshold"): a token enters when its routing probability sigmoid(ell) is at
 * least 1/2, i.e. ell >= 0 (-0 included, NaN never). Each sequence selects its own number of
 * tokens; the selection is written flat, sequence after sequence, ascending within each:
 *   counts [B] int32 out: tokens selected in sequence b;
 *   offsets [B] int32 out: first flat row of sequence b (sum of the counts before it);
 *   src [B*T] int32 out: flat row m -> row b*T + t of x (only the first *n_total are written);
 *   gate [B*T] fp32 out or NULL: sigmoid(ell) of flat row m;
 *   n_total [1] int32 out: number of selected tokens (device memory: no host sync happens);
 *   bias [B,T] fp32 in/out or NULL: bias[b,t] += delta for every selected token. */
xmod_status xmod_threshold_select(const float *logits, int32_t B, int32_t T, int32_t *counts,
                                  int32_t *offsets, int32_t *src, float *gate, int32_t *n_total,
                                  float *bias, float delta, void *stream);

/* Forward of one sparse layer with the eval-time causal threshold rule (same layer as
 * xmod_sparse_layer_fwd, every token with ell >= 0 selected), in place on x. The number of
 * selected rows stays on the device: the kernels are launched for all B*T rows and the surplus
 * workgroups exit at once, so the call never waits for the host. Attention is causal within each
 * sequence's own selected rows. Workspace: xmod_workspace_bytes(dims, 1,
 * XMOD_WS_SPARSE_THRESHOLD) (sized for B*T rows).
 *   bias [B,T] fp32 in/out or NULL: read for ell, then bias[selected] += delta.
 *   src_out [B*T], counts_out [B], n_total_out [1] int32: optional copies of the selection
 *   (as xmod_threshold_select; NULL to keep them in the workspace). */
xmod_status xmod_sparse_layer_fwd_threshold(void *x, const xmod_layer *layer,
                                            const xmod_dims *dims, float *bias, float tau,
                                            float delta, int32_t *src_out, int32_t *counts_out,
                                            int32_t *n_total_out, void *ws, size_t ws_bytes,
                                            void *stream);

/* Mask agreement of one sparse layer ([XMOD] "routing diagnostics", Table 10): from the same
 * logits [B,T] fp32, the top-k mask (idx [B,k] int32, the selected positions) and the threshold
 * mask (logit >= 0) are compared position by position; *agree (one uint32 in device memory) is
 * increased by the number of positions where both select or both skip. The caller zeroes
 * *agree and may accumulate over layers; the rate is agree / (B*T*layers). */
xmod_status xmod_mask_agreement(const float *logits, const int32_t *idx, int32_t B, int32_t T,
                                int32_t k, uint32_t *agree, void *stream);

/* --- Mechanism controls ([XMOD] "mechanism controls: conditional capacity vs attention
 * context", Table 7). ------------------------------------------------------------------------ */

/* One routed FFN refinement of the Routed-FFN control, in place on x: the sparse layer's router
 * and top-1/K selection, then only the FFN on the selected rows,
 *   y_S = X + (varsigma * r) * f,  f = SwiGLU(RMSNorm(X; g_ffn)),
 * unselected rows untouched, bias[idx] += delta. Uses w_router, router_bias, varsigma, g_ffn,
 * w_gate, w_up, w_down of the layer. Workspace: XMOD_WS_ROUTED_FFN. */
xmod_status xmod_routed_ffn_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                int32_t K, float *bias, float tau, float delta,
                                int32_t *idx_out, float *gate_out, void *ws, size_t ws_bytes,
                                void *stream);

/* The full-sequence attention block of the Routed-FFN control, in place on x:
 * y = x + Attn(RMSNorm(x; g_attn)) W_o^T for every token (causal over the whole sequence, GQA,
 * optional QK-norm / RoPE), no FFN. Uses g_attn, w_qkv, w_o and the layer-form options.
 * Workspace: XMOD_WS_ATTN_LAYER (K ignored). */
xmod_status xmod_attention_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                     void *ws, size_t ws_bytes, void *stream);

/* The Selected-Q/full-KV control, in place on x: the sparse layer's router, top-1/K selection,
 * gate, FFN and residual, but every token supplies keys and values: with u = RMSNorm(x; g_attn)
 * over all rows, K and V come from every row and Q from the selected rows, and the selected
 * query at original position t attends to all positions <= t. Workspace: XMOD_WS_SPARSE_FULLKV
 * (keys and values of all B*T rows). Arguments as xmod_sparse_layer_fwd. */
xmod_status xmod_sparse_layer_fwd_fullkv(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                         int32_t K, float *bias, float tau, float delta,
                                         int32_t *idx_out, float *gate_out, void *ws,
                                         size_t ws_bytes, void *stream);

/* Forward of one dense layer (every token, no gate): y = x + (a + f), in place on x, with
 * a = Attn(RMSNorm(x)) causal over the whole sequence and f = SwiGLU(RMSNorm(x + a)): the
 * [Dense] layer of the stacks of [XMOD] Eqs. (1) and (3) (the anchor of every block, the dense
 * prefix), pre-norm as [MOD] "basic architecture". Workspace: XMOD_WS_DENSE_LAYER. */
xmod_status xmod_dense_layer_fwd(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                 void *ws, size_t ws_bytes, void *stream);

/* Forward of the stack [Dense]xN0 + ([Sparse(K)]xAK + [Dense])xN1 ([XMOD] Eq. (3)), in place.
 * layers: host array of n_layers = N0 + N1*(A*K + 1) entries, in stack order. bias [B,T] fp32
 * is scratch for the carried bias: zeroed at the start of every block (the reset at each dense
 * anchor), grown by delta for each selection. A*K must be an integer (within 1e-6). */
xmod_status xmod_block_fwd(void *x, const xmod_layer *layers, int32_t n_layers,
                           const xmod_dims *dims, int32_t N0, int32_t N1, float A, int32_t K,
                           float *bias, float tau, float delta, void *ws, size_t ws_bytes,
                           void *stream);

/* --- Training: the sparse layer's backward pass. ----------------------------------------------
 *
 * [XMOD] "training-time top-k, eval-time causal threshold": the layer is trained with the
 * top-k routing and, beside the language-model loss, a routing loss (Eq. (9)): the binary
 * cross-entropy between the top-k decision q_i of every token and p_i = sigmoid(s_i), the
 * router's probability (s_i = w_r . x_i + beta_r, without the carried bias), averaged over the
 * n = B*T tokens and added with a small coefficient (the page picks 1e-4). The top-k choice and
 * the carried bias pass no gradient; the router's weights get theirs through the gate r of the
 * selected tokens (Eqs. (7)-(8)) and through the routing loss. Core layer form only: residual 0,
 * no QK-norm, no RoPE (XMOD_ERR_UNSUPPORTED otherwise). */

/* Gradients of one layer's parameters: device fp32 arrays with the shapes of the weights
 * (router_bias and varsigma: one float each). The backward writes them (no accumulation). */
typedef struct {
  float *w_router;     /* [d] */
  float *router_bias;  /* [1] */
  float *varsigma;     /* [1] */
  float *g_attn;       /* [d] */
  float *w_qkv;        /* [Hq*hd + 2*Hkv*hd, d] */
  float *w_o;          /* [d, Hq*hd] */
  float *g_ffn;        /* [d] */
  float *w_gate;       /* [F, d] */
  float *w_up;         /* [F, d] */
  float *w_down;       /* [d, F] */
} xmod_layer_grads;

/* xmod_sparse_layer_fwd (same arguments and results) that also keeps in `saved` (device, at
 * least xmod_workspace_bytes(dims, K, XMOD_WS_TRAIN_SAVED) bytes, caller-owned) everything the
 * backward reads: the router logits s, the selection and gates, the packed input rows X and
 * every intermediate of the attention and FFN of the selected rows. The contents of `saved`
 * are opaque and stay valid until the caller reuses the buffer. No other workspace. */
xmod_status xmod_sparse_layer_fwd_train(void *x, const xmod_layer *layer, const xmod_dims *dims,
                                        int32_t K, float *bias, float tau, float delta,
                                        int32_t *idx_out, float *gate_out, void *saved,
                                        size_t saved_bytes, void *stream);

/* Backward of the layer that xmod_sparse_layer_fwd_train ran (same layer, dims, K; its `saved`
 * unchanged since) for the objective <dy, y> + route_coef * L_route:
 *   x    [B, T, d] bf16: the hidden state as that forward left it (its unselected rows are the
 *        layer's input there);
 *   dy   [B, T, d] bf16: gradient of the objective's first term with respect to the output y;
 *   dx   [B, T, d] bf16 out: gradient with respect to the layer's input (may be dy itself);
 *   grads: parameter gradients (written); loss_route: device float receiving L_route, or NULL.
 * Workspace: XMOD_WS_BACKWARD. Gradients of activations are carried in bf16, weight gradients
 * and every sum in fp32; the sums over tokens are taken in a fixed order (deterministic). */
xmod_status xmod_sparse_layer_bwd(const void *x, const void *dy, void *dx,
                                  const xmod_layer *layer, const xmod_dims *dims, int32_t K,
                                  float route_coef, const void *saved, size_t saved_bytes,
                                  const xmod_layer_grads *grads, float *loss_route, void *ws,
                                  size_t ws_bytes, void *stream);

/* --- Stages of the path, exposed for stage-by-stage parity checks. ------------------------ */

/* Row-wise RMSNorm of gathered rows: out[m] = bf16(X / sqrt(mean(X^2) + eps) * gain), with
 * X = x[b, idx[b,j]] for m = b*k + j, or X = x[m] when idx is NULL (rows = B*k then). */
xmod_status xmod_rmsnorm_rows(const void *x, const int32_t *idx, const void *gain, float eps,
                              int32_t B, int32_t T, int32_t d, int32_t k, void *out, void *stream);

/* C[M,N] = bf16(A[M,K] B[N,K]^T), fp32 accumulate; all row-major, leading dims in elements.
 * K must be a multiple of 64; M*lda, N*ldb and M*ldc below 2^31 (XMOD_ERR_UNSUPPORTED). */
xmod_status xmod_gemm_bf16_nt(const void *A, int32_t lda, const void *Bm, int32_t ldb, void *C,
                              int32_t ldc, int32_t M, int32_t N, int32_t K, void *stream);

/* The products of the layer's backward pass (and the forward's, layout NT):
 * C[M, N] = sum_k A(m, k) B(n, k) with fp32 accumulation, where
 *   XMOD_GEMM_NT: A is [M, K] (lda >= K) and B is [N, K] (ldb >= K)     - x W^T (forward);
 *   XMOD_GEMM_NN: A is [M, K] (lda >= K) and B is [K, N] (ldb >= N)     - dY W (input gradient);
 *   XMOD_GEMM_TN: A is [K, M] (lda >= M) and B is [K, N] (ldb >= N)     - dY^T X (weight
 *                 gradient, a sum over the K token rows).
 * All row-major bf16, leading dimensions in elements, 16-byte aligned pointers. C is bf16
 * (round to nearest even, out_f32 = 0) or fp32 (out_f32 = 1); TN needs out_f32 = 1.
 * UNSUPPORTED: K not a multiple of 64, N or a leading dimension not a multiple of 8, M of a
 * k-major A not a multiple of 8, or an operand of 2^31 elements or more. */
enum { XMOD_GEMM_NT = 0, XMOD_GEMM_NN = 1, XMOD_GEMM_TN = 2 };
xmod_status xmod_gemm_bf16(int32_t layout, const void *A, int32_t lda, const void *Bm, int32_t ldb,
                           void *C, int32_t ldc, int32_t out_f32, int32_t M, int32_t N,
                           int32_t K, void *stream);

/* Causal attention over packed sequences ([XMOD] Table 7 "selected subset"; [MODA] 2.1 GQA):
 * qkv [B*k, ld_qkv] bf16 holds Q (Hq*hd columns), then K and V (Hkv*hd each) per row;
 * o [B*k, ld_o] bf16 out (Hq*hd columns). Row j of a sequence attends to rows 0..j. */
xmod_status xmod_attention_fwd(const void *qkv, int32_t ld_qkv, void *o, int32_t ld_o,
                               int32_t B, int32_t k, int32_t n_q_heads, int32_t n_kv_heads,
                               int32_t head_dim, void *stream);

/* Causal attention as xmod_attention_fwd that also stores lse [B*k, n_q_heads] fp32: for each
 * query row and head, log2 of the softmax normaliser in units where the weight of key j is
 * exp2(S_j * log2(e) / sqrt(head_dim) - lse). Needed by xmod_attention_bwd. */
xmod_status xmod_attention_fwd_lse(const void *qkv, int32_t ld_qkv, void *o, int32_t ld_o,
                                   float *lse, int32_t B, int32_t k, int32_t n_q_heads,
                                   int32_t n_kv_heads, int32_t head_dim, void *stream);

/* Backward of xmod_attention_fwd_lse for an output gradient dO [B*k, ld_do] bf16: with
 * D_q = sum_i dO[q][i] O[q][i], P = softmax of the scaled scores, dP = dO V^T and
 * dS = P * (dP - D_q): dQ = dS K / sqrt(hd), dK = dS^T Q / sqrt(hd), dV = P^T dO, dK and dV summed
 * over the query heads sharing a key/value head. Writes dqkv [B*k, ld_dqkv] bf16 in the [Q|K|V]
 * column layout of qkv (every column). D [B*k, n_q_heads] fp32 is caller scratch (written).
 * o and lse are the forward's outputs. Requirements as xmod_attention_fwd. */
xmod_status xmod_attention_bwd(const void *qkv, int32_t ld_qkv, const void *o, int32_t ld_o,
                               const float *lse, const void *dO, int32_t ld_do, float *D,
                               void *dqkv, int32_t ld_dqkv, int32_t B, int32_t k,
                               int32_t n_q_heads, int32_t n_kv_heads, int32_t head_dim,
                               void *stream);

/* --- Measurement hook. ------------------------------------------------------------------------
 * While enabled, the layer and block entry points record a hipEvent on their stream before
 * their first kernel and after every kernel they launch (events are created on first use, kept,
 * and record no system-scope fence); xmod_phase_timing_slots(mask) limits the recording to the
 * two ends of the kernel slots whose bit is set (default: every slot), so that a timed run pays
 * for two events per call instead of one per kernel. xmod_phase_times() waits for the last
 * recorded event, adds the time between the two events around each recorded kernel of every
 * recorded call into ms[i] for kernel slot i (sparse layer slots:
 * 0 router, 1 top-k, 2 gather+RMSNorm, 3 QKV GEMM, 4 attention, 5 O GEMM, 6 residual+RMSNorm,
 * 7 gate/up GEMM with SwiGLU, 8 down GEMM with gated scatter; a dense layer fills slots 2-8;
 * the training forward uses slots 0-8 as the sparse layer; the backward fills slots 9-22:
 * 9 gated residual, 10 dg GEMM with SwiGLU backward, 11 dW_down, 12 dv GEMM, 13 dW_gate|up,
 * 14 RMSNorm-2, 15 dO GEMM, 16 dW_o, 17 attention, 18 du GEMM, 19 dW_qkv, 20 RMSNorm-1 with dx of
 * the selected rows, 21 router and routing loss over every token, 22 sums of partial rows),
 * stores the number of recorded calls in *n_calls, and forgets the recorded events.
 * Not thread safe; meant for benchmarks, not for production calls or graph capture. */
void xmod_phase_timing_enable(int32_t on);
void xmod_phase_timing_slots(uint32_t mask);
xmod_status xmod_phase_times(float *ms, int32_t n_slots, int32_t *n_calls);

/* --- Ceiling probes (measurement only; no part of the layer). ----------------------------------
 * What the part sustains on the two kinds of work the layer's kernels are bound by, for a
 * benchmark to print beside the vendor peaks. Both enqueue one kernel of 1024 workgroups of 256
 * threads on the stream and write one value per thread to out (caller-owned device memory of
 * 1024 * 256 elements).
 * xmod_probe_mfma: every wave issues 4 * iters independent v_mfma_f32_32x32x16_bf16 on all-ones
 *   operands back to back (32768 flops each, 4 waves per workgroup); out[t] = 64 * iters
 *   (4 accumulators of 16 per product). INVALID_ARG: out NULL or iters outside [1, 2^18].
 * xmod_probe_read: reads `bytes` (a multiple of 16, 16-byte aligned) of src with 16-byte loads in
 *   a grid-stride pass, loads_in_flight (4, 8 or 16) independent loads outstanding per thread
 *   (16 * loads_in_flight KB per CU); out[t] = the 32-bit wrap-around sum of the words thread t
 *   read, so the sum over t equals that of every 32-bit word of src. INVALID_ARG: NULL pointer,
 *   bytes 0 or not a multiple of 16, loads_in_flight not 4, 8 or 16.
 * xmod_probe_read_chunked: the same read and the same out, but each of the 1024 workgroups reads
 *   its own contiguous 1/1024 share of src with non-temporal 16-byte loads (four 4 KB blocks of
 *   the share in flight), the faster way to stream a buffer larger than the last-level cache.
 *   Its lines are not kept by the caches, so unlike xmod_probe_read it does not flush them.
 *   INVALID_ARG: NULL pointer, bytes 0 or not a multiple of 16, src not 16-byte aligned. */
xmod_status xmod_probe_mfma(float *out, int32_t iters, void *stream);
xmod_status xmod_probe_read(const void *src, size_t bytes, int32_t loads_in_flight, uint32_t *out,
                            void *stream);
xmod_status xmod_probe_read_chunked(const void *src, size_t bytes, uint32_t *out, void *stream);

const char *xmod_status_string(xmod_status st);
int32_t xmod_last_hip_error(void);

#ifdef __cplusplus
}
#endif

#endif /* XMOD_H */
