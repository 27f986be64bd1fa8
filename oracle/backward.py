"""CPU oracle of the backward pass of one X-MoD Sparse(K) layer (test infrastructure only).

Plain float64 NumPy; see oracle/__init__.py for who may use it. Every gradient is the exact
derivative of the float64 forward of oracle.layer.sparse_layer (the fp32 rounding of the
router logit is treated as the identity), written out step by step with the chain rule in
the forward's order, reversed.

Sources (cited by page title and section / equation):
  [XMOD] "X-MoD: Practical Scaling Laws for Sparse-Depth Routing Beyond Mixture-of-Depths",
         close-reading page: Eq. (7) (gated residual of the selected rows with the layer
         scalar varsigma), Eq. (8) (gate r = sigmoid(s - tau*b)), "training-time top-k,
         eval-time causal threshold" (Eq. (9): the binary cross-entropy between the top-k
         decisions q_i and the routing probabilities p_i = sigmoid(s_i), averaged over the
         n tokens, added to the language-model loss with a small coefficient, 1e-4 chosen).
  [MOD]  "Mixture-of-Depths explained", "basic architecture": the gradient reaches the router
         only through the router weights that multiply the block output (top-k is a discrete
         choice and passes no gradient).

Readings:
  * The training objective of one layer is  <dy, y> + route_coef * L_route  for an upstream
    gradient dy of the hidden state; the top-k choice and the carried bias b receive no
    gradient (b is state, not a parameter); ell = s - tau*b, so d ell / d s = 1.
  * L_route uses p_i = sigmoid(s_i), the router logit without the carried bias, as Eq. (9)
    writes it, and n = B*T (every token of the batch is a decision of the router).
  * Gradients are taken of the core layer form (Eq. (7) residual, no QK-norm, no RoPE).
"""
from __future__ import annotations

import numpy as np

from .layer import _f64, router_logits, topk_select, sigmoid, causal_attention


def rmsnorm_grad(X, gain, eps, dY):
    """Gradients of Y = X / sqrt(mean(X^2) + eps) * gain over the last axis.

    With r = (mean(X^2) + eps)^(-1/2) and G = dY * gain:  dX = r*G - (r^3 / d) * (G . X) X,
    dgain = sum over rows of dY * X * r. Returns (dX, dgain)."""
    X = np.asarray(X, dtype=np.float64)
    dY = np.asarray(dY, dtype=np.float64)
    g = _f64(gain)
    d = X.shape[-1]
    r = 1.0 / np.sqrt(np.mean(X * X, axis=-1, keepdims=True) + float(eps))
    G = dY * g
    dX = r * G - (r ** 3 / d) * np.sum(G * X, axis=-1, keepdims=True) * X
    dgain = np.sum(dY * X * r, axis=tuple(range(X.ndim - 1)))
    return dX, dgain


def causal_attention_grad(Q, Kt, Vt, q_pos, n_q_heads, n_kv_heads, head_dim, dO):
    """Gradients of causal_attention (same arguments) for an output gradient dO [n, Hq*hd].

    Per query head h with KV head g = floor(h*Hkv/Hq): S = q k^T / sqrt(hd) on visible keys,
    P = softmax(S), O = P v.  dv_g += P^T dO_h;  dP = dO_h v_g^T;  dS = P * (dP - rowsum(dP*P));
    dq_h = dS k_g / sqrt(hd);  dk_g += dS^T q_h / sqrt(hd). Returns (dQ, dK, dV)."""
    Q = np.asarray(Q, dtype=np.float64)
    Kt = np.asarray(Kt, dtype=np.float64)
    Vt = np.asarray(Vt, dtype=np.float64)
    dO = np.asarray(dO, dtype=np.float64)
    q_pos = np.asarray(q_pos)
    n, m = Q.shape[0], Kt.shape[0]
    visible = np.arange(m)[None, :] <= q_pos[:, None]
    scale = 1.0 / np.sqrt(head_dim)
    dQ = np.zeros_like(Q)
    dK = np.zeros_like(Kt)
    dV = np.zeros_like(Vt)
    for h in range(n_q_heads):
        g = (h * n_kv_heads) // n_q_heads
        qs = slice(h * head_dim, (h + 1) * head_dim)
        ks = slice(g * head_dim, (g + 1) * head_dim)
        S = np.where(visible, (Q[:, qs] @ Kt[:, ks].T) * scale, -np.inf)
        P = np.exp(S - np.max(S, axis=1, keepdims=True))
        P = P / np.sum(P, axis=1, keepdims=True)
        dOh = dO[:, qs]
        dV[:, ks] += P.T @ dOh
        dP = dOh @ Vt[:, ks].T
        dS = P * (dP - np.sum(dP * P, axis=1, keepdims=True))
        dQ[:, qs] = (dS @ Kt[:, ks]) * scale
        dK[:, ks] += (dS.T @ Q[:, qs]) * scale
    return dQ, dK, dV


def silu_grad(z):
    """d/dz of z*sigmoid(z) = sigmoid(z) * (1 + z*(1 - sigmoid(z)))."""
    sg = sigmoid(z)
    return sg * (1.0 + z * (1.0 - sg))


def route_bce(s, idx):
    """[XMOD] Eq. (9): -(1/n) sum_i [q_i log p_i + (1 - q_i) log(1 - p_i)], p_i = sigmoid(s_i),
    q_i = 1 for the tokens the top-k chose (idx [B, k]); n = B*T. log p and log(1-p) are taken
    as -log(1 + e^-s) and -log(1 + e^s) (the same numbers, without cancellation)."""
    s = np.asarray(s, dtype=np.float64)
    B, T = s.shape
    q = np.zeros((B, T))
    q[np.arange(B)[:, None], np.asarray(idx)] = 1.0
    log_p = -np.logaddexp(0.0, -s)
    log_1mp = -np.logaddexp(0.0, s)
    return float(-np.sum(q * log_p + (1.0 - q) * log_1mp) / (B * T))


def route_bce_grad(s, idx):
    """d L_route / d s_i = (p_i - q_i) / n."""
    s = np.asarray(s, dtype=np.float64)
    B, T = s.shape
    q = np.zeros((B, T))
    q[np.arange(B)[:, None], np.asarray(idx)] = 1.0
    return (sigmoid(s) - q) / (B * T)


def sparse_layer_grad(x, lay, dims, K, dy, bias=None, tau=1.0, route_coef=1e-4,
                      forced_idx=None, exact_logits=False):
    """Backward of oracle.layer.sparse_layer (core form) for the objective
    <dy, y> + route_coef * L_route.

    x: [B, T, d] bf16 bits or values; dy: [B, T, d] upstream gradient (bits or values).
    Returns a dict: dx [B, T, d]; d_w_router [d], d_router_bias, d_varsigma (scalars);
    d_g_attn, d_g_ffn [d]; d_w_qkv, d_w_o, d_w_gate, d_w_up, d_w_down (shapes of the weights);
    loss_route (Eq. (9)); and the forward's idx and gate. exact_logits as in sparse_layer
    (fp32 logits by default, the precision the selection is decided in).

    Per sequence, on the packed selected rows X (ascending positions):
      forward  u = RMSNorm(X; g_attn), [Q|K|V] = u W_qkv^T, O = attention, a = O W_o^T,
               h = X + a, v = RMSNorm(h; g_ffn), zg = v W_gate^T, zu = v W_up^T,
               g = SiLU(zg) * zu, f = g W_down^T, t = a + f, c = varsigma * r,
               y = X + c t (Eq. (7));
      backward G = dy[S]; dt = c G; dc = rowsum(G * t); dr = varsigma dc;
               d varsigma = sum r dc; df = da = dt; then the FFN, RMSNorm-2 (dh adds to da
               and to dX), O projection, attention, QKV projection and RMSNorm-1 (adds to
               dX); dx[S] = G + dX.
    Router (every token): ds = [selected] dr * r(1 - r) + route_coef * (p - q)/n;
      d w_router = sum_t ds_t x_t, d router_bias = sum_t ds_t, dx_t += ds_t w_router.
    """
    if int(lay.get("residual", 0)) != 0 or lay.get("q_norm") is not None \
            or lay.get("k_norm") is not None or float(lay.get("rope_theta", 0.0) or 0.0) > 0:
        raise NotImplementedError("gradients of the core layer form only")
    x = _f64(x)
    dy = _f64(dy)
    B, T, d = x.shape
    k = T // K
    assert k >= 1
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    s, ell = router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau,
                           exact=exact_logits)
    idx = topk_select(ell, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    gate = sigmoid(np.asarray(ell, dtype=np.float64)[np.arange(B)[:, None], idx])
    vs = float(lay.get("varsigma", 1.0))
    eps = dims.rms_eps
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv, Wo = _f64(lay["w_qkv"]), _f64(lay["w_o"])
    Wg, Wu, Wd = _f64(lay["w_gate"]), _f64(lay["w_up"]), _f64(lay["w_down"])
    g1, g2 = _f64(lay["g_attn"]), _f64(lay["g_ffn"])

    out = {k_: np.zeros_like(v_) for k_, v_ in
           (("d_w_qkv", Wqkv), ("d_w_o", Wo), ("d_w_gate", Wg), ("d_w_up", Wu),
            ("d_w_down", Wd), ("d_g_attn", g1), ("d_g_ffn", g2))}
    d_vs = 0.0
    dx = dy.copy()
    dell = np.zeros((B, T))
    for b in range(B):
        sel = idx[b]
        X = x[b, sel]
        r = gate[b][:, None]
        # forward, keeping what the backward reads
        r1 = 1.0 / np.sqrt(np.mean(X * X, axis=1, keepdims=True) + eps)
        u = X * r1 * g1
        Q, Kt, Vt = u @ Wqkv[:dq].T, u @ Wqkv[dq:dq + dkv].T, u @ Wqkv[dq + dkv:].T
        pos = np.arange(len(sel))
        O = causal_attention(Q, Kt, Vt, pos, Hq, Hkv, hd)
        a = O @ Wo.T
        h = X + a
        r2 = 1.0 / np.sqrt(np.mean(h * h, axis=1, keepdims=True) + eps)
        v = h * r2 * g2
        zg, zu = v @ Wg.T, v @ Wu.T
        sg = sigmoid(zg)
        gact = zg * sg * zu
        f = gact @ Wd.T
        t = a + f
        # backward
        G = dy[b, sel]
        dt = (vs * r) * G
        dc = np.sum(G * t, axis=1)
        d_vs += float(np.sum(r[:, 0] * dc))
        dell[b, sel] = vs * dc * r[:, 0] * (1.0 - r[:, 0])
        # FFN
        out["d_w_down"] += dt.T @ gact
        dg = dt @ Wd
        dzg = dg * zu * silu_grad(zg)
        dzu = dg * zg * sg
        out["d_w_gate"] += dzg.T @ v
        out["d_w_up"] += dzu.T @ v
        dv = dzg @ Wg + dzu @ Wu
        dh, dg2 = rmsnorm_grad(h, g2, eps, dv)
        out["d_g_ffn"] += dg2
        da = dt + dh
        dX = G + dh
        # attention block
        out["d_w_o"] += da.T @ O
        dO = da @ Wo
        dQ, dK, dV = causal_attention_grad(Q, Kt, Vt, pos, Hq, Hkv, hd, dO)
        dqkv = np.concatenate([dQ, dK, dV], axis=1)
        out["d_w_qkv"] += dqkv.T @ u
        du = dqkv @ Wqkv
        dX1, dg1 = rmsnorm_grad(X, g1, eps, du)
        out["d_g_attn"] += dg1
        dx[b, sel] = dX + dX1
    ds = dell + float(route_coef) * route_bce_grad(s, idx)
    w_r = _f64(lay["w_router"])
    dx += ds[:, :, None] * w_r[None, None, :]
    out.update({"dx": dx, "d_w_router": np.einsum("bt,btc->c", ds, x),
                "d_router_bias": float(np.sum(ds)), "d_varsigma": d_vs,
                "loss_route": route_bce(s, idx), "idx": idx, "gate": gate, "ds": ds})
    return out
