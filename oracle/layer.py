"""CPU oracle of one X-MoD sparse-depth layer and of a dense layer (test infrastructure only).

Plain float64 NumPy written from the pages; see oracle/__init__.py for who may use it.

Sources (cited by page title and section / equation):
  [XMOD] "X-MoD: Practical Scaling Laws for Sparse-Depth Routing Beyond Mixture-of-Depths",
         close-reading page. Sections "X-MoD: decoupling token sparsity K and anchor stride A"
         (Eqs. (3)-(5), Fig. 1(b)), "three stabilisers" (Eqs. (6)-(8)), "training-time top-k",
         "backbone configuration" (Table 4), "mechanism controls" (Table 7), "training-time
         top-k, eval-time causal threshold", "routing diagnostics" (Table 10).
  [MOD]  "Mixture-of-Depths explained" blog page, section "basic architecture" (the MoDLayer
         sketch: scalar Linear(d, 1) router, top-k of int(T * ratio) tokens, RMSNorm before
         attention and before the FFN, skipped rows passed through).
  [MOE]  "Beyond dense Transformers: MoE, SSMs and hybrids" page, section on stored versus
         evaluated parameters (bias-free SwiGLU with gate, value and down projections).
  [MODA] "Mixture-of-Depths Attention" reading notes, section 2.1 (GQA: query head h reads
         key/value head ceil(h/G), 1-based, G = Hq/Hkv).

Readings taken where the pages are silent or ambiguous:
  * ell = s - tau*b, with the gate r = sigmoid(ell) taken from the biased logit (Eq. (8)).
  * Selection ranks fp32 ell, ties to the lower position; -0 equals +0. k = floor(T/K).
  * Selected rows are packed in ascending position; attention is causal over the selected
    subset only, per sequence (Table 7: KV context "selected subset").
  * FFN input is RMSNorm(X + a) (sequential pre-norm); output y = X + varsigma*r*(a + f).
  * The bias update b[S] += delta happens after the gate is read.
  * Softmax scale 1/sqrt(head_dim); GQA head h uses KV head floor(h*Hkv/Hq) (0-based).
  * Layer-form options (lay keys, absent = off): "residual" 1 for MoD's Eq. (6); "q_norm" /
    "k_norm" gains for a per-head RMSNorm of queries / keys and "rope_theta" > 0 for rotary
    embedding (rotate-half pairs) at original positions, applied in that order, as in the
    Qwen3 structure the page's backbones follow.
  * Eval-time threshold routing: the probability that is compared with 1/2 is the gate of
    Eq. (8), sigmoid(s - tau*b) (the pages' routing diagnostics run threshold-driven forwards
    with and without the carried bias and get different coverage), decided as ell >= 0.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_to_f64


def _f64(a):
    a = np.asarray(a)
    if a.dtype == np.uint16:
        return bf16_to_f64(a)
    return a.astype(np.float64)


# --- router: [MOD] "basic architecture" (Linear(d, 1) score), [XMOD] Eq. (8) -------------------

def router_logits(x, w_router, router_bias=0.0, bias=None, tau=1.0, exact=False):
    """Router logit s_t = w_r . x_t + beta_r and bias-adjusted logit ell_t = s_t - tau * b_t.

    The dot product is taken in float64 and rounded once to fp32 ("the oracle's logit"). The
    adjustment is fp32 arithmetic: tau*b rounded, then the subtraction rounded ([XMOD] Eq. (8)
    subtracts tau*b_i before the top-1/K choice). Returns (s, ell), both float32 [B, T].

    exact=True keeps both in float64 with no rounding (a smooth function of the inputs, for
    derivative checks by finite differences); the selection is still ranked on fp32 values.
    """
    x = _f64(x)
    w = _f64(w_router)
    if bias is None:
        bias = np.zeros(x.shape[:2], dtype=np.float32)
    if exact:
        s = x @ w + float(router_bias)
        return s, s - float(tau) * np.asarray(bias, dtype=np.float64)
    s = (x @ w + float(router_bias)).astype(np.float32)
    tb = np.float32(tau) * np.asarray(bias, dtype=np.float32)
    ell = (s - tb).astype(np.float32)
    return s, ell


# --- selection: [XMOD] "training-time top-k", [MOD] "basic architecture" -----------------------

def topk_select(ell, k):
    """Per sequence, the k tokens with the largest fp32 ell; equal values go to the lower index.

    Returns idx int64 [B, k] in ascending position order. [XMOD] Eq. (1): a Sparse(K) layer
    processes only the top-1/K share of tokens; the ordering among equal logits is not fixed by
    the pages and is taken as lower position first.
    """
    ell = np.asarray(ell, dtype=np.float32)
    assert np.all(np.isfinite(ell)), "router logits must be finite"
    B, T = ell.shape
    assert 1 <= k <= T
    out = np.empty((B, k), dtype=np.int64)
    pos = np.arange(T)
    for b in range(B):
        # Primary key: -ell ascending (ell descending); secondary: position ascending.
        order = np.lexsort((pos, -ell[b].astype(np.float64)))
        out[b] = np.sort(order[:k])
    return out


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


# --- layer pieces ------------------------------------------------------------------------------

def rmsnorm(X, gain, eps):
    """RMSNorm over the last axis: X / sqrt(mean(X^2) + eps) * gain ([MOD] norm1/norm2)."""
    X = np.asarray(X, dtype=np.float64)
    ms = np.mean(X * X, axis=-1, keepdims=True)
    return X / np.sqrt(ms + float(eps)) * _f64(gain)


def causal_attention(Q, Kt, Vt, q_pos, n_q_heads, n_kv_heads, head_dim):
    """Causal multi-head attention with grouped KV heads, over one packed sequence.

    Q: [n, Hq*hd] rows for queries at packed positions q_pos; Kt, Vt: [m, Hkv*hd] for packed
    positions 0..m-1. Query i sees keys j <= q_pos[i]. Head h reads KV head floor(h*Hkv/Hq)
    ([MODA] section 2.1, 0-based). Scores scaled by 1/sqrt(hd), softmax over visible keys.
    """
    Q = np.asarray(Q, dtype=np.float64)
    Kt = np.asarray(Kt, dtype=np.float64)
    Vt = np.asarray(Vt, dtype=np.float64)
    q_pos = np.asarray(q_pos)
    n, m = Q.shape[0], Kt.shape[0]
    assert np.all(q_pos < m)
    visible = np.arange(m)[None, :] <= q_pos[:, None]          # [n, m]
    out = np.empty((n, n_q_heads * head_dim), dtype=np.float64)
    scale = 1.0 / np.sqrt(head_dim)
    for h in range(n_q_heads):
        g = (h * n_kv_heads) // n_q_heads
        q = Q[:, h * head_dim:(h + 1) * head_dim]
        kk = Kt[:, g * head_dim:(g + 1) * head_dim]
        vv = Vt[:, g * head_dim:(g + 1) * head_dim]
        S = (q @ kk.T) * scale
        S = np.where(visible, S, -np.inf)
        S = S - np.max(S, axis=1, keepdims=True)
        P = np.exp(S)
        P = P / np.sum(P, axis=1, keepdims=True)
        out[:, h * head_dim:(h + 1) * head_dim] = P @ vv
    return out


def silu(z):
    z = np.asarray(z, dtype=np.float64)
    return z * sigmoid(z)


def swiglu_ffn(v, w_gate, w_up, w_down):
    """Bias-free SwiGLU: (SiLU(v Wg^T) * (v Wu^T)) Wd^T ([MOE] gate, value and down projections)."""
    return (silu(v @ _f64(w_gate).T) * (v @ _f64(w_up).T)) @ _f64(w_down).T


# --- layer-form options of the Qwen3-style backbones: [XMOD] "backbone configuration" ---------

def qk_head_norm(Z, n_heads, head_dim, gain, eps):
    """RMSNorm of every head_dim slice of Z [n, n_heads*head_dim], gain [head_dim] shared by
    the heads (QK-norm of the Qwen3 backbones the page's 556M / 1.65B models follow)."""
    Z = np.asarray(Z, dtype=np.float64).reshape(Z.shape[0], n_heads, head_dim)
    ms = np.mean(Z * Z, axis=-1, keepdims=True)
    return (Z / np.sqrt(ms + float(eps)) * _f64(gain)).reshape(Z.shape[0], n_heads * head_dim)


def rope(Z, positions, n_heads, head_dim, theta):
    """Rotary position embedding of every head of Z [n, n_heads*head_dim] at positions [n].

    Pairs (i, i + head_dim/2), i < head_dim/2, rotate by the angle p * theta^(-2i/head_dim):
    (z_i, z_j) -> (z_i cos - z_j sin, z_j cos + z_i sin). The positions are the tokens'
    original positions in their sequence (a routed token keeps its place in the text)."""
    Z = np.asarray(Z, dtype=np.float64).reshape(Z.shape[0], n_heads, head_dim)
    h = head_dim // 2
    inv = float(theta) ** (-2.0 * np.arange(h) / head_dim)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * inv[None, :]      # [n, h]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    z1, z2 = Z[..., :h], Z[..., h:]
    out = np.concatenate([z1 * c - z2 * s, z2 * c + z1 * s], axis=-1)
    return out.reshape(Z.shape[0], n_heads * head_dim)


def _qk_form(Q, Kt, lay, dims, q_pos_orig, k_pos_orig):
    """Apply the optional QK-norm (lay["q_norm"], lay["k_norm"]) then RoPE (lay["rope_theta"]
    > 0) to query and key rows at their original positions."""
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    if lay.get("q_norm") is not None:
        Q = qk_head_norm(Q, Hq, hd, lay["q_norm"], dims.rms_eps)
    if lay.get("k_norm") is not None:
        Kt = qk_head_norm(Kt, Hkv, hd, lay["k_norm"], dims.rms_eps)
    theta = float(lay.get("rope_theta", 0.0) or 0.0)
    if theta > 0:
        Q = rope(Q, q_pos_orig, Hq, hd, theta)
        Kt = rope(Kt, k_pos_orig, Hkv, hd, theta)
    return Q, Kt


def _attn_ffn_on_rows(X, lay, dims, out_rows, positions=None):
    """Attention residual a and FFN residual f for rows out_rows of one packed sequence X.

    u = RMSNorm(X; g_attn); [Q|K|V] = u W_qkv^T; optional QK-norm and RoPE at the rows'
    original positions (positions[j] for packed row j); O = causal attention over X's rows;
    a = O W_o^T; v = RMSNorm(X + a; g_ffn); f = SwiGLU(v). Only rows 0..max(out_rows) of X
    are needed (causality), so only those are projected to keys and values.
    """
    out_rows = np.asarray(out_rows)
    m = int(out_rows.max()) + 1
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv = _f64(lay["w_qkv"])
    u = rmsnorm(X[:m], lay["g_attn"], dims.rms_eps)
    Q = u[out_rows] @ Wqkv[:dq].T
    Kt = u @ Wqkv[dq:dq + dkv].T
    Vt = u @ Wqkv[dq + dkv:dq + 2 * dkv].T
    pos = np.arange(X.shape[0]) if positions is None else np.asarray(positions)
    Q, Kt = _qk_form(Q, Kt, lay, dims, pos[out_rows], pos[:m])
    O = causal_attention(Q, Kt, Vt, out_rows, Hq, Hkv, hd)
    a = O @ _f64(lay["w_o"]).T
    v = rmsnorm(X[out_rows] + a, lay["g_ffn"], dims.rms_eps)
    f = swiglu_ffn(v, lay["w_gate"], lay["w_up"], lay["w_down"])
    return a, f


# --- the Sparse(K) layer: [XMOD] Fig. 1(b), Eqs. (7)-(8) ---------------------------------------

def _routed_layer(x, lay, dims, ell, sel, bias, delta, sample):
    """The routed part of a sparse layer for given selections sel[b] (ascending positions).

    gate r = sigmoid(ell) on the selected tokens; attention and FFN over the packed selected
    rows only; y_S = X + varsigma * r * (a + f) ([XMOD] Eq. (7)), or with lay["residual"] == 1
    the MoD form y_S = X + a + r * f (Eq. (6)); unselected rows y = x (Fig. 1(b), skip path);
    then b[S] += delta in fp32. sample: None or {b: packed rows}.
    """
    B = x.shape[0]
    gate = [sigmoid(ell[b, sel[b]]) for b in range(B)]
    bias_out = bias.copy()
    for b in range(B):
        bias_out[b, sel[b]] = (bias[b, sel[b]] + np.float32(delta)).astype(np.float32)
    vs = float(lay.get("varsigma", 1.0))
    res = {"gate": gate, "bias_out": bias_out}
    seqs = range(B) if sample is None else sorted(sample)
    y = x.copy() if sample is None else None
    rows = {}
    for b in seqs:
        if len(sel[b]) == 0:
            continue
        X = x[b, sel[b]]                                      # packed, ascending position
        out_rows = np.arange(len(sel[b])) if sample is None else np.asarray(sample[b])
        if len(out_rows) == 0:
            continue
        a, f = _attn_ffn_on_rows(X, lay, dims, out_rows, positions=sel[b])
        r = gate[b][out_rows][:, None]
        if int(lay.get("residual", 0)) == 1:       # MoD, [XMOD] Eq. (6): only f is gated
            y_sel = X[out_rows] + a + r * f
        else:                                      # X-MoD, Eq. (7)
            y_sel = X[out_rows] + (vs * r) * (a + f)
        if sample is None:
            y[b, sel[b]] = y_sel
        else:
            rows[b] = (out_rows, sel[b][out_rows], y_sel)
    if sample is None:
        res["y"] = y
    else:
        res["rows"] = rows
    return res


def sparse_layer(x, lay, dims, K, bias=None, tau=1.0, delta=0.0, forced_idx=None, sample=None,
                 exact_logits=False):
    """Forward of one X-MoD Sparse(K) layer with the training-time top-k selection.

    x: [B, T, d] bf16 bits or float64 values. lay: dict of layer weights (bf16 bits) plus
    "router_bias" and "varsigma". bias: fp32 [B, T] carried bias or None (zeros).

    Steps: router logit and bias adjustment (Eq. (8)); per sequence top-k with k = floor(T/K);
    gate r = sigmoid(ell) on the selected tokens; attention and FFN over the packed selected
    rows only; y_S = X + varsigma * r * (a + f) (Eq. (7)); unselected rows y = x (Fig. 1(b),
    skip path); then b[S] += delta in fp32 (the bias grows when a token is chosen).

    sample: None for the whole output, or {b: packed rows} to evaluate only those rows of those
    sequences (each output row is computed exactly as in the full evaluation).
    exact_logits: float64 logits with no fp32 rounding (router_logits(exact=True)).

    Returns a dict with s, ell (fp32), idx (int64 [B, k]), gate (float64 [B, k]), bias_out
    (fp32), and either y (float64 [B, T, d]) or rows {b: (packed rows, positions, y rows)}.
    """
    x = _f64(x)
    B, T, d = x.shape
    k = T // K
    assert k >= 1, "floor(T/K) must be at least 1"
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    s, ell = router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau,
                           exact=exact_logits)
    idx = topk_select(ell, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    res = _routed_layer(x, lay, dims, ell, [idx[b] for b in range(B)], bias, delta, sample)
    res.update({"s": s, "ell": ell, "idx": idx, "gate": np.stack(res["gate"])})
    return res


# --- eval-time causal threshold routing: [XMOD] "training-time top-k, eval-time causal threshold"

def threshold_select(ell):
    """Per sequence, the tokens whose routing probability sigmoid(ell) is at least 1/2.

    sigmoid(ell) >= 1/2 exactly when ell >= 0, so the rule is taken on the fp32 logit itself
    (-0 counts as 0); it is causal, each token's decision reads only its own logit. Returns a
    list of int64 arrays of ascending positions, one per sequence (possibly empty).
    """
    ell = np.asarray(ell, dtype=np.float32)
    assert np.all(np.isfinite(ell)), "router logits must be finite"
    return [np.nonzero(ell[b] >= 0)[0].astype(np.int64) for b in range(ell.shape[0])]


def sparse_layer_threshold(x, lay, dims, bias=None, tau=1.0, delta=0.0, sample=None,
                           forced_sel=None):
    """Forward of one sparse layer with the eval-time causal threshold rule.

    Identical to sparse_layer except for the selection: every token with ell = s - tau*b >= 0
    enters (Eq. (8)'s r = sigmoid(ell) >= 1/2), so each sequence routes its own number of
    tokens k_b (0 .. T). The carried bias is updated on the selected tokens as in training.
    forced_sel: a given selection (list of ascending position arrays, one per sequence) used
    instead of the rule, as sparse_layer's forced_idx.

    Returns a dict with s, ell, idx (list of int64 arrays), counts (int64 [B]), gate (list),
    bias_out, and y or rows (as sparse_layer; sample: {b: packed rows of that sequence}).
    """
    x = _f64(x)
    B, T, d = x.shape
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    s, ell = router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau)
    sel = threshold_select(ell) if forced_sel is None else [np.asarray(v, dtype=np.int64)
                                                             for v in forced_sel]
    res = _routed_layer(x, lay, dims, ell, sel, bias, delta, sample)
    res.update({"s": s, "ell": ell, "idx": sel,
                "counts": np.array([len(v) for v in sel], dtype=np.int64)})
    return res


def mask_agreement(ell, idx):
    """Mask agreement of [XMOD] "routing diagnostics" (Table 10) for one sparse layer.

    From the same routing scores ell, the top-k mask (positions idx [B, k]) and the threshold
    mask (ell >= 0) are compared position by position; a position agrees when both select it
    or both skip it. Returns (agreeing positions, all positions).
    """
    ell = np.asarray(ell, dtype=np.float32)
    B, T = ell.shape
    topk = np.zeros((B, T), dtype=bool)
    topk[np.arange(B)[:, None], np.asarray(idx)] = True
    thr = ell >= 0
    return int(np.sum(topk == thr)), B * T


def differing_selected_share(agreement, K):
    """The page's rough reading of a mask agreement rate (Table 10 commentary): if both masks
    select the same number of tokens, the disagreeing positions split evenly into top-k-only
    and threshold-only tokens, so the share of selected tokens that differ is
    ((1 - agreement) / 2) / (1 / K)."""
    return (1.0 - float(agreement)) / 2.0 * float(K)


# --- mechanism controls: [XMOD] "mechanism controls: conditional capacity vs attention
#     context" (Table 7 and the two counterfactuals above it) ----------------------------------

def attention_layer(x, lay, dims, sample=None):
    """The full-sequence attention block of the Routed-FFN control: y = x + Attn(RMSNorm(x))
    for every token (causal over the whole sequence; optional QK-norm / RoPE), no FFN.
    sample: None or {b: positions}."""
    x = _f64(x)
    B, T, d = x.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv = _f64(lay["w_qkv"])
    out = x.copy() if sample is None else {}
    for b in (range(B) if sample is None else sorted(sample)):
        rows = np.arange(T) if sample is None else np.asarray(sample[b])
        m = int(rows.max()) + 1
        u = rmsnorm(x[b, :m], lay["g_attn"], dims.rms_eps)
        Q = u[rows] @ Wqkv[:dq].T
        Kt = u @ Wqkv[dq:dq + dkv].T
        Vt = u @ Wqkv[dq + dkv:].T
        Q, Kt = _qk_form(Q, Kt, lay, dims, rows, np.arange(m))
        y = x[b, rows] + causal_attention(Q, Kt, Vt, rows, Hq, Hkv, hd) @ _f64(lay["w_o"]).T
        if sample is None:
            out[b] = y
        else:
            out[b] = (rows, y)
    return out


def routed_ffn_layer(x, lay, dims, K, bias=None, tau=1.0, delta=0.0, forced_idx=None):
    """A routed FFN refinement of the Routed-FFN control: the router and top-1/K selection of
    the sparse layer, then only the FFN on the selected rows, y_S = X + varsigma * r * f with
    f = SwiGLU(RMSNorm(X; g_ffn)) (the gated residual of Eq. (7) with no attention part);
    unselected rows unchanged; b[S] += delta. Returns the same dict as sparse_layer (no
    sampling: the FFN is row-local, so every row is cheap). forced_idx: a given selection
    [B, k] instead of the top-k, as in sparse_layer."""
    x = _f64(x)
    B, T, d = x.shape
    k = T // K
    assert k >= 1
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    s, ell = router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau)
    idx = topk_select(ell, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    bsel = np.arange(B)[:, None]
    gate = sigmoid(ell[bsel, idx])
    bias_out = bias.copy()
    bias_out[bsel, idx] = (bias[bsel, idx] + np.float32(delta)).astype(np.float32)
    vs = float(lay.get("varsigma", 1.0))
    y = x.copy()
    for b in range(B):
        X = x[b, idx[b]]
        f = swiglu_ffn(rmsnorm(X, lay["g_ffn"], dims.rms_eps), lay["w_gate"], lay["w_up"],
                       lay["w_down"])
        y[b, idx[b]] = X + (vs * gate[b])[:, None] * f
    return {"s": s, "ell": ell, "idx": idx, "gate": gate, "bias_out": bias_out, "y": y}


def sparse_layer_fullkv(x, lay, dims, K, bias=None, tau=1.0, delta=0.0, sample=None,
                        forced_idx=None):
    """The Selected-Q/full-KV control: the sparse layer's router, selection, gate, FFN and
    residual (Eq. (7)), but every token of the sequence supplies keys and values: the query of
    a selected token at original position t attends to all tokens at positions <= t.

    u = RMSNorm(x; g_attn) over all rows; K, V from every row; Q from the selected rows;
    optional QK-norm / RoPE at original positions. sample: None or {b: packed rows};
    forced_idx: a given selection [B, k] instead of the top-k, as in sparse_layer."""
    x = _f64(x)
    B, T, d = x.shape
    k = T // K
    assert k >= 1
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    bias = np.asarray(bias, dtype=np.float32)
    s, ell = router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau)
    idx = topk_select(ell, k) if forced_idx is None else np.asarray(forced_idx, dtype=np.int64)
    bsel = np.arange(B)[:, None]
    gate = sigmoid(ell[bsel, idx])
    bias_out = bias.copy()
    bias_out[bsel, idx] = (bias[bsel, idx] + np.float32(delta)).astype(np.float32)
    vs = float(lay.get("varsigma", 1.0))
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv = _f64(lay["w_qkv"])
    res = {"s": s, "ell": ell, "idx": idx, "gate": gate, "bias_out": bias_out}
    y = x.copy() if sample is None else None
    rows_out = {}
    for b in (range(B) if sample is None else sorted(sample)):
        prow = np.arange(k) if sample is None else np.asarray(sample[b])
        pos = idx[b, prow]                                   # original positions of the queries
        m = int(pos.max()) + 1
        u = rmsnorm(x[b, :m], lay["g_attn"], dims.rms_eps)
        Q = u[pos] @ Wqkv[:dq].T
        Kt = u @ Wqkv[dq:dq + dkv].T
        Vt = u @ Wqkv[dq + dkv:].T
        Q, Kt = _qk_form(Q, Kt, lay, dims, pos, np.arange(m))
        a = causal_attention(Q, Kt, Vt, pos, Hq, Hkv, hd) @ _f64(lay["w_o"]).T
        X = x[b, pos]
        f = swiglu_ffn(rmsnorm(X + a, lay["g_ffn"], dims.rms_eps), lay["w_gate"], lay["w_up"],
                       lay["w_down"])
        y_sel = X + (vs * gate[b, prow])[:, None] * (a + f)
        if sample is None:
            y[b, pos] = y_sel
        else:
            rows_out[b] = (prow, pos, y_sel)
    if sample is None:
        res["y"] = y
    else:
        res["rows"] = rows_out
    return res


# --- the dense layer: every token enters, no gate ---------------------------------------------

def dense_layer(x, lay, dims, sample=None):
    """Pre-norm dense layer over whole sequences: y = x + a + f.

    a = Attn(RMSNorm(x)) causal over all T positions; f = SwiGLU(RMSNorm(x + a)). This is the
    [Dense] layer of the stack in [XMOD] Eq. (3). Written independently of the routed path:
    it never gathers, scatters or gates. sample: None or {b: positions}.
    """
    x = _f64(x)
    B, T, d = x.shape
    Hq, Hkv, hd = dims.n_q_heads, dims.n_kv_heads, dims.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv = _f64(lay["w_qkv"])
    Wo = _f64(lay["w_o"])
    out = x.copy() if sample is None else {}
    for b in (range(B) if sample is None else sorted(sample)):
        rows = np.arange(T) if sample is None else np.asarray(sample[b])
        m = int(rows.max()) + 1
        u = rmsnorm(x[b, :m], lay["g_attn"], dims.rms_eps)
        Q = u[rows] @ Wqkv[:dq].T
        Kt = u @ Wqkv[dq:dq + dkv].T
        Vt = u @ Wqkv[dq + dkv:].T
        Q, Kt = _qk_form(Q, Kt, lay, dims, rows, np.arange(m))
        a = causal_attention(Q, Kt, Vt, rows, Hq, Hkv, hd) @ Wo.T
        h = x[b, rows] + a
        f = swiglu_ffn(rmsnorm(h, lay["g_ffn"], dims.rms_eps), lay["w_gate"], lay["w_up"], lay["w_down"])
        y = x[b, rows] + a + f
        if sample is None:
            out[b] = y
        else:
            out[b] = (rows, y)
    return out
