"""A float64 model of the sparse layer whose only roundings are bf16 operand roundings (tests only).

Not the oracle. The oracle (oracle/) computes the layer in float64 with no intermediate
rounding. Any implementation that feeds the matrix cores bf16 operands stores some of the
layer's intermediates in bf16, and those roundings alone move the output away from the
float64 result; how far depends on the depth of the contractions that follow them (d, F, k).
This model measures that distance on the same inputs: it takes the oracle's own selection and
computes the routed rows exactly as the oracle does (X-MoD review Fig. 1(b), Eqs. (7)-(8);
causal attention over the selected subset, Table 7; bias-free SwiGLU of the MoE/SSM chapter),
except that the values a bf16-operand implementation stores in bf16 are rounded to bf16
(nearest even) at the point where they are produced:

  u = bf16(RMSNorm(X; g_attn))             operand of the QKV product
  Q, K, V = bf16(u W^T)                    operands of the attention products
  P = bf16(exp(S - rowmax))  (optional)    operand of the P V product (the sum l stays exact)
  O = bf16(P V / l)                        operand of the O product
  v = bf16(RMSNorm(X + a; g_ffn))          operand of the gate/up product
  g = bf16(SiLU(v Wg^T) * (v Wu^T))        operand of the down product

a = O W_o^T and f = g W_down^T stay float64 (they only feed the residual), and so do the
residual y = X + varsigma * r * (a + f) and every sum. The model shares no code with the HIP
library; it reuses the oracle's router, selection, RMSNorm and SiLU.
"""
from __future__ import annotations

import numpy as np

import oracle


def _bf16(v):
    return oracle.round_to_bf16(v)


def _attention_bf16(Q, Kt, Vt, q_rows, Hq, Hkv, hd, round_p, rnd, acc):
    n, m = Q.shape[0], Kt.shape[0]
    visible = np.arange(m)[None, :] <= np.asarray(q_rows)[:, None]
    out = np.empty((n, Hq * hd), dtype=acc)
    scale = acc(1.0 / np.sqrt(hd))
    for h in range(Hq):
        g = (h * Hkv) // Hq
        S = (Q[:, h * hd:(h + 1) * hd] @ Kt[:, g * hd:(g + 1) * hd].T) * scale
        S = np.where(visible, S, -np.inf)
        P = np.exp(S - S.max(axis=1, keepdims=True))
        l = P.sum(axis=1, keepdims=True)
        if round_p:
            P = rnd(P).astype(acc)
        out[:, h * hd:(h + 1) * hd] = (P @ Vt[:, g * hd:(g + 1) * hd]) / l
    return out


def sparse_layer_rows(xb, lay, w, K, bias=None, tau=1.0, sample=None, round_p=False,
                      rounding=True, forced_idx=None, accumulate=np.float64):
    """Routed output rows of one sparse layer under the bf16-operand model.

    xb: bf16 bits [B, T, d]; lay: layer weights as produced by workload.make_layer; sample:
    {b: packed rows} (None: every routed row of every sequence). The selection is the oracle's
    (top-k of the fp32 logits) unless forced_idx [B, k] gives one. accumulate=np.float32 takes
    every product and sum after the router in fp32 (the precision a matrix core accumulates in)
    instead of float64; the residual is still formed in float64. rounding=False leaves every value in float64 (the model is then
    the oracle's layer, computed in a different order). Returns {b: (packed rows, positions,
    y rows float64)}.
    """
    acc = accumulate
    rnd = (lambda v: _bf16(v).astype(acc)) if rounding else (lambda v: np.asarray(v, dtype=acc))
    x = oracle.bf16_to_f64(xb)
    B, T, d = x.shape
    k = T // K
    if bias is None:
        bias = np.zeros((B, T), dtype=np.float32)
    _, ell = oracle.router_logits(x, lay["w_router"], lay.get("router_bias", 0.0), bias, tau)
    idx = oracle.topk_select(ell, k) if forced_idx is None else np.asarray(forced_idx, np.int64)
    Hq, Hkv, hd = w.n_q_heads, w.n_kv_heads, w.head_dim
    dq, dkv = Hq * hd, Hkv * hd
    Wqkv = oracle.bf16_to_f64(lay["w_qkv"]).astype(acc)
    Wo = oracle.bf16_to_f64(lay["w_o"]).astype(acc)
    Wg, Wu, Wd = (oracle.bf16_to_f64(lay[n]).astype(acc) for n in ("w_gate", "w_up", "w_down"))
    vs = float(lay.get("varsigma", 1.0))
    out = {}
    for b in (range(B) if sample is None else sorted(sample)):
        rows = np.arange(k) if sample is None else np.asarray(sample[b])
        m = int(rows.max()) + 1
        X = x[b, idx[b]]
        u = rnd(oracle.rmsnorm(X[:m], lay["g_attn"], w.rms_eps))
        Q = rnd(u[rows] @ Wqkv[:dq].T)
        Kt = rnd(u @ Wqkv[dq:dq + dkv].T)
        Vt = rnd(u @ Wqkv[dq + dkv:].T)
        O = rnd(_attention_bf16(Q, Kt, Vt, rows, Hq, Hkv, hd, round_p, rnd, acc))
        a = O @ Wo.T
        v = rnd(oracle.rmsnorm(X[rows] + a, lay["g_ffn"], w.rms_eps))
        zg, zu = v @ Wg.T, v @ Wu.T
        g = rnd(zg / (1 + np.exp(-zg)) * zu)
        f = g @ Wd.T
        r = oracle.sigmoid(ell[b, idx[b, rows]].astype(np.float64))[:, None]
        out[b] = (rows, idx[b, rows],
                  X[rows] + (vs * r) * (a.astype(np.float64) + f.astype(np.float64)))
    return out


def gap(model_rows, ref_rows):
    """Largest |model - oracle| and the relative L2 distance over the rows both hold."""
    num = den = 0.0
    worst = 0.0
    for b, (prow, pos, y) in model_rows.items():
        rp, rpos, ry = ref_rows[b]
        assert np.array_equal(prow, rp) and np.array_equal(pos, rpos)
        worst = max(worst, float(np.max(np.abs(y - ry))))
        num += float(np.sum((y - ry) ** 2))
        den += float(np.sum(ry ** 2))
    return worst, (num / den) ** 0.5
