"""CPU oracle of the X-MoD layer stack and its closed forms (test infrastructure only).

Sources, cited by page and section / equation:
  [XMOD] "X-MoD: Practical Scaling Laws for Sparse-Depth Routing Beyond Mixture-of-Depths"
         close-reading page: "structural ceiling of the original MoD" (Eqs. (1)-(2)),
         "decoupling K and A" (Eqs. (3)-(5)), "three stabilisers" (Eq. (8) and the bias
         reset at the next dense anchor), "baselines and X-MoD layer constructions"
         (Eqs. (34)-(36)), Table 6 (FLOPs/token convention), "routing diagnostics" (Table 10
         and its two analytic references), "total depth scaling" (Table 9).
"""
from __future__ import annotations

import numpy as np

from .layer import dense_layer, sparse_layer
from .numerics import round_to_bf16


# --- hierarchy: [XMOD] Eq. (3) -----------------------------------------------------------------

def stack_layer_kinds(N0, N1, A, K):
    """Layer list of [Dense] x N0 + ([Sparse(K)] x AK + [Dense]) x N1 as 'D'/'S' characters.

    A*K must be a whole number of sparse layers per block (A may be fractional, e.g. 0.5).
    The original MoD stack of Eq. (1) is the case N0 = 0, A*K = 1.
    """
    ak = A * K
    n_sparse = int(round(ak))
    assert abs(ak - n_sparse) < 1e-9 and n_sparse >= 0, "A*K must be an integer"
    return ["D"] * N0 + (["S"] * n_sparse + ["D"]) * N1


def physical_layers(kinds):
    return len(kinds)


def active_equivalent_layers(kinds, K):
    """Layers a token passes through on average: dense layers count 1, sparse layers 1/K."""
    return sum(1.0 if c == "D" else 1.0 / K for c in kinds)


def total_params(N_layer, kinds):
    """Eq. (4): every physical layer holds N_layer parameters."""
    return N_layer * len(kinds)


def active_params(N_layer, kinds, K):
    """Eq. (5): parameters a token meets on average (sparse layers weigh 1/K)."""
    return N_layer * active_equivalent_layers(kinds, K)


def layer_params(d, n_q_heads, n_kv_heads, head_dim, ffn_hidden):
    """Linear parameters of one layer: Q, K, V and O projections plus a bias-free SwiGLU FFN
    with gate, value and down projections (three d x F matrices)."""
    dq, dkv = n_q_heads * head_dim, n_kv_heads * head_dim
    return d * (dq + 2 * dkv) + dq * d + 3 * d * ffn_hidden


def flops_per_token_pages_convention(N_layer, kinds, K, L, d_q):
    """Counted training FLOPs per token in Table 6's convention.

    Projections and FFN: 2 FLOPs per active parameter. Attention matrix products at full
    length L, non-causal: 4*L*d_q per dense layer, and 1/K^2 of that per sparse layer (1/K of
    the queries see 1/K of the keys).
    """
    n_d = sum(1 for c in kinds if c == "D")
    n_s = sum(1 for c in kinds if c == "S")
    return 2.0 * active_params(N_layer, kinds, K) + 4.0 * L * d_q * (n_d + n_s / K ** 2)


# --- block forward: [XMOD] Eq. (3) with the bias carry of Eq. (8) ------------------------------

def block_forward(x, layers, dims, kinds, K, tau=1.0, delta=0.0, record=False):
    """Walk the stack. Each layer's output is stored back as bf16 (the hidden-state format).

    The carried bias starts at zero, grows by delta for every token a sparse layer selects,
    and is cleared at every dense layer (the anchor reset of the "three stabilisers" section;
    the dense prefix layers clear it too, which changes nothing since it starts at zero).

    layers: list of per-layer weight dicts, one per entry of kinds. Returns the final x
    (float64 values of bf16) and, if record, per-layer inputs/outputs for lock-step checks.
    """
    x = np.asarray(x)
    if x.dtype == np.uint16:
        from .numerics import bf16_to_f64
        x = bf16_to_f64(x)
    B, T, _ = x.shape
    b = np.zeros((B, T), dtype=np.float32)
    trace = []
    for lay, kind in zip(layers, kinds):
        entry = {"kind": kind, "x_in": x, "bias_in": b}
        if kind == "D":
            y = dense_layer(x, lay, dims)
            b = np.zeros((B, T), dtype=np.float32)
        else:
            r = sparse_layer(x, lay, dims, K, bias=b, tau=tau, delta=delta)
            y = r["y"]
            b = r["bias_out"]
            entry.update(idx=r["idx"], ell=r["ell"])
        entry["y"] = y
        x = round_to_bf16(y)
        entry["bias_out"] = b
        if record:
            trace.append(entry)
    return (x, trace) if record else x


# --- routing diagnostics: [XMOD] "routing diagnostics", Table 10 -------------------------------

def coverage(selections, T):
    """Share of tokens selected at least once over a window of consecutive sparse layers.

    selections: list (one per layer) of index arrays for one sequence.
    """
    hit = np.zeros(T, dtype=bool)
    for s in selections:
        hit[np.asarray(s)] = True
    return float(hit.mean())


def adjacent_jaccard(selections):
    """Mean Jaccard index of the selected sets of adjacent layers (pairs with a non-empty union)."""
    vals = []
    for a, b in zip(selections[:-1], selections[1:]):
        sa, sb = set(np.asarray(a).tolist()), set(np.asarray(b).tolist())
        u = len(sa | sb)
        if u:
            vals.append(len(sa & sb) / u)
    return float(np.mean(vals)) if vals else float("nan")


def coverage_independent_reference(p, n_layers):
    """Expected coverage if each of n_layers picks an independent random p-share of tokens."""
    return 1.0 - (1.0 - p) ** n_layers


def jaccard_independent_reference(p):
    """Large-sequence Jaccard of two independent random p-share subsets."""
    return p / (2.0 - p)
