"""Parity of the HIP backward pass against the backward oracle (needs an MI355X).

Bounds are derived from where the kernels round: P and dS enter the matrix cores as bf16
(relative 2^-9 each), D is formed from the bf16 forward output, gradients are stored as bf16
(half an ulp) or fp32, and every sum accumulates in fp32. Each case prints its name before it
touches the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from parity import bf16_vals, dev_bf16, host_bits, say, ulp_bf16

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def x():
    from sparse_depth_token_amd import xmod
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return xmod


def _attn_terms(Q, Kt, Vt, dO, Hq, Hkv, hd):
    """Per head: P, dS and the row sums of |dO||O| that bound the kernels' rounding."""
    m = Q.shape[0]
    vis = np.tril(np.ones((m, m), bool))
    sc = 1 / np.sqrt(hd)
    out = []
    for h in range(Hq):
        g = (h * Hkv) // Hq
        q, kk, vv = (Q[:, h * hd:(h + 1) * hd], Kt[:, g * hd:(g + 1) * hd],
                     Vt[:, g * hd:(g + 1) * hd])
        S = np.where(vis, q @ kk.T * sc, -np.inf)
        P = np.exp(S - S.max(1, keepdims=True))
        P /= P.sum(1, keepdims=True)
        O = P @ vv
        do = dO[:, h * hd:(h + 1) * hd]
        dP = do @ vv.T
        Dq = np.sum(do * O, 1, keepdims=True)
        dS = P * (dP - Dq)
        out.append((g, P, dS, np.sum(np.abs(do) * np.abs(O), 1, keepdims=True)))
    return out


@pytest.mark.parametrize("B,k,Hq,Hkv,hd", [(2, 256, 4, 4, 64), (1, 333, 4, 2, 128),
                                           (3, 200, 8, 2, 64), (2, 512, 16, 16, 128),
                                           (1, 1, 2, 1, 128), (2, 65, 4, 4, 64),
                                           (1, 129, 2, 2, 128), (1, 700, 8, 2, 128),
                                           # more dQ workgroups than CUs: one 256-row q-tile
                                           # per workgroup, ragged last tiles
                                           (1, 600, 96, 8, 64), (2, 300, 96, 12, 128),
                                           # a forward with 128-row key tiles (2048 rows or
                                           # more) hands the backward its normaliser
                                           (1, 2100, 4, 2, 128)])
def test_attention_backward(x, B, k, Hq, Hkv, hd):
    say(f"[attention bwd] B{B} k{k} Hq{Hq} Hkv{Hkv} hd{hd}")
    rng = np.random.default_rng(21)
    dq, dkv = Hq * hd, Hkv * hd
    n = dq + 2 * dkv
    qkv = wl.f32_to_bf16_bits((rng.standard_normal((B * k, n)) * 1.5).astype(np.float32))
    dOb = wl.f32_to_bf16_bits(rng.standard_normal((B * k, dq)).astype(np.float32))
    qkv_d, dO_d = dev_bf16(qkv), dev_bf16(dOb)
    o = torch.empty((B * k, dq), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B * k, Hq), dtype=torch.float32, device="cuda")
    D = torch.empty((B * k, Hq), dtype=torch.float32, device="cuda")
    dqkv = torch.full((B * k, n), float("nan"), dtype=torch.bfloat16, device="cuda")
    x.attention_fwd_lse(qkv_d, o, lse, B, k, Hq, Hkv, hd)
    x.attention_bwd(qkv_d, o, lse, dO_d, D, dqkv, B, k, Hq, Hkv, hd)
    torch.cuda.synchronize()
    got = bf16_vals(host_bits(dqkv))
    lse_g = lse.cpu().numpy().astype(np.float64)
    qv, dov = bf16_vals(qkv), bf16_vals(dOb)
    sc = 1 / np.sqrt(hd)
    for b in range(B):
        rows = slice(b * k, (b + 1) * k)
        Q, Kt, Vt = qv[rows, :dq], qv[rows, dq:dq + dkv], qv[rows, dq + dkv:]
        dO = dov[rows]
        # lse: log2 of sum_j exp(S_j / sqrt(hd)) over the visible keys, by definition
        vis = np.tril(np.ones((k, k), bool))
        for h in range(Hq):
            g = (h * Hkv) // Hq
            S = np.where(vis, Q[:, h * hd:(h + 1) * hd] @ Kt[:, g * hd:(g + 1) * hd].T * sc,
                         -np.inf)
            mx = S.max(1)
            want = (mx + np.log(np.exp(S - mx[:, None]).sum(1))) / np.log(2)
            assert np.allclose(lse_g[rows, h], want, rtol=0, atol=2e-5), f"lse head {h}"
        dQ, dK, dV = oracle.causal_attention_grad(Q, Kt, Vt, np.arange(k), Hq, Hkv, hd, dO)
        # bounds: dS carries P * 2^-8 sum|dO||O| (D from the bf16 O) and 2^-8 |dS| (bf16
        # rounding, with the bf16 P inside dP's partner); P carries 2^-8 P; factor 2 margin
        eQ, eK, eV = np.zeros_like(dQ), np.zeros_like(dK), np.zeros_like(dV)
        for h, (g, P, dS, sdo) in enumerate(_attn_terms(Q, Kt, Vt, dO, Hq, Hkv, hd)):
            e_ds = P * 2.0 ** -8 * sdo + 2.0 ** -8 * np.abs(dS)
            eQ[:, h * hd:(h + 1) * hd] = sc * e_ds @ np.abs(Kt[:, g * hd:(g + 1) * hd])
            eK[:, g * hd:(g + 1) * hd] += sc * e_ds.T @ np.abs(Q[:, h * hd:(h + 1) * hd])
            eV[:, g * hd:(g + 1) * hd] += 2.0 ** -8 * P.T @ np.abs(dO[:, h * hd:(h + 1) * hd])
        for name, gv, ref, e in (("dQ", got[rows, :dq], dQ, eQ),
                                 ("dK", got[rows, dq:dq + dkv], dK, eK),
                                 ("dV", got[rows, dq + dkv:], dV, eV)):
            assert np.all(np.isfinite(gv)), f"{name}: non-finite (unwritten?)"
            err = np.abs(gv - ref)
            bound = 2 * e + 0.5 * ulp_bf16(ref) + 1e-30
            rel = np.linalg.norm(gv - ref) / max(np.linalg.norm(ref), 1e-30)
            say(f"    seq {b} {name}: max|diff| {err.max():.3g}, worst excess "
                f"{(err - bound).max():.3g}, relL2 {rel:.3g}")
            assert np.all(err <= bound), f"seq {b} {name}: worst excess {(err - bound).max():.3g}"


# ---------------------------------------------------------------------------------------------
# the layer: training forward (bit-identical to the forward) and backward against the oracle
# ---------------------------------------------------------------------------------------------

GRAD_NAMES = ("w_router", "g_attn", "w_qkv", "w_o", "g_ffn", "w_gate", "w_up", "w_down")
# Tolerance: gradients pass through at most eight bf16 roundings in
# series (saved activations, activation gradients, P and dS), each relative 2^-9, against two
# for the forward's output; the forward's 5e-3 relative L2 scales to 2e-2, and no element may
# stray further than 5e-2 of the tensor's largest magnitude.
REL_L2, REL_MAX = 2e-2, 5e-2

LAYER_CASES = {
    "tiny K2 B2 T512 d256, gains, biases, varsigma": (wl.scaled(
        wl.WORKLOADS["sparse_k2_b2x512_d256"], seed=31, gain_std=0.1, bias_std=0.1,
        varsigma_range=(0.5, 1.5), router_bias=0.05), 1e-4),
    "ragged B3 T700 K3 (k=233) d512 GQA 4/2 hd128 F1536, routing loss 0.5": (wl.Workload(
        "bw_ragged", 32, 3, 700, 512, 4, 2, 128, 1536, 3, bias_std=0.1, gain_std=0.1,
        varsigma_range=(0.5, 1.5)), 0.5),
    "B2 T1024 K4 d1024 GQA 8/2 hd128 F2816": (wl.Workload(
        "bw_gqa", 33, 2, 1024, 1024, 8, 2, 128, 2816, 4, gain_std=0.1), 1e-4),
    "bench shape B8 T4096 K8 d2048": (wl.WORKLOADS["sparse_k8_b8x4096_d2048"], 1e-4),
    # degenerate cases: one routed token per sequence (62 zero padding rows in the
    # weight-gradient sums), every token routed (no unselected rows), no routing loss
    "k = 1 (B2 T50 K50 d256)": (wl.Workload("bw_k1", 34, 2, 50, 256, 4, 4, 64, 512, 50,
                                             gain_std=0.1, varsigma_range=(0.5, 1.5)), 1e-4),
    "K = 1, every token (B1 T300 d256 GQA 4/2)": (wl.Workload(
        "bw_kall", 35, 1, 300, 256, 4, 2, 64, 512, 1, gain_std=0.1, bias_std=0.1), 1e-4),
    "no routing loss (tiny K2)": (wl.scaled(wl.WORKLOADS["sparse_k2_b2x512_d256"], seed=36,
                                             gain_std=0.1), 0.0),
}


def _dims(x, w):
    return x.make_dims(w.B, w.T, w.d, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden,
                       w.rms_eps)


@pytest.mark.parametrize("case", list(LAYER_CASES))
def test_layer_backward(x, case):
    from parity import compare_selection, layer_to_device
    w, coef = LAYER_CASES[case]
    say(f"[layer bwd] {case}")
    dims = _dims(x, w)
    k = w.k
    xb, lay, bias, dyb = wl.make_x(w), wl.make_layer(w, 0), wl.make_bias(w), wl.make_dy(w)
    L = x.make_layer(layer_to_device(lay))
    # forward: the training form must give the forward's results bit for bit
    xt0 = dev_bf16(xb)
    b0 = torch.from_numpy(bias.copy()).cuda()
    ws_f = x.alloc_workspace(dims, w.K, x.WS_SPARSE_LAYER)
    idx0 = torch.empty((w.B, k), dtype=torch.int32, device="cuda")
    x.sparse_layer_fwd(xt0, L, dims, w.K, b0, w.tau, w.delta, ws_f, idx_out=idx0)
    del ws_f
    xt = dev_bf16(xb)
    bt = torch.from_numpy(bias.copy()).cuda()
    saved = x.alloc_workspace(dims, w.K, x.WS_TRAIN_SAVED)
    idx = torch.empty((w.B, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((w.B, k), dtype=torch.float32, device="cuda")
    x.sparse_layer_fwd_train(xt, L, dims, w.K, bt, w.tau, w.delta, saved, idx_out=idx,
                             gate_out=gate)
    torch.cuda.synchronize()
    assert torch.equal(idx, idx0), "training forward selected differently"
    assert torch.equal(xt.view(torch.int16), xt0.view(torch.int16)), "training forward output differs"
    assert torch.equal(bt, b0), "training forward bias differs"
    # backward, dx in place of dy
    dyt = dev_bf16(dyb)
    grads = x.alloc_grads(dims)
    G = x.make_grads(grads)
    ws = x.alloc_workspace(dims, w.K, x.WS_BACKWARD)
    loss = torch.empty(1, dtype=torch.float32, device="cuda")
    x.sparse_layer_bwd(xt, dyt, dyt, L, dims, w.K, coef, saved, G, ws, loss_route=loss)
    torch.cuda.synchronize()
    idx_g = idx.cpu().numpy().astype(np.int64)
    # oracle on the GPU's selection (allowed only where the oracle's logits nearly tie)
    s_ref, ell_ref = oracle.router_logits(xb, lay["w_router"], lay["router_bias"], bias, w.tau)
    compare_selection(idx_g, oracle.topk_select(ell_ref, k), ell_ref)
    ref = oracle.sparse_layer_grad(xb, lay, w, w.K, dyb, bias=bias, tau=w.tau, route_coef=coef,
                                   forced_idx=idx_g)
    dx = bf16_vals(host_bits(dyt)).reshape(w.B, w.T, w.d)
    sel = np.zeros((w.B, w.T), bool)
    sel[np.arange(w.B)[:, None], idx_g] = True
    # unselected rows: dy plus a router term far below half a bf16 spacing of dy
    got_u, ref_u = dx[~sel], ref["dx"][~sel]
    assert np.all(np.abs(got_u - ref_u) <= 0.5 * ulp_bf16(ref_u) + 1e-6 * np.abs(ref_u) + 1e-12), \
        "unselected rows of dx"

    def close(name, got, want):
        got, want = np.asarray(got, np.float64), np.asarray(want, np.float64)
        assert np.all(np.isfinite(got)), f"{name}: non-finite"
        rel = np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)
        mx = np.abs(got - want).max() / max(np.abs(want).max(), 1e-30)
        say(f"    {name}: relL2 {rel:.3g}, max|diff|/max|ref| {mx:.3g}")
        assert rel <= REL_L2 and mx <= REL_MAX, f"{name}: relL2 {rel:.3g}, max rel {mx:.3g}"

    close("dx (selected rows)", dx[sel], ref["dx"][sel])
    for n in GRAD_NAMES:
        close("d " + n, grads[n].cpu().numpy(), ref["d_" + n])
    for n in ("router_bias", "varsigma"):
        got = float(grads[n].item())
        want = ref["d_" + n]
        say(f"    d {n}: {got:.6g} vs {want:.6g}")
        assert abs(got - want) <= REL_L2 * abs(want) + 1e-9, n
    got_l = float(loss.item())
    say(f"    L_route: {got_l:.7g} vs {ref['loss_route']:.7g}")
    assert abs(got_l - ref["loss_route"]) <= 1e-5 * abs(ref["loss_route"])
