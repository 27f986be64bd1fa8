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
                                           (1, 129, 2, 2, 128), (1, 700, 8, 2, 128)])
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
