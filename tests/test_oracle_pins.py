"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU needed).

Each test ties an oracle function to something other than the oracle itself: numbers printed
on the pages (tests/golden/, each file cites its table or equation), closed forms, brute force
on tiny inputs written as plain loops, and special cases with a textbook answer.
"""
import itertools
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle.numerics import bf16_to_f64, round_to_bf16
import workload as wl


def _read_table(golden_dir, name):
    rows = []
    with open(os.path.join(golden_dir, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line)
    return rows


class Dims:
    def __init__(self, Hq, Hkv, hd, eps=1e-6):
        self.n_q_heads, self.n_kv_heads, self.head_dim, self.rms_eps = Hq, Hkv, hd, eps


def _rand_layer(rng, d, Hq, Hkv, hd, F, std=0.3, gain=True):
    dq, dkv = Hq * hd, Hkv * hd
    r = lambda *s: wl.f32_to_bf16_bits((rng.standard_normal(s) * std).astype(np.float32))
    g = lambda: wl.f32_to_bf16_bits((1 + 0.2 * rng.standard_normal(d)).astype(np.float32)) if gain \
        else wl.f32_to_bf16_bits(np.ones(d, np.float32))
    return {"w_router": r(d), "w_qkv": r(dq + 2 * dkv, d), "w_o": r(d, dq), "w_gate": r(F, d),
            "w_up": r(F, d), "w_down": r(d, F), "g_attn": g(), "g_ffn": g(),
            "router_bias": 0.0, "varsigma": 1.0}


# ---------------------------------------------------------------------------------------------
# bf16 rounding of the oracle (used by the stack walk) vs torch's fp32 -> bf16 conversion
# ---------------------------------------------------------------------------------------------

def test_round_to_bf16_matches_library_conversion():
    rng = np.random.default_rng(0)
    v = np.concatenate([rng.standard_normal(20000) * s for s in (1e-30, 1e-3, 1.0, 37.0, 1e30)])
    v32 = v.astype(np.float32)
    ref = torch.from_numpy(v32).to(torch.bfloat16).to(torch.float64).numpy()
    got = round_to_bf16(v32.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_to_bf16_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties go to the even mantissa (1.0).
    assert round_to_bf16(np.array([1 + 2.0 ** -8]))[0] == 1.0
    assert round_to_bf16(np.array([1 + 3 * 2.0 ** -8]))[0] == 1 + 2 * 2.0 ** -7
    # just above the halfway point rounds up
    assert round_to_bf16(np.array([1 + 2.0 ** -8 + 2.0 ** -30]))[0] == 1 + 2.0 ** -7


# ---------------------------------------------------------------------------------------------
# router logit and bias adjustment (MoD blog "basic architecture"; X-MoD Eq. (8))
# ---------------------------------------------------------------------------------------------

def test_router_dot_product_exact_sum():
    rng = np.random.default_rng(1)
    x = wl.f32_to_bf16_bits(rng.standard_normal((2, 7, 96)).astype(np.float32))
    w = wl.f32_to_bf16_bits((rng.standard_normal(96) * 0.02).astype(np.float32))
    s, ell = oracle.router_logits(x, w, 0.25, None, 1.0)
    xf, wf = bf16_to_f64(x), bf16_to_f64(w)
    for b in range(2):
        for t in range(7):
            exact = math.fsum([float(xf[b, t, c]) * float(wf[c]) for c in range(96)] + [0.25])
            assert s[b, t] == np.float32(exact)
    assert np.array_equal(s, ell)        # zero bias: ell == s


def test_router_bias_subtracts_tau_b():
    # w_r = 0: every logit is beta - tau*b, computed in fp32 (product rounded, then difference)
    x = wl.f32_to_bf16_bits(np.ones((1, 4, 8), np.float32))
    w = wl.f32_to_bf16_bits(np.zeros(8, np.float32))
    b = np.array([[0.0, 0.05, 0.1, -0.3]], np.float32)
    s, ell = oracle.router_logits(x, w, 1.5, b, 2.0)
    assert np.all(s == np.float32(1.5))
    want = np.array([1.5, 1.4, 1.3, 2.1], np.float32)
    assert np.allclose(ell, want, atol=1e-6)
    assert ell[0, 3] > ell[0, 0] > ell[0, 1] > ell[0, 2]   # a larger bias lowers the logit


# ---------------------------------------------------------------------------------------------
# top-k selection: brute force over all subsets, ties, +-0
# ---------------------------------------------------------------------------------------------

def _brute_topk(ell, k):
    """The unique k-subset S with: for i in S, j not in S, ell_i > ell_j or (== and i < j)."""
    T = len(ell)
    found = []
    for S in itertools.combinations(range(T), k):
        Sset = set(S)
        ok = all((ell[i] > ell[j]) or (ell[i] == ell[j] and i < j)
                 for i in S for j in range(T) if j not in Sset)
        if ok:
            found.append(list(S))
    assert len(found) == 1
    return found[0]


@pytest.mark.parametrize("levels", [None, 3, 2])
def test_topk_brute_force(levels):
    rng = np.random.default_rng(2 + (levels or 0))
    for trial in range(40):
        T = int(rng.integers(1, 13))
        k = int(rng.integers(1, T + 1))
        if levels is None:
            ell = rng.standard_normal(T).astype(np.float32)
        else:
            ell = rng.integers(0, levels, T).astype(np.float32) - 1.0
            ell[rng.random(T) < 0.3] = -0.0      # mix -0 and +0 (equal by value)
        got = oracle.topk_select(ell[None, :], k)[0].tolist()
        assert got == _brute_topk([float(v) for v in ell], k)


def test_topk_special_cases():
    e = np.full((2, 9), 0.5, np.float32)
    assert oracle.topk_select(e, 4).tolist() == [[0, 1, 2, 3]] * 2     # all equal: lowest positions
    r = np.random.default_rng(3).standard_normal((3, 11)).astype(np.float32)
    assert oracle.topk_select(r, 11).tolist() == [list(range(11))] * 3  # k = T: everything
    z = np.array([[0.0, -0.0, -0.0, 0.0]], np.float32)
    assert oracle.topk_select(z, 2).tolist() == [[0, 1]]                 # -0 == +0


def test_topk_counts_and_order_large():
    # check (2): exactly k per sequence, strictly increasing, unique, in range
    ell = np.random.default_rng(4).standard_normal((5, 1000)).astype(np.float32)
    idx = oracle.topk_select(ell, 125)
    assert idx.shape == (5, 125)
    assert np.all(np.diff(idx, axis=1) > 0) and idx.min() >= 0 and idx.max() < 1000
    for b in range(5):
        thr = np.sort(ell[b])[::-1][124]
        assert np.all(ell[b, idx[b]] >= thr)


# ---------------------------------------------------------------------------------------------
# RMSNorm, SiLU, SwiGLU: textbook special cases
# ---------------------------------------------------------------------------------------------

def test_rmsnorm_special_cases():
    c = 3.0
    u = oracle.rmsnorm(np.full((1, 16), c), np.ones(16), 1e-6)
    assert np.allclose(u, c / math.sqrt(c * c + 1e-6), rtol=1e-15)
    X = np.random.default_rng(5).standard_normal((4, 64))
    u = oracle.rmsnorm(X, np.ones(64), 0.0)
    assert np.allclose(np.mean(u * u, axis=1), 1.0, rtol=1e-13)         # unit RMS
    assert np.allclose(oracle.rmsnorm(7.0 * X, np.ones(64), 0.0), u)    # scale invariance
    g = np.random.default_rng(6).standard_normal(64)
    assert np.allclose(oracle.rmsnorm(X, g, 0.0), u * g)                # gain is per channel


def test_silu_and_swiglu():
    assert oracle.silu(0.0) == 0.0
    assert abs(oracle.silu(1.0) - 1.0 / (1.0 + math.exp(-1.0))) < 1e-16
    assert abs(oracle.silu(-40.0)) < 1e-15 and abs(oracle.silu(40.0) - 40.0) < 1e-12
    rng = np.random.default_rng(7)
    v = rng.standard_normal((3, 8))
    wg, wd = rng.standard_normal((5, 8)), rng.standard_normal((8, 5))
    assert np.all(oracle.swiglu_ffn(v, wg, np.zeros((5, 8)), wd) == 0.0)  # value proj 0 -> f = 0
    # one hidden unit, explicit scalar form
    wg1, wu1, wd1 = rng.standard_normal((1, 8)), rng.standard_normal((1, 8)), rng.standard_normal((8, 1))
    f = oracle.swiglu_ffn(v, wg1, wu1, wd1)
    for r in range(3):
        zg = sum(v[r, c] * wg1[0, c] for c in range(8))
        zu = sum(v[r, c] * wu1[0, c] for c in range(8))
        hid = zg / (1 + math.exp(-zg)) * zu
        assert np.allclose(f[r], [hid * wd1[c, 0] for c in range(8)], rtol=1e-12)


# ---------------------------------------------------------------------------------------------
# causal attention: loop brute force, GQA mapping of the MoDA notes (1-based ceil(h/G))
# ---------------------------------------------------------------------------------------------

def _brute_attention(Q, Kt, Vt, q_pos, Hq, Hkv, hd):
    G = Hq // Hkv
    out = np.zeros((Q.shape[0], Hq * hd))
    for i in range(Q.shape[0]):
        for h1 in range(1, Hq + 1):                      # 1-based head index
            g1 = math.ceil(h1 / G)                       # 1-based KV head
            qs = Q[i, (h1 - 1) * hd:h1 * hd]
            scores = []
            for j in range(q_pos[i] + 1):
                kj = Kt[j, (g1 - 1) * hd:g1 * hd]
                scores.append(sum(qs[c] * kj[c] for c in range(hd)) / math.sqrt(hd))
            mx = max(scores)
            wts = [math.exp(s - mx) for s in scores]
            z = sum(wts)
            for c in range(hd):
                out[i, (h1 - 1) * hd + c] = sum(wts[j] * Vt[j, (g1 - 1) * hd + c] for j in range(len(wts))) / z
    return out


@pytest.mark.parametrize("Hq,Hkv", [(4, 4), (4, 2), (6, 2), (4, 1)])
def test_attention_brute_force(Hq, Hkv):
    rng = np.random.default_rng(8 + Hq + Hkv)
    m, hd = 9, 4
    Kt, Vt = rng.standard_normal((m, Hkv * hd)), rng.standard_normal((m, Hkv * hd))
    q_pos = np.array([0, 3, 4, 8])
    Q = rng.standard_normal((4, Hq * hd)) * 2
    got = oracle.causal_attention(Q, Kt, Vt, q_pos, Hq, Hkv, hd)
    assert np.allclose(got, _brute_attention(Q, Kt, Vt, q_pos, Hq, Hkv, hd), rtol=1e-12, atol=1e-13)


def test_attention_closed_forms():
    rng = np.random.default_rng(9)
    Kt, Vt = rng.standard_normal((6, 8)), rng.standard_normal((6, 8))
    # first position sees only itself: O = V_0
    O = oracle.causal_attention(rng.standard_normal((1, 8)), Kt, Vt, np.array([0]), 2, 2, 4)
    assert np.allclose(O, Vt[0:1], rtol=1e-15)
    # Q = 0: uniform weights, O_i = mean of V_0..V_i
    O = oracle.causal_attention(np.zeros((6, 8)), Kt, Vt, np.arange(6), 2, 2, 4)
    for i in range(6):
        assert np.allclose(O[i], Vt[:i + 1].mean(axis=0), rtol=1e-14)


# ---------------------------------------------------------------------------------------------
# the sparse layer: brute-force loop implementation on tiny shapes, and checks (1)-(4)
# ---------------------------------------------------------------------------------------------

def _brute_sparse_layer(x, lay, Hq, Hkv, hd, eps, K, bias, tau, delta, threshold=False):
    # layer-form options, written out as loops: per-head RMSNorm of q / k, rotary embedding at
    # the original position (rotate-half pairs), MoD's Eq. (6) residual
    """Plain-loop X-MoD layer written from the pages' steps, for tiny shapes only.

    threshold=True takes the eval-time rule instead of top-k: a token enters when its routing
    probability 1 / (1 + exp(-logit)) is at least 1/2 (evaluated here as written, in float64)."""
    B, T, d = x.shape
    k = T // K
    f64 = lambda a: bf16_to_f64(a) if np.asarray(a).dtype == np.uint16 else np.asarray(a, float)
    wr, wqkv, wo = f64(lay["w_router"]), f64(lay["w_qkv"]), f64(lay["w_o"])
    wg, wu, wd = f64(lay["w_gate"]), f64(lay["w_up"]), f64(lay["w_down"])
    g1, g2 = f64(lay["g_attn"]), f64(lay["g_ffn"])
    F = wg.shape[0]
    dq, dkv = Hq * hd, Hkv * hd
    y = x.copy()
    b_out = bias.copy()

    def norm(vec, g):
        r = math.sqrt(sum(v * v for v in vec) / len(vec) + eps)
        return [vec[c] / r * g[c] for c in range(len(vec))]

    def matvec(Wm, vec, rows):
        return [sum(Wm[r, c] * vec[c] for c in range(len(vec))) for r in rows]

    for b in range(B):
        logit = []
        for t in range(T):
            s = np.float32(math.fsum([x[b, t, c] * wr[c] for c in range(d)]) + lay["router_bias"])
            logit.append(np.float32(s - np.float32(np.float32(tau) * bias[b, t])))
        if threshold:
            S = [t for t in range(T) if 1.0 / (1.0 + math.exp(-float(logit[t]))) >= 0.5]
        else:
            ranked = sorted(range(T), key=lambda t: (-float(logit[t]), t))
            S = sorted(ranked[:k])
        u = [norm(list(x[b, t]), g1) for t in S]
        q = [matvec(wqkv, uu, range(0, dq)) for uu in u]
        kk = [matvec(wqkv, uu, range(dq, dq + dkv)) for uu in u]
        vv = [matvec(wqkv, uu, range(dq + dkv, dq + 2 * dkv)) for uu in u]

        def head_form(vec, n_heads, gain, pos):
            out = list(vec)
            for hh in range(n_heads):
                seg = out[hh * hd:(hh + 1) * hd]
                if gain is not None:
                    seg = norm(seg, f64(gain))
                theta = lay.get("rope_theta", 0.0)
                if theta:
                    half = hd // 2
                    rot = list(seg)
                    for i in range(half):
                        ang = pos * theta ** (-2.0 * i / hd)
                        rot[i] = seg[i] * math.cos(ang) - seg[i + half] * math.sin(ang)
                        rot[i + half] = seg[i + half] * math.cos(ang) + seg[i] * math.sin(ang)
                    seg = rot
                out[hh * hd:(hh + 1) * hd] = seg
            return out
        q = [head_form(q[i], Hq, lay.get("q_norm"), S[i]) for i in range(len(S))]
        kk = [head_form(kk[i], Hkv, lay.get("k_norm"), S[i]) for i in range(len(S))]
        G = Hq // Hkv
        for i, t in enumerate(S):
            o = []
            for h in range(Hq):
                g = h // G
                sc = [sum(q[i][h * hd + c] * kk[j][g * hd + c] for c in range(hd)) / math.sqrt(hd)
                      for j in range(i + 1)]
                mx = max(sc)
                w = [math.exp(s - mx) for s in sc]
                o += [sum(w[j] * vv[j][g * hd + c] for j in range(i + 1)) / sum(w) for c in range(hd)]
            a = matvec(wo, o, range(d))
            hres = [x[b, t, c] + a[c] for c in range(d)]
            v = norm(hres, g2)
            gate_pre = matvec(wg, v, range(F))
            up = matvec(wu, v, range(F))
            hid = [gate_pre[n] / (1 + math.exp(-gate_pre[n])) * up[n] for n in range(F)]
            f = matvec(wd, hid, range(d))
            r = 1.0 / (1.0 + math.exp(-float(logit[t])))
            for c in range(d):
                if lay.get("residual", 0) == 1:
                    y[b, t, c] = x[b, t, c] + a[c] + r * f[c]
                else:
                    y[b, t, c] = x[b, t, c] + lay["varsigma"] * r * (a[c] + f[c])
            b_out[b, t] = np.float32(bias[b, t] + np.float32(delta))
    return y, b_out


@pytest.mark.parametrize("Hq,Hkv,K", [(2, 2, 2), (4, 2, 3), (2, 1, 1)])
def test_sparse_layer_brute_force(Hq, Hkv, K):
    rng = np.random.default_rng(10 + Hq + K)
    B, T, d, hd, F = 2, 7, 8, 2, 6
    lay = _rand_layer(rng, d, Hq, Hkv, hd, F)
    lay["router_bias"] = 0.3
    lay["varsigma"] = 0.8
    x = bf16_to_f64(wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32)))
    bias = (rng.standard_normal((B, T)) * 0.2).astype(np.float32)
    dims = Dims(Hq, Hkv, hd, 1e-5)
    got = oracle.sparse_layer(x, lay, dims, K, bias=bias, tau=1.5, delta=0.05)
    want_y, want_b = _brute_sparse_layer(x, lay, Hq, Hkv, hd, 1e-5, K, bias, 1.5, 0.05)
    assert np.allclose(got["y"], want_y, rtol=1e-11, atol=1e-12)
    assert np.array_equal(got["bias_out"], want_b)


def _tiny(seed=11, B=2, T=24, d=16, Hq=4, Hkv=2, hd=4, F=24):
    rng = np.random.default_rng(seed)
    lay = _rand_layer(rng, d, Hq, Hkv, hd, F, std=0.25)
    x = bf16_to_f64(wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32)))
    return x, lay, Dims(Hq, Hkv, hd)


def test_check1_k1_unit_gate_equals_dense_layer():
    # K = 1, varsigma = 1 and r = 1 (w_r = 0, beta = 100: sigmoid(100) == 1.0 in float64)
    x, lay, dims = _tiny()
    lay["w_router"] = wl.f32_to_bf16_bits(np.zeros(16, np.float32))
    lay["router_bias"] = 100.0
    assert oracle.sigmoid(np.float32(100.0)) == 1.0
    ys = oracle.sparse_layer(x, lay, dims, 1)["y"]
    yd = oracle.dense_layer(x, lay, dims)
    assert np.allclose(ys, yd, rtol=1e-13, atol=1e-13)


def test_k1_general_gate_is_dense_residual_scaled():
    # K = 1 with any gate: y = x + varsigma*r*(dense(x) - x)
    x, lay, dims = _tiny(seed=12)
    lay["varsigma"] = 0.7
    r = oracle.sparse_layer(x, lay, dims, 1)
    yd = oracle.dense_layer(x, lay, dims)
    want = x + 0.7 * r["gate"][:, :, None] * (yd - x)
    assert np.allclose(r["y"], want, rtol=1e-12, atol=1e-12)


def test_sparse_equals_dense_on_packed_subsequence():
    # Attention and FFN act on the selected rows as if they were a sequence of their own.
    x, lay, dims = _tiny(seed=13, T=40)
    lay["varsigma"] = 1.3
    r = oracle.sparse_layer(x, lay, dims, 4)
    for b in range(x.shape[0]):
        S = r["idx"][b]
        sub = x[b][S][None]                                   # [1, k, d]
        dsub = oracle.dense_layer(sub, lay, dims)[0]
        want = sub[0] + 1.3 * r["gate"][b][:, None] * (dsub - sub[0])
        assert np.allclose(r["y"][b, S], want, rtol=1e-12, atol=1e-12)


def test_checks_2_3_4_and_varsigma_linearity():
    x, lay, dims = _tiny(seed=14, T=33)
    bias = (np.random.default_rng(15).standard_normal((2, 33)) * 0.1).astype(np.float32)
    r1 = oracle.sparse_layer(x, lay, dims, 4, bias=bias, delta=0.05)
    k = 33 // 4
    idx = r1["idx"]
    # (2) exactly k per sequence, ascending, unique
    assert idx.shape == (2, k) and np.all(np.diff(idx, axis=1) > 0)
    # (3) unselected rows bit-identical
    mask = np.zeros((2, 33), bool)
    mask[np.arange(2)[:, None], idx] = True
    assert np.array_equal(r1["y"][~mask], x[~mask])
    # bias: +delta exactly on the selected tokens, untouched elsewhere
    assert np.array_equal(r1["bias_out"][mask], (bias[mask] + np.float32(0.05)).astype(np.float32))
    assert np.array_equal(r1["bias_out"][~mask], bias[~mask])
    # (4) varsigma = 0 is the identity
    lay0 = dict(lay, varsigma=0.0)
    assert np.array_equal(oracle.sparse_layer(x, lay0, dims, 4, bias=bias)["y"], x)
    # linearity in varsigma
    lay2 = dict(lay, varsigma=2.5)
    r2 = oracle.sparse_layer(x, lay2, dims, 4, bias=bias)
    assert np.allclose(r2["y"] - x, 2.5 * (r1["y"] - x), rtol=1e-12, atol=1e-13)


def test_gate_uses_pre_update_bias_and_sampling_matches_full():
    x, lay, dims = _tiny(seed=16, T=48)
    bias = (np.random.default_rng(17).standard_normal((2, 48)) * 0.5).astype(np.float32)
    r = oracle.sparse_layer(x, lay, dims, 3, bias=bias, tau=1.0, delta=0.05)
    ell_sel = r["ell"][np.arange(2)[:, None], r["idx"]]
    assert np.array_equal(r["gate"], oracle.sigmoid(ell_sel))
    sample = {1: np.array([0, 5, 15])}
    rs = oracle.sparse_layer(x, lay, dims, 3, bias=bias, sample=sample)
    rows, pos, ysel = rs["rows"][1]
    assert np.array_equal(pos, r["idx"][1, rows])
    assert np.allclose(ysel, r["y"][1, pos], rtol=1e-13, atol=1e-14)
    ds = oracle.dense_layer(x, lay, dims, sample={0: np.array([3, 47])})
    assert np.allclose(ds[0][1], oracle.dense_layer(x, lay, dims)[0, [3, 47]], rtol=1e-13)


# ---------------------------------------------------------------------------------------------
# stack: layer counts, parameters, FLOPs convention, Eq. (2) ratio (printed numbers)
# ---------------------------------------------------------------------------------------------

def _kinds_from_segments(seg_text):
    kinds, K = [], None
    for seg in seg_text.split(";"):
        N0, N1, A, K = seg.split(",")
        kinds += oracle.stack_layer_kinds(int(N0), int(N1), float(A), int(K))
    return kinds, int(K)


def test_layer_constructions_printed(golden_dir):
    for row in _read_table(golden_dir, "layer_constructions.txt"):
        name, segs, phys, act = [c.strip() for c in row.split("|")]
        kinds, K = _kinds_from_segments(segs)
        assert oracle.physical_layers(kinds) == int(phys), name
        assert oracle.active_equivalent_layers(kinds, K) == pytest.approx(float(act), abs=1e-12), name


def test_mod_ratio_eq2(golden_dir):
    K, num, den, printed = _read_table(golden_dir, "mod_ratio.txt")[0].split()
    kinds = oracle.stack_layer_kinds(0, 100, 1.0 / int(K), int(K))     # ([Sparse]+[Dense]) x N
    ratio = oracle.total_params(1, kinds) / oracle.active_params(1, kinds, int(K))
    assert ratio == pytest.approx(int(num) / int(den), rel=1e-12)
    assert round(ratio, 2) == float(printed)
    for Kx in (2, 4, 64, 1024):                                           # always below 2
        kk = oracle.stack_layer_kinds(0, 3, 1.0 / Kx, Kx)
        assert oracle.total_params(1, kk) / oracle.active_params(1, kk, Kx) < 2


def _backbones(golden_dir):
    out = {}
    for row in _read_table(golden_dir, "backbones.txt"):
        lab, d, hd, L, H, Hkv, F = row.split()
        out[lab] = dict(d=int(d), hd=int(hd), H=int(H), Hkv=int(Hkv), F=int(F))
    return out


_MODEL_SEGMENTS = {"Dense": ("0,0,0,8 ; 28,0,0,8", 8), "MoD": ("1,0,0,8 ; 0,24,0.125,8", 8),
                   "A4K8": ("4,0,0,8 ; 0,1,3,8 ; 0,4,4,8", 8), "A3K16": ("4,6,3,16", 16)}


def test_param_totals_and_flops_table6(golden_dir):
    bb = _backbones(golden_dir)
    for row in _read_table(golden_dir, "table6_totals_flops.txt"):
        scale, model, layers, n_printed, fl_printed, note = row.split()
        c = bb[scale]
        Nl = oracle.layer_params(c["d"], c["H"], c["Hkv"], c["hd"], c["F"])
        kinds, K = _kinds_from_segments(_MODEL_SEGMENTS[model][0])
        assert oracle.physical_layers(kinds) == int(layers)
        assert oracle.active_equivalent_layers(kinds, K) == pytest.approx(28.0)
        total = oracle.total_params(Nl, kinds) + 2 * 50257 * c["d"]
        if note == "ok":
            digits = len(n_printed.split(".")[1])
            assert round(total / 1e9, digits) == pytest.approx(float(n_printed)), (scale, model)
        else:
            assert round(total / 1e9, 2) != float(n_printed)          # documented mismatch
        fl = oracle.flops_per_token_pages_convention(Nl, kinds, K, 32768, c["H"] * c["hd"])
        printed = float(fl_printed) if "e" in fl_printed else float(fl_printed) * 1e9
        assert float(f"{fl:.1e}") == pytest.approx(printed), (scale, model)   # 2 significant figures


def test_attention_share_eq40(golden_dir):
    layers = {"A4K8": ("0,9,0,8", "0,1,19,8", 8), "A3K16": ("0,10,0,16", "0,1,18,16", 16),
              "MoD": ("0,25,0,8", "0,1,3,8", 8)}
    for row in _read_table(golden_dir, "mechanism_attention_ratio.txt"):
        model, printed = row.split()
        dense = int(layers[model][0].split(",")[1])
        n_sparse = {"A4K8": 152, "A3K16": 288, "MoD": 24}[model]
        K = layers[model][2]
        kinds = ["D"] * dense + ["S"] * n_sparse
        # attention term of the FLOPs convention, relative to 28 dense layers
        att = oracle.flops_per_token_pages_convention(0, kinds, K, 1, 1)
        att_dense = oracle.flops_per_token_pages_convention(0, ["D"] * 28, K, 1, 1)
        assert round(att / att_dense, 3) == float(printed)


# ---------------------------------------------------------------------------------------------
# routing diagnostics (Table 10) and the bias carry of the block walk
# ---------------------------------------------------------------------------------------------

def test_routing_reference_columns(golden_dir):
    for row in _read_table(golden_dir, "routing_references.txt"):
        m, K, n, rc, rj, ic, ij = row.split()
        K, n = int(K), int(n)
        p = 1.0 / K
        assert round(100 * oracle.coverage_independent_reference(p, n), 2) == float(ic)
        assert round(100 * oracle.jaccard_independent_reference(p), 3) == float(ij)
        # "repeat the same subset": measured with the diagnostics on an explicit selection
        T = 4096
        sel = [np.arange(0, T, K)] * n
        assert round(100 * oracle.coverage(sel, T), 3) == pytest.approx(float(rc))
        assert 100 * oracle.adjacent_jaccard(sel) == float(rj)
        # independent random subsets: the diagnostics land on the printed references
        rng = np.random.default_rng(K * 1000 + n)
        T = 32768
        sel = [np.sort(rng.permutation(T)[:T // K]) for _ in range(n)]
        assert 100 * oracle.coverage(sel, T) == pytest.approx(float(ic), abs=0.8)
        assert 100 * oracle.adjacent_jaccard(sel) == pytest.approx(float(ij), abs=0.15)


def _shared_router_stack(K, AK, varsigma, delta, seed=20, B=2, T=32, d=16):
    rng = np.random.default_rng(seed)
    base = _rand_layer(rng, d, 2, 2, 4, 16, std=0.3)
    layers = []
    for kind in ["S"] * AK + ["D"]:
        lay = dict(base)
        lay["varsigma"] = varsigma
        layers.append(lay)
    x = wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32))
    return x, layers, Dims(2, 2, 4)


def test_bias_carry_rotation_covers_every_token_once():
    # Shared router weights, varsigma = 0 (x frozen), delta far above the logit range: the
    # carried bias makes consecutive sparse layers rotate through the tokens, each chosen once
    # per K layers (coverage 100 %, adjacent Jaccard 0).
    K, AK = 4, 8
    x, layers, dims = _shared_router_stack(K, AK, 0.0, 1000.0)
    kinds = oracle.stack_layer_kinds(0, 1, AK / K, K)
    _, trace = oracle.block_forward(x, layers, dims, kinds, K, tau=1.0, delta=1000.0, record=True)
    sparse = [e for e in trace if e["kind"] == "S"]
    for b in range(2):
        sels = [e["idx"][b] for e in sparse]
        for start in range(0, AK, K):
            window = np.concatenate(sels[start:start + K])
            assert np.array_equal(np.sort(window), np.arange(32))
        assert oracle.adjacent_jaccard(sels) == 0.0
    # the anchor clears the bias
    assert np.all(trace[-1]["bias_out"] == 0)
    assert np.all(sparse[-1]["bias_out"] == np.float32(2000.0))


def test_bias_off_repeats_the_same_subset():
    K, AK = 4, 6
    x, layers, dims = _shared_router_stack(K, AK, 0.0, 0.0)
    kinds = oracle.stack_layer_kinds(0, 1, AK / K, K)
    _, trace = oracle.block_forward(x, layers, dims, kinds, K, delta=0.0, record=True)
    sels = [e["idx"][0] for e in trace if e["kind"] == "S"]
    assert oracle.coverage(sels, 32) == 1.0 / K
    assert oracle.adjacent_jaccard(sels) == 1.0


def test_block_walk_rounds_to_bf16_and_resets_bias():
    rng = np.random.default_rng(21)
    d = 16
    layers = [_rand_layer(rng, d, 2, 2, 4, 16) for _ in range(5)]
    x = wl.f32_to_bf16_bits(rng.standard_normal((2, 24, d)).astype(np.float32))
    dims = Dims(2, 2, 4)
    kinds = oracle.stack_layer_kinds(1, 2, 0.5, 2)        # D, S, D, S, D
    assert kinds == ["D", "S", "D", "S", "D"]
    xf, trace = oracle.block_forward(x, layers, dims, kinds, 2, delta=0.05, record=True)
    # manual walk
    cur = bf16_to_f64(x)
    b = np.zeros((2, 24), np.float32)
    for lay, kind, e in zip(layers, kinds, trace):
        assert np.array_equal(e["x_in"], cur)
        if kind == "D":
            y = oracle.dense_layer(cur, lay, dims)
            b = np.zeros_like(b)
        else:
            r = oracle.sparse_layer(cur, lay, dims, 2, bias=b, delta=0.05)
            y, b = r["y"], r["bias_out"]
        cur = round_to_bf16(y)
    assert np.array_equal(xf, cur)


# ---------------------------------------------------------------------------------------------
# eval-time causal threshold routing and the mask agreement of Table 10
# ---------------------------------------------------------------------------------------------

def test_threshold_select_definition():
    ell = np.array([[-1.0, 0.0, -0.0, 2.0, -1e-30, 1e-30, -3.5, 0.25]], dtype=np.float32)
    assert oracle.threshold_select(ell)[0].tolist() == [1, 2, 3, 5, 7]
    # away from 0, the rule is sigmoid >= 1/2 evaluated as written
    rng = np.random.default_rng(40)
    ell = (rng.standard_normal((3, 500)) * 2).astype(np.float32)
    ell[np.abs(ell) < 1e-6] = 1.0
    sel = oracle.threshold_select(ell)
    for b in range(3):
        want = [t for t in range(500) if 1.0 / (1.0 + math.exp(-float(ell[b, t]))) >= 0.5]
        assert sel[b].tolist() == want


@pytest.mark.parametrize("Hq,Hkv,shift", [(2, 2, 0.0), (4, 2, 0.4), (2, 1, -0.6)])
def test_sparse_layer_threshold_brute_force(Hq, Hkv, shift):
    rng = np.random.default_rng(50 + Hq)
    B, T, d, hd, F = 3, 7, 8, 2, 6
    lay = _rand_layer(rng, d, Hq, Hkv, hd, F)
    lay["router_bias"] = shift
    lay["varsigma"] = 0.7
    x = bf16_to_f64(wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32)))
    bias = (rng.standard_normal((B, T)) * 0.3).astype(np.float32)
    dims = Dims(Hq, Hkv, hd, 1e-5)
    got = oracle.sparse_layer_threshold(x, lay, dims, bias=bias, tau=1.2, delta=0.05)
    want_y, want_b = _brute_sparse_layer(x, lay, Hq, Hkv, hd, 1e-5, 1, bias, 1.2, 0.05,
                                         threshold=True)
    assert got["counts"].sum() > 0
    assert np.allclose(got["y"], want_y, rtol=1e-11, atol=1e-12)
    assert np.array_equal(got["bias_out"], want_b)


def test_threshold_extremes():
    x, lay, dims = _tiny(seed=41)
    bias = (np.random.default_rng(42).standard_normal(x.shape[:2]) * 0.1).astype(np.float32)
    lay_all = dict(lay, router_bias=100.0)          # every ell >= 0: all tokens, like K = 1
    r = oracle.sparse_layer_threshold(x, lay_all, dims, bias=bias, delta=0.05)
    r1 = oracle.sparse_layer(x, lay_all, dims, 1, bias=bias, delta=0.05)
    assert np.array_equal(r["counts"], np.full(x.shape[0], x.shape[1]))
    assert np.array_equal(r["y"], r1["y"]) and np.array_equal(r["bias_out"], r1["bias_out"])
    lay_none = dict(lay, router_bias=-100.0)        # no token enters: identity, bias unchanged
    r = oracle.sparse_layer_threshold(x, lay_none, dims, bias=bias, delta=0.05)
    assert np.all(r["counts"] == 0)
    assert np.array_equal(r["y"], x) and np.array_equal(r["bias_out"], bias)


def test_threshold_sampling_matches_full():
    x, lay, dims = _tiny(seed=43, T=40)
    r = oracle.sparse_layer_threshold(x, lay, dims)
    assert np.all(r["counts"] > 3)
    sample = {b: np.array([0, 2, int(r["counts"][b]) - 1]) for b in range(x.shape[0])}
    rs = oracle.sparse_layer_threshold(x, lay, dims, sample=sample)
    for b, (prow, pos, ysel) in rs["rows"].items():
        assert np.array_equal(pos, r["idx"][b][prow])
        assert np.array_equal(ysel, r["y"][b, pos])


def test_mask_agreement_counts():
    rng = np.random.default_rng(44)
    B, T, k = 4, 64, 8
    ell = (rng.standard_normal((B, T)) - 1.0).astype(np.float32)
    idx = oracle.topk_select(ell, k)
    agree, n = oracle.mask_agreement(ell, idx)
    # symmetric difference of the two position sets, counted by hand
    diff = 0
    for b in range(B):
        a = set(idx[b].tolist())
        t = {i for i in range(T) if ell[b, i] >= 0}
        diff += len(a ^ t)
    assert n == B * T and agree == B * T - diff
    # when exactly the top-k logits are non-negative, the two masks coincide
    ell2 = ell.copy()
    for b in range(B):
        ell2[b] = -1.0
        ell2[b, idx[b]] = 1.0
    assert oracle.mask_agreement(ell2, idx) == (B * T, B * T)


def test_mask_agreement_reading_table10(golden_dir):
    for line in _read_table(golden_dir, "mask_agreement.txt"):
        _, K, agree, share = line.split()
        got = 100.0 * oracle.differing_selected_share(float(agree) / 100.0, int(K))
        assert round(got) == int(share), (line, got)


# ---------------------------------------------------------------------------------------------
# layer-form options: QK-norm, rotary embedding at original positions, MoD's Eq. (6) residual
# ---------------------------------------------------------------------------------------------

def test_rope_rotation_and_relative_positions():
    rng = np.random.default_rng(90)
    z = rng.standard_normal((5, 2))
    pos = np.array([0, 1, 2, 7, 100])
    got = oracle.rope(z, pos, 1, 2, 10000.0)          # head_dim 2: one pair, angle = position
    for i, p_ in enumerate(pos):
        R = np.array([[math.cos(p_), -math.sin(p_)], [math.sin(p_), math.cos(p_)]])
        assert np.allclose(got[i], R @ z[i], rtol=1e-13, atol=1e-13)
    Hh, hd = 3, 8
    q = rng.standard_normal((1, Hh * hd))
    k = rng.standard_normal((1, Hh * hd))
    assert np.array_equal(oracle.rope(q, [0], Hh, hd, 500.0), q)           # position 0: identity
    for theta in (10000.0, 1e6):
        for (m, n, c) in [(5, 2, 11), (40, 40, 3), (3, 17, 250)]:
            d1 = oracle.rope(q, [m], Hh, hd, theta) * oracle.rope(k, [n], Hh, hd, theta)
            d2 = oracle.rope(q, [m + c], Hh, hd, theta) * oracle.rope(k, [n + c], Hh, hd, theta)
            for hh in range(Hh):                       # per-head scores depend on m - n only
                s1 = d1[0, hh * hd:(hh + 1) * hd].sum()
                s2 = d2[0, hh * hd:(hh + 1) * hd].sum()
                assert abs(s1 - s2) < 1e-11
        r = oracle.rope(q, [123], Hh, hd, theta).reshape(Hh, 2, hd // 2)
        q3 = q.reshape(Hh, 2, hd // 2)
        assert np.allclose((r ** 2).sum(axis=1), (q3 ** 2).sum(axis=1))    # pairs keep their norm


def test_qk_head_norm():
    rng = np.random.default_rng(91)
    Z = rng.standard_normal((4, 3 * 16)) * 5
    ones = wl.f32_to_bf16_bits(np.ones(16, np.float32))
    out = oracle.qk_head_norm(Z, 3, 16, ones, 0.0).reshape(4, 3, 16)
    assert np.allclose(np.mean(out ** 2, axis=-1), 1.0)
    assert np.allclose(oracle.qk_head_norm(7.0 * Z, 3, 16, ones, 0.0), oracle.qk_head_norm(Z, 3, 16, ones, 0.0))


@pytest.mark.parametrize("form", ["qknorm+rope", "rope", "mod"])
def test_sparse_layer_options_brute_force(form):
    rng = np.random.default_rng(92 + len(form))
    B, T, d, Hq, Hkv, hd, F, K = 2, 9, 8, 2, 1, 4, 6, 2
    lay = _rand_layer(rng, d, Hq, Hkv, hd, F)
    lay["router_bias"] = 0.1
    lay["varsigma"] = 0.9
    if "qknorm" in form:
        lay["q_norm"] = wl.f32_to_bf16_bits((1 + 0.3 * rng.standard_normal(hd)).astype(np.float32))
        lay["k_norm"] = wl.f32_to_bf16_bits((1 + 0.3 * rng.standard_normal(hd)).astype(np.float32))
    if "rope" in form:
        lay["rope_theta"] = 50.0
    if form == "mod":
        lay["residual"] = 1
    x = bf16_to_f64(wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32)))
    bias = (rng.standard_normal((B, T)) * 0.2).astype(np.float32)
    dims = Dims(Hq, Hkv, hd, 1e-5)
    got = oracle.sparse_layer(x, lay, dims, K, bias=bias, tau=1.0, delta=0.05)
    want_y, _ = _brute_sparse_layer(x, lay, Hq, Hkv, hd, 1e-5, K, bias, 1.0, 0.05)
    assert np.allclose(got["y"], want_y, rtol=1e-11, atol=1e-12)


def test_mod_residual_with_zero_attention_output_equals_gated_form():
    x, lay, dims = _tiny(seed=93)
    lay = dict(lay, varsigma=1.0, w_o=np.zeros_like(lay["w_o"]))     # a = 0
    y7 = oracle.sparse_layer(x, lay, dims, 3)["y"]
    y6 = oracle.sparse_layer(x, dict(lay, residual=1), dims, 3)["y"]
    assert np.array_equal(y6, y7)


def test_check1_with_rope_and_qknorm_equals_dense_layer():
    x, lay, dims = _tiny(seed=94)
    rng = np.random.default_rng(95)
    lay = dict(lay, w_router=np.zeros_like(lay["w_router"]), router_bias=100.0, varsigma=1.0,
               rope_theta=1000.0,
               q_norm=wl.f32_to_bf16_bits((1 + 0.2 * rng.standard_normal(4)).astype(np.float32)),
               k_norm=wl.f32_to_bf16_bits((1 + 0.2 * rng.standard_normal(4)).astype(np.float32)))
    ys = oracle.sparse_layer(x, lay, dims, 1)["y"]
    yd = oracle.dense_layer(x, lay, dims)
    assert np.allclose(ys, yd, rtol=1e-12, atol=1e-12)


# ---------------------------------------------------------------------------------------------
# mechanism controls (Table 7): Routed-FFN and Selected-Q/full-KV
# ---------------------------------------------------------------------------------------------

def test_attention_block_then_full_ffn_refinement_is_the_dense_layer():
    x, lay, dims = _tiny(seed=120)
    lay = dict(lay, w_router=np.zeros_like(lay["w_router"]), router_bias=100.0, varsigma=1.0)
    h = oracle.attention_layer(x, lay, dims)
    y = oracle.routed_ffn_layer(h, lay, dims, 1)["y"]           # every token, r = 1
    assert np.array_equal(y, oracle.dense_layer(x, lay, dims))


def test_fullkv_with_every_token_selected_is_the_sparse_layer():
    x, lay, dims = _tiny(seed=121)
    bias = (np.random.default_rng(122).standard_normal(x.shape[:2]) * 0.1).astype(np.float32)
    a = oracle.sparse_layer_fullkv(x, lay, dims, 1, bias=bias, delta=0.05)
    b = oracle.sparse_layer(x, lay, dims, 1, bias=bias, delta=0.05)
    assert np.array_equal(a["y"], b["y"]) and np.array_equal(a["bias_out"], b["bias_out"])


def _brute_fullkv_and_routed_ffn(x, lay, Hq, Hkv, hd, eps, K, bias, tau, delta, mode):
    """Plain loops: mode "fullkv" (selected queries, every token's keys / values at positions
    <= the query's) or "ffn" (the FFN alone on the selected rows)."""
    B, T, d = x.shape
    k = T // K
    f64 = lambda a: bf16_to_f64(a) if np.asarray(a).dtype == np.uint16 else np.asarray(a, float)
    wr, wqkv, wo = f64(lay["w_router"]), f64(lay["w_qkv"]), f64(lay["w_o"])
    wg, wu, wd = f64(lay["w_gate"]), f64(lay["w_up"]), f64(lay["w_down"])
    g1, g2 = f64(lay["g_attn"]), f64(lay["g_ffn"])
    F = wg.shape[0]
    dq, dkv = Hq * hd, Hkv * hd
    y = x.copy()

    def norm(vec, g):
        r = math.sqrt(sum(v * v for v in vec) / len(vec) + eps)
        return [vec[c] / r * g[c] for c in range(len(vec))]

    def matvec(Wm, vec, rows):
        return [sum(Wm[r, c] * vec[c] for c in range(len(vec))) for r in rows]

    def ffn(v):
        gp, up = matvec(wg, v, range(F)), matvec(wu, v, range(F))
        return matvec(wd, [gp[n] / (1 + math.exp(-gp[n])) * up[n] for n in range(F)], range(d))

    for b in range(B):
        logit = []
        for t in range(T):
            s = np.float32(math.fsum([x[b, t, c] * wr[c] for c in range(d)]) + lay["router_bias"])
            logit.append(np.float32(s - np.float32(np.float32(tau) * bias[b, t])))
        S = sorted(sorted(range(T), key=lambda t: (-float(logit[t]), t))[:k])
        u_all = [norm(list(x[b, t]), g1) for t in range(T)]
        kk = [matvec(wqkv, u_all[t], range(dq, dq + dkv)) for t in range(T)]
        vv = [matvec(wqkv, u_all[t], range(dq + dkv, dq + 2 * dkv)) for t in range(T)]
        for t in S:
            r = 1.0 / (1.0 + math.exp(-float(logit[t])))
            if mode == "ffn":
                f = ffn(norm(list(x[b, t]), g2))
                for c in range(d):
                    y[b, t, c] = x[b, t, c] + lay["varsigma"] * r * f[c]
                continue
            q = matvec(wqkv, u_all[t], range(dq))
            o = []
            for h in range(Hq):
                g = h // (Hq // Hkv)
                sc = [sum(q[h * hd + c] * kk[j][g * hd + c] for c in range(hd)) / math.sqrt(hd)
                      for j in range(t + 1)]
                mx = max(sc)
                w = [math.exp(v - mx) for v in sc]
                o += [sum(w[j] * vv[j][g * hd + c] for j in range(t + 1)) / sum(w) for c in range(hd)]
            a = matvec(wo, o, range(d))
            f = ffn(norm([x[b, t, c] + a[c] for c in range(d)], g2))
            for c in range(d):
                y[b, t, c] = x[b, t, c] + lay["varsigma"] * r * (a[c] + f[c])
    return y


@pytest.mark.parametrize("mode", ["fullkv", "ffn"])
def test_mechanism_controls_brute_force(mode):
    rng = np.random.default_rng(123 if mode == "fullkv" else 124)
    B, T, d, Hq, Hkv, hd, F, K = 2, 9, 8, 2, 1, 2, 6, 3
    lay = _rand_layer(rng, d, Hq, Hkv, hd, F)
    lay["router_bias"] = -0.2
    lay["varsigma"] = 1.3
    x = bf16_to_f64(wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32)))
    bias = (rng.standard_normal((B, T)) * 0.2).astype(np.float32)
    dims = Dims(Hq, Hkv, hd, 1e-5)
    if mode == "fullkv":
        got = oracle.sparse_layer_fullkv(x, lay, dims, K, bias=bias, tau=1.0, delta=0.05)
    else:
        got = oracle.routed_ffn_layer(x, lay, dims, K, bias=bias, tau=1.0, delta=0.05)
    want = _brute_fullkv_and_routed_ffn(x, lay, Hq, Hkv, hd, 1e-5, K, bias, 1.0, 0.05, mode)
    assert np.allclose(got["y"], want, rtol=1e-11, atol=1e-12)


def test_fullkv_sampling_matches_full():
    x, lay, dims = _tiny(seed=125, T=32)
    r = oracle.sparse_layer_fullkv(x, lay, dims, 4)
    rs = oracle.sparse_layer_fullkv(x, lay, dims, 4, sample={0: np.array([0, 3, 7]), 1: np.array([5])})
    for b, (prow, pos, ysel) in rs["rows"].items():
        # same arithmetic on fewer rows: equal up to the blocking of the float64 products
        assert np.allclose(ysel, r["y"][b, pos], rtol=1e-13, atol=1e-13)
