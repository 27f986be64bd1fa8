"""Pins of the backward oracle (oracle/backward.py), no GPU needed.

The backward is the chain rule written out by hand; these tests tie it to things other than
itself: central finite differences of the float64 forward oracle (oracle.sparse_layer, a
separate piece of code) for every parameter and input, the Eq. (9) routing loss against a
library routine and its closed form at s = 0, and special cases with a known answer.
"""
import numpy as np
import pytest

import oracle


class Dims:
    def __init__(self, Hq, Hkv, hd, eps=1e-6):
        self.n_q_heads, self.n_kv_heads, self.head_dim, self.rms_eps = Hq, Hkv, hd, eps


PARAMS = ("w_router", "g_attn", "w_qkv", "w_o", "g_ffn", "w_gate", "w_up", "w_down")


def _setup(seed, B=2, T=8, d=8, Hq=2, Hkv=1, hd=4, F=12, K=2, std=0.4):
    rng = np.random.default_rng(seed)
    dq, dkv = Hq * hd, Hkv * hd
    w = lambda *s: rng.standard_normal(s) * std
    lay = {"w_router": w(d), "g_attn": 1 + 0.3 * rng.standard_normal(d), "w_qkv": w(dq + 2 * dkv, d),
           "w_o": w(d, dq), "g_ffn": 1 + 0.3 * rng.standard_normal(d), "w_gate": w(F, d),
           "w_up": w(F, d), "w_down": w(d, F), "router_bias": 0.1, "varsigma": 0.9}
    x = rng.standard_normal((B, T, d))
    bias = (0.3 * rng.standard_normal((B, T))).astype(np.float32)
    dy = rng.standard_normal((B, T, d))
    return x, lay, Dims(Hq, Hkv, hd, 1e-5), bias, dy


def _objective(x, lay, dims, K, bias, tau, dy, coef, idx_ref):
    res = oracle.sparse_layer(x, lay, dims, K, bias=bias, tau=tau, exact_logits=True)
    assert np.array_equal(res["idx"], idx_ref), "a perturbation changed the selection"
    return float(np.sum(dy * res["y"])) + coef * oracle.route_bce(res["s"], res["idx"])


def _selection_margin(x, lay, bias, tau, K):
    s, ell = oracle.router_logits(x, lay["w_router"], lay["router_bias"], bias, tau, exact=True)
    k = x.shape[1] // K
    gaps = []
    for b in range(x.shape[0]):
        srt = np.sort(ell[b])[::-1]
        if k < len(srt):
            gaps.append(srt[k - 1] - srt[k])
    return min(gaps) if gaps else np.inf


@pytest.mark.parametrize("Hq,Hkv,K,coef", [(2, 1, 2, 1e-4), (2, 2, 1, 0.0), (4, 2, 3, 0.5)])
def test_grad_matches_central_differences(Hq, Hkv, K, coef):
    """Every gradient of sparse_layer_grad against (L(p + h) - L(p - h)) / 2h of the forward
    oracle, L = <dy, y> + coef * L_route, for every entry of every parameter and of x."""
    tau = 1.3
    for seed in range(20, 60):
        x, lay, dims, bias, dy = _setup(seed, Hq=Hq, Hkv=Hkv, K=K, T=9 if K == 3 else 8)
        if _selection_margin(x, lay, bias, tau, K) > 1e-3:
            break
    g = oracle.sparse_layer_grad(x, lay, dims, K, dy, bias=bias, tau=tau, route_coef=coef,
                                 exact_logits=True)
    idx = g["idx"]
    h = 1e-6
    L = lambda xx, ll: _objective(xx, ll, dims, K, bias, tau, dy, coef, idx)

    def fd_tensor(get, put, shape):
        out = np.zeros(shape)
        for i in np.ndindex(*shape):
            put(i, +h); lp = L(x_cur[0], lay_cur[0])
            put(i, -2 * h); lm = L(x_cur[0], lay_cur[0])
            put(i, +h)
            out[i] = (lp - lm) / (2 * h)
        return out

    x_cur, lay_cur = [x.copy()], [{k_: (v.copy() if isinstance(v, np.ndarray) else v)
                                   for k_, v in lay.items()}]
    for name in PARAMS:
        arr = lay_cur[0][name]

        def put(i, dv, arr=arr):
            arr[i] += dv
        num = fd_tensor(None, put, arr.shape)
        ana = g["d_" + name]
        assert np.allclose(ana, num, rtol=1e-5, atol=1e-7), \
            f"{name}: max |ana - num| = {np.abs(ana - num).max():.3g}"

    def put_x(i, dv):
        x_cur[0][i] += dv
    num = fd_tensor(None, put_x, x.shape)
    assert np.allclose(g["dx"], num, rtol=1e-5, atol=1e-7), \
        f"dx: max |ana - num| = {np.abs(g['dx'] - num).max():.3g}"

    for name in ("router_bias", "varsigma"):
        lp = dict(lay, **{name: lay[name] + h})
        lm = dict(lay, **{name: lay[name] - h})
        num = (L(x, lp) - L(x, lm)) / (2 * h)
        assert abs(g["d_" + name] - num) <= 1e-5 * abs(num) + 1e-7, (name, g["d_" + name], num)


def test_attention_grad_central_differences():
    """causal_attention_grad against finite differences of causal_attention, GQA 4/2 heads,
    queries at a subset of positions."""
    rng = np.random.default_rng(3)
    Hq, Hkv, hd, m = 4, 2, 3, 7
    Q = rng.standard_normal((m, Hq * hd))
    Kt = rng.standard_normal((m, Hkv * hd))
    Vt = rng.standard_normal((m, Hkv * hd))
    dO = rng.standard_normal((m, Hq * hd))
    pos = np.arange(m)
    dQ, dK, dV = oracle.causal_attention_grad(Q, Kt, Vt, pos, Hq, Hkv, hd, dO)
    h = 1e-6
    f = lambda q, k_, v: float(np.sum(dO * oracle.causal_attention(q, k_, v, pos, Hq, Hkv, hd)))
    for arr, ana in ((Q, dQ), (Kt, dK), (Vt, dV)):
        num = np.zeros_like(arr)
        for i in np.ndindex(*arr.shape):
            arr[i] += h; lp = f(Q, Kt, Vt)
            arr[i] -= 2 * h; lm = f(Q, Kt, Vt)
            arr[i] += h
            num[i] = (lp - lm) / (2 * h)
        assert np.allclose(ana, num, rtol=1e-6, atol=1e-8)


def test_rmsnorm_grad_central_differences():
    rng = np.random.default_rng(4)
    X = rng.standard_normal((3, 6))
    gain = 1 + 0.3 * rng.standard_normal(6)
    dY = rng.standard_normal((3, 6))
    dX, dg = oracle.rmsnorm_grad(X, gain, 1e-3, dY)
    h = 1e-6
    f = lambda X_, g_: float(np.sum(dY * oracle.rmsnorm(X_, g_, 1e-3)))
    for arr, ana in ((X, dX), (gain, dg)):
        num = np.zeros_like(arr)
        for i in np.ndindex(*arr.shape):
            arr[i] += h; lp = f(X, gain)
            arr[i] -= 2 * h; lm = f(X, gain)
            arr[i] += h
            num[i] = (lp - lm) / (2 * h)
        assert np.allclose(ana, num, rtol=1e-6, atol=1e-9)


def test_route_bce_against_library_and_closed_form():
    """Eq. (9) equals scikit-learn's log_loss of the top-k labels against sigmoid(s), and
    log 2 at s = 0 whatever the labels."""
    from sklearn.metrics import log_loss
    rng = np.random.default_rng(5)
    B, T, k = 3, 20, 5
    s = rng.standard_normal((B, T)) * 2
    idx = np.sort(np.argsort(-s, axis=1)[:, :k], axis=1)
    q = np.zeros((B, T)); q[np.arange(B)[:, None], idx] = 1
    p = 1 / (1 + np.exp(-s))
    assert abs(oracle.route_bce(s, idx) - log_loss(q.ravel(), p.ravel())) < 1e-12
    assert abs(oracle.route_bce(np.zeros((B, T)), idx) - np.log(2.0)) < 1e-15
    # the gradient of the mean loss in s is (p - q) / n
    g = oracle.route_bce_grad(s, idx)
    h = 1e-6
    for i in [(0, 0), (1, 7), (2, 19)]:
        sp, sm = s.copy(), s.copy()
        sp[i] += h; sm[i] -= h
        num = (oracle.route_bce(sp, idx) - oracle.route_bce(sm, idx)) / (2 * h)
        assert abs(g[i] - num) < 1e-9


def test_zero_varsigma_passes_dy_through():
    """varsigma = 0 makes the layer the identity (Eq. (7)): with no routing loss, dx = dy
    exactly, every weight and gain gradient is zero, and only varsigma itself gets one."""
    x, lay, dims, bias, dy = _setup(7)
    lay = dict(lay, varsigma=0.0)
    g = oracle.sparse_layer_grad(x, lay, dims, 2, dy, bias=bias, route_coef=0.0)
    assert np.array_equal(g["dx"], dy)
    for name in PARAMS:
        assert not np.any(g["d_" + name]), name
    assert g["d_router_bias"] == 0.0
    assert g["d_varsigma"] != 0.0


def test_unselected_rows_get_dy_plus_router_term():
    """A token outside the top-k has dx = dy + ds * w_router, where ds is only the routing
    loss's (p - q)/n scaled by the coefficient (q = 0 there)."""
    x, lay, dims, bias, dy = _setup(8)
    coef = 0.25
    g = oracle.sparse_layer_grad(x, lay, dims, 2, dy, bias=bias, route_coef=coef)
    s, _ = oracle.router_logits(x, lay["w_router"], lay["router_bias"], bias, 1.0)
    B, T = s.shape
    for b in range(B):
        for t in sorted(set(range(T)) - set(g["idx"][b].tolist())):
            p = 1 / (1 + np.exp(-float(s[b, t])))
            want = dy[b, t] + coef * p / (B * T) * lay["w_router"]
            assert np.allclose(g["dx"][b, t], want, rtol=0, atol=1e-15)
