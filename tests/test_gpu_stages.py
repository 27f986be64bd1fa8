"""Stage-by-stage parity of the HIP path against the oracle (needs an MI355X).

Integer work (top-k indices, pack, scatter) must be bit-exact; floating-point stages must stay
within bounds derived from their arithmetic. Each case prints its name before touching the GPU.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from parity import (bf16_vals, check_values, compare_selection, dev_bf16, host_bits, say,
                    ulp_bf16)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def x():
    from sparse_depth_token_amd import xmod
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return xmod


# ---------------------------------------------------------------------------------------------
# top-k: bit-exact against the oracle on identical fp32 logits
# ---------------------------------------------------------------------------------------------

def _logit_cases():
    rng = np.random.default_rng(100)
    cases = []
    for B, T, k in [(1, 1, 1), (3, 7, 3), (2, 1000, 333), (8, 4096, 512), (4, 4096, 256),
                    (1, 32768, 8192), (2, 5000, 1), (2, 300, 300), (1, 65536, 20000)]:
        cases.append((f"normal B{B} T{T} k{k}", rng.standard_normal((B, T)).astype(np.float32), k))
    lv = rng.integers(0, 4, (4, 2048)).astype(np.float32) - 2.0
    lv[rng.random(lv.shape) < 0.25] = -0.0
    cases.append(("4-level ties with +-0", lv, 700))
    cases.append(("all equal", np.full((2, 3000), 0.25, np.float32), 1111))
    tiny = (rng.standard_normal((3, 4096)) * 1e-30).astype(np.float32)
    cases.append(("tiny magnitudes", tiny, 512))
    big = (rng.standard_normal((2, 4096)) * 1e30).astype(np.float32)
    big[0, ::7] = np.inf
    big[1, ::5] = -np.inf
    cases.append(("huge and infinite", big, 600))
    # long sequences (8 to 32 keys per thread: the strided key layout) with ties across
    # rows of 1024 positions and across waves, where the first `need` equal keys must win
    for B, T, k, levels in [(3, 6000, 1500, 4), (2, 32768, 8192, 3), (1, 20000, 7777, 1)]:
        lv = rng.integers(0, levels, (B, T)).astype(np.float32) - 1.0
        lv[rng.random(lv.shape) < 0.2] = -0.0
        cases.append((f"{levels}-level ties B{B} T{T} k{k}", lv, k))
    # shapes of the chunked select (4096-position chunks): a ragged last chunk, k = 1 and k = T,
    # many sequences (1370 x 3 chunks: two groups of at most 4096 chunks), and NaN / infinities
    # across chunks
    for B, T, k in [(2, 8193, 1), (1, 9000, 9000), (70, 12288, 100), (2, 65535, 30000),
                    (1370, 8200, 2050)]:
        cases.append((f"normal B{B} T{T} k{k}", rng.standard_normal((B, T)).astype(np.float32), k))
    odd = rng.standard_normal((3, 12000)).astype(np.float32)
    odd[0, ::3] = np.nan
    odd[1, ::11] = np.inf
    odd[1, 5::13] = -np.inf
    odd[2, :] = np.nan
    odd[2, 7000:7010] = -np.inf
    cases.append(("NaN and infinities B3 T12000", odd, 4000))
    return cases


def _ref_topk(ell, k):
    """The selection with +-inf ordered by value and NaN below everything (then position)."""
    if np.all(np.isfinite(ell)):
        return oracle.topk_select(ell, k)
    B, T = ell.shape
    nan = np.isnan(ell)
    v = np.where(nan, 0.0, ell.astype(np.float64))
    return np.stack([np.sort(np.lexsort((np.arange(T), -v[b], nan[b]))[:k]) for b in range(B)])


# (case, chunked): every case on one workgroup per sequence, and the cases long enough for the
# chunked select (more than 8192 positions) again with its workspace
_TOPK_PARAMS = [(i, False) for i in range(len(_logit_cases()))] + \
    [(i, True) for i, (_, ell, _) in enumerate(_logit_cases()) if ell.shape[1] > 8192]


@pytest.mark.parametrize("case,chunked", _TOPK_PARAMS)
def test_topk_bit_exact(x, case, chunked):
    name, ell, k = _logit_cases()[case]
    say(f"[topk] {name} chunked={chunked}")
    B, T = ell.shape
    lg = torch.from_numpy(ell).cuda()
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((B, k), dtype=torch.float32, device="cuda")
    bias0 = (np.random.default_rng(case).standard_normal((B, T)) * 0.1).astype(np.float32)
    bias = torch.from_numpy(bias0).cuda()
    ws = None
    if chunked:
        n = x.topk_workspace_bytes(B, T)
        assert n > 0
        ws = torch.full((n,), 0xA5, dtype=torch.uint8, device="cuda")  # not zeroed: unused
    x.topk_from_logits(lg, k, idx, gate, bias, 0.05, ws=ws)
    torch.cuda.synchronize()
    ref = _ref_topk(ell, k)
    got = idx.cpu().numpy()
    assert np.array_equal(got, ref), f"{name}: first mismatch {np.argwhere(got != ref)[:3]}"
    with np.errstate(all="ignore"):
        want_gate = oracle.sigmoid(ell[np.arange(B)[:, None], ref])
    assert np.allclose(gate.cpu().numpy(), want_gate, rtol=2e-6, atol=1e-30, equal_nan=True)
    want_bias = bias0.copy()
    want_bias[np.arange(B)[:, None], ref] = (bias0[np.arange(B)[:, None], ref] + np.float32(0.05))
    assert np.array_equal(bias.cpu().numpy(), want_bias)


# ---------------------------------------------------------------------------------------------
# router logits: forward error bound of the GPU's fp32 summation order
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("name,B,T,d,skew", [("d256", 2, 512, 256, 0.0), ("d2048", 8, 4096, 2048, 0.0),
                                             ("d1536 ragged", 3, 999, 1536, 0.0),
                                             ("d4096 skewed", 1, 8192, 4096, 0.01),
                                             ("d8192 widest, ragged", 2, 1000, 8192, 0.0)])
def test_router_logits(x, name, B, T, d, skew):
    say(f"[router] {name}")
    w = wl.scaled(wl.WORKLOADS["sparse_k2_b2x512_d256"], B=B, T=T, d=d, skew_frac=skew, seed=7)
    xb = wl.make_x(w)
    rng = np.random.default_rng(8)
    wr = wl.f32_to_bf16_bits((rng.standard_normal(d) * 0.02).astype(np.float32))
    bias = (rng.standard_normal((B, T)) * 0.1).astype(np.float32)
    K = 4
    k = T // K
    dims = x.make_dims(B, T, d, 2, 2, 64, 64)
    xt, wt = dev_bf16(xb), dev_bf16(wr)
    bt = torch.from_numpy(bias).cuda()
    logits = torch.empty((B, T), dtype=torch.float32, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    gate = torch.empty((B, k), dtype=torch.float32, device="cuda")
    x.route_topk(xt, wt, 0.125, bt, 1.0, K, dims, logits, idx, gate)
    torch.cuda.synchronize()
    s_ref, ell_ref = oracle.router_logits(xb, wr, 0.125, bias, 1.0)
    got = logits.cpu().numpy().astype(np.float64)
    # |error| <= (d/64 + 8) * u * sum|x_i w_i| (per-lane sequential sums, then a 6-level tree),
    # plus the roundings of +beta, tau*b and the subtraction.
    absprod = np.abs(bf16_vals(xb)) @ np.abs(bf16_vals(wr))
    u = 2.0 ** -24
    bound = (d / 64 + 8) * u * absprod + 4 * u * (np.abs(ell_ref) + np.abs(s_ref) + np.abs(bias)) + 1e-30
    assert np.all(np.abs(got - ell_ref) <= bound)
    # selection: the oracle's, except swaps between near-equal oracle logits
    compare_selection(idx.cpu().numpy(), oracle.topk_select(ell_ref, k), ell_ref)


# ---------------------------------------------------------------------------------------------
# pack, scatter, RMSNorm rows
# ---------------------------------------------------------------------------------------------

def _rand_idx(rng, B, T, k):
    return np.stack([np.sort(rng.permutation(T)[:k]) for _ in range(B)]).astype(np.int32)


@pytest.mark.parametrize("B,T,d,k", [(2, 512, 256, 256), (3, 777, 1536, 100), (1, 4096, 4096, 1024),
                                     (2, 300, 8192, 77)])
def test_pack_bit_exact(x, B, T, d, k):
    say(f"[pack] B{B} T{T} d{d} k{k}")
    rng = np.random.default_rng(9)
    xb = wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32))
    idx = _rand_idx(rng, B, T, k)
    out = torch.empty((B * k, d), dtype=torch.bfloat16, device="cuda")
    x.pack(dev_bf16(xb), torch.from_numpy(idx).cuda(), out)
    torch.cuda.synchronize()
    want = xb[np.arange(B)[:, None], idx].reshape(B * k, d)
    assert np.array_equal(host_bits(out), want)


def _f32_gated(X, g, a, f):
    """The gated residual's fp32 operation order: t = a + f, p = g*t, y = X + p."""
    t = (a.astype(np.float32) + f.astype(np.float32)).astype(np.float32)
    p = (g.astype(np.float32) * t).astype(np.float32)
    return (X.astype(np.float32) + p).astype(np.float32)


@pytest.mark.parametrize("B,T,d,k", [(2, 512, 256, 256), (3, 777, 1536, 100), (2, 300, 8192, 77)])
def test_scatter_bit_exact_and_untouched_rows(x, B, T, d, k):
    say(f"[scatter] B{B} T{T} d{d} k{k}")
    rng = np.random.default_rng(10)
    xb = wl.f32_to_bf16_bits(rng.standard_normal((B, T, d)).astype(np.float32))
    ab = wl.f32_to_bf16_bits(rng.standard_normal((B * k, d)).astype(np.float32))
    fb = wl.f32_to_bf16_bits(rng.standard_normal((B * k, d)).astype(np.float32))
    idx = _rand_idx(rng, B, T, k)
    gate = rng.random(B * k).astype(np.float32)
    vs = np.float32(1.3)
    xt = dev_bf16(xb)
    x.scatter_gated(xt, torch.from_numpy(idx).cuda(), torch.from_numpy(gate).cuda(), float(vs),
                    dev_bf16(ab), dev_bf16(fb))
    torch.cuda.synchronize()
    got = host_bits(xt)
    sel = np.zeros((B, T), bool)
    sel[np.arange(B)[:, None], idx] = True
    assert np.array_equal(got[~sel], xb[~sel])                       # untouched rows
    X = wl.bf16_bits_to_f32(xb[np.arange(B)[:, None], idx].reshape(B * k, d))
    g = (vs * gate).astype(np.float32)[:, None]
    y32 = _f32_gated(X, g, wl.bf16_bits_to_f32(ab), wl.bf16_bits_to_f32(fb))
    want = wl.f32_to_bf16_bits(y32)
    assert np.array_equal(got[np.arange(B)[:, None], idx].reshape(B * k, d), want)
    # and against the oracle's float64 definition: within fp32 rounding + the bf16 output step
    y64 = X.astype(np.float64) + (float(vs) * gate.astype(np.float64))[:, None] * (
        bf16_vals(ab) + bf16_vals(fb))
    gv = bf16_vals(got[np.arange(B)[:, None], idx].reshape(B * k, d))
    assert np.all(np.abs(gv - y64) <= 0.5 * ulp_bf16(y64) + 1e-5 * (1 + np.abs(y64)))


@pytest.mark.parametrize("B,T,d,k,use_idx", [(2, 512, 256, 256, True), (3, 777, 1536, 100, True),
                                             (2, 64, 4096, 64, False), (2, 300, 6144, 50, True),
                                             (1, 64, 8192, 64, False)])
def test_rmsnorm_rows(x, B, T, d, k, use_idx):
    say(f"[rmsnorm] B{B} T{T} d{d} k{k} idx={use_idx}")
    rng = np.random.default_rng(11)
    xb = wl.f32_to_bf16_bits((rng.standard_normal((B, T, d)) * 3).astype(np.float32))
    gain = wl.f32_to_bf16_bits((1 + 0.3 * rng.standard_normal(d)).astype(np.float32))
    idx = _rand_idx(rng, B, T, k) if use_idx else None
    out = torch.empty((B * k, d), dtype=torch.bfloat16, device="cuda")
    x.rmsnorm_rows(dev_bf16(xb), torch.from_numpy(idx).cuda() if use_idx else None, dev_bf16(gain),
                   1e-6, k, out)
    torch.cuda.synchronize()
    X = bf16_vals(xb)[np.arange(B)[:, None], idx].reshape(B * k, d) if use_idx else \
        bf16_vals(xb).reshape(B * T, d)[:B * k]
    ref = oracle.rmsnorm(X, bf16_vals(gain), 1e-6)
    got = bf16_vals(host_bits(out))
    assert np.all(np.abs(got - ref) <= 0.5 * ulp_bf16(ref) + 2e-6 * np.abs(ref) + 1e-30)


# ---------------------------------------------------------------------------------------------
# GEMM and attention against float64 definitions
# ---------------------------------------------------------------------------------------------

@pytest.mark.parametrize("M,N,K", [(512, 768, 256), (300, 200, 128), (4096, 2048, 2048),
                                   (1000, 1536, 1024), (8192, 6144, 512),
                                   # wide grids: several waves of 256x128 tiles, ragged rows
                                   (4096, 6144, 128), (3900, 6144, 192),
                                   # small grids of 64x64 tiles (32-row wave tiles): the
                                   # A3K16 layer's O and down shapes, ragged rows and columns
                                   (1024, 1024, 1024), (1024, 1024, 2816), (1000, 1000, 640),
                                   (72, 136, 64),
                                   # 28 x 20 tiles of 256x256 (more than two waves on the
                                   # 256 CUs), ragged rows and columns
                                   (7000, 5000, 192)])
def test_gemm(x, M, N, K):
    say(f"[gemm] M{M} N{N} K{K}")
    rng = np.random.default_rng(12)
    A = wl.f32_to_bf16_bits(rng.standard_normal((M, K)).astype(np.float32))
    Bw = wl.f32_to_bf16_bits((rng.standard_normal((N, K)) * 0.05).astype(np.float32))
    C = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")  # unwritten: NaN
    x.gemm_bf16_nt(dev_bf16(A), dev_bf16(Bw), C)
    torch.cuda.synchronize()
    Af, Bf = bf16_vals(A), bf16_vals(Bw)
    ref = Af @ Bf.T
    acc_bound = K * 2.0 ** -24 * (np.abs(Af) @ np.abs(Bf).T)       # fp32 accumulation
    got = bf16_vals(host_bits(C))
    assert np.all(np.abs(got - ref) <= 0.5 * ulp_bf16(ref) + acc_bound + 1e-30)


@pytest.mark.parametrize("layout,M,N,K,f32,pad", [
    # dY W products of the backward (B stored [K, N]); ragged rows, a K split over many tiles
    ("NN", 512, 256, 1024, False, 0), ("NN", 700, 2048, 6144, True, 0),
    ("NN", 4096, 5632, 2048, False, 0), ("NN", 96, 1536, 128, True, 64),
    # weight gradients dY^T X (sums over K token rows); M and N multiples of 8, not of the tile
    ("TN", 256, 768, 512, True, 0), ("TN", 2048, 5632, 4096, True, 0),
    ("TN", 1544, 1032, 192, True, 32), ("TN", 11264, 2048, 256, True, 0),
    ("NT", 640, 384, 256, True, 0),
    # 256x256 tiles over more than two waves: fp32 and bf16 stores, ragged tiles, a strided A
    ("NT", 7000, 5000, 192, True, 0), ("NT", 6500, 5200, 256, False, 24)])
def test_gemm_layouts(x, layout, M, N, K, f32, pad):
    say(f"[gemm {layout}] M{M} N{N} K{K} f32={f32} pad={pad}")
    rng = np.random.default_rng(14)
    lay = {"NT": x.GEMM_NT, "NN": x.GEMM_NN, "TN": x.GEMM_TN}[layout]
    a_shape = (K, M) if layout == "TN" else (M, K)
    b_shape = (N, K) if layout == "NT" else (K, N)
    A = wl.f32_to_bf16_bits(rng.standard_normal(a_shape).astype(np.float32))
    Bw = wl.f32_to_bf16_bits((rng.standard_normal(b_shape) * 0.05).astype(np.float32))
    # optional row padding of A: a strided view (leading dimension > its columns)
    Ad = dev_bf16(np.pad(A, ((0, 0), (0, pad)))) [:, :a_shape[1]] if pad else dev_bf16(A)
    C = torch.full((M, N), float("nan"), dtype=torch.float32 if f32 else torch.bfloat16,
                   device="cuda")  # an element the kernel leaves unwritten stays NaN
    x.gemm_bf16(lay, Ad, dev_bf16(Bw), C)
    torch.cuda.synchronize()
    Af, Bf = bf16_vals(A), bf16_vals(Bw)
    Am = Af.T if layout == "TN" else Af
    Bm = Bf if layout != "NT" else Bf.T
    ref = Am @ Bm
    acc_bound = K * 2.0 ** -24 * (np.abs(Am) @ np.abs(Bm))       # fp32 accumulation
    if f32:
        got = C.cpu().numpy().astype(np.float64)
        out_round = np.abs(ref) * 2.0 ** -24
    else:
        got = bf16_vals(host_bits(C))
        out_round = 0.5 * ulp_bf16(ref)
    err = np.abs(got - ref) - (out_round + acc_bound + 1e-30)
    assert np.all(err <= 0), f"worst excess {err.max():.3g} at {np.unravel_index(err.argmax(), err.shape)}"


@pytest.mark.parametrize("B,k,Hq,Hkv,hd", [(2, 256, 4, 4, 64), (1, 333, 4, 2, 128), (3, 200, 8, 2, 64),
                                           (2, 512, 16, 16, 128), (1, 1100, 4, 1, 128),
                                           (1, 1, 2, 1, 128), (2, 65, 4, 4, 64), (1, 129, 2, 2, 128),
                                           (1, 64, 2, 2, 64),
                                           # more workgroups than CUs: one 256-row q-tile per
                                           # workgroup, ragged last tiles
                                           (1, 1100, 64, 8, 64), (2, 700, 48, 6, 128),
                                           # sequences of 2048 rows and more: 128-row key
                                           # tiles (pair split on a small grid, one-tile split
                                           # on a large one; ragged and exact last tiles)
                                           (1, 2100, 8, 2, 128), (2, 2048, 4, 4, 64),
                                           (1, 2500, 48, 8, 128)])
def test_attention(x, B, k, Hq, Hkv, hd):
    say(f"[attention] B{B} k{k} Hq{Hq} Hkv{Hkv} hd{hd}")
    rng = np.random.default_rng(13)
    n = (Hq + 2 * Hkv) * hd
    qkv = wl.f32_to_bf16_bits((rng.standard_normal((B * k, n)) * 1.5).astype(np.float32))
    o = torch.empty((B * k, Hq * hd), dtype=torch.bfloat16, device="cuda")
    x.attention_fwd(dev_bf16(qkv), o, B, k, Hq, Hkv, hd)
    torch.cuda.synchronize()
    got = bf16_vals(host_bits(o))
    qv = bf16_vals(qkv)
    for b in range(B):
        rows = qv[b * k:(b + 1) * k]
        ref = oracle.causal_attention(rows[:, :Hq * hd], rows[:, Hq * hd:(Hq + Hkv) * hd],
                                      rows[:, (Hq + Hkv) * hd:], np.arange(k), Hq, Hkv, hd)
        # probabilities are rounded to bf16 before the P*V product: relative 2^-8 per weight
        check_values(got[b * k:(b + 1) * k], ref, f"attention seq {b}", abs_tol=1.5e-2, rel_tol=6e-3)
