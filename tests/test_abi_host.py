"""Host-side checks of the C ABI (no GPU): the library loads, exports every symbol the header
declares, sizes workspaces, and rejects invalid arguments before touching a device."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
LIB = os.path.join(ROOT, "sparse_depth_token_amd", "libxmod.so")
HEADER = os.path.join(ROOT, "include", "xmod.h")



@pytest.fixture(scope="module")
def x():
    # a fresh checkout has no library (built files are not versioned): build it, so that these
    # checks never pass by being skipped (hipcc cross-compiles gfx950 without a GPU)
    if not os.path.exists(LIB):
        from sparse_depth_token_amd import build
        build.build()
    from sparse_depth_token_amd import xmod
    # XMOD_TEST_LIB: run these checks against another build of the library (the host
    # AddressSanitizer build of tests/test_host_asan.py), through the same signatures
    other = os.environ.get("XMOD_TEST_LIB")
    if other:
        L = ctypes.CDLL(other)
        for name, (res, args) in xmod._sig.items():
            f = getattr(L, name)
            f.restype, f.argtypes = res, args
        xmod.lib = L
    return xmod


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(xmod_[a-z_0-9]+)\s*\(", text)))


def test_header_symbols_exported(x):
    declared = _declared()
    assert len(declared) >= 13
    for name in declared:
        assert hasattr(x.lib, name), name
    assert sorted(x.EXPORTED) == declared


def test_status_strings(x):
    for st in range(5):
        assert x.lib.xmod_status_string(st)
    assert x.lib.xmod_last_hip_error() == 0


def _dims(x, **kw):
    base = dict(B=8, T=4096, d=2048, n_q_heads=16, n_kv_heads=16, head_dim=128, ffn_hidden=5632,
                rms_eps=1e-6)
    base.update(kw)
    return x.Dims(**base)


def test_workspace_sizes(x):
    dm = _dims(x)
    M = 8 * 512
    ws = x.workspace_bytes(dm, 8, x.WS_SPARSE_LAYER)
    # logits + idx + gate + u + qkv + o + a (fp32) + g (each rounded up to 256 bytes)
    want = (8 * 4096 * 4 + 2 * M * 4 + M * 2048 * 2 + M * 6144 * 2 + M * 2048 * 2 + M * 2048 * 4
            + M * 5632 * 2)
    assert want <= ws <= want + 8 * 256
    dense = x.workspace_bytes(dm, 8, x.WS_DENSE_LAYER)
    assert x.workspace_bytes(dm, 8, x.WS_BLOCK) == max(ws, dense)
    assert x.workspace_bytes(dm, 8, x.WS_ROUTE_TOPK) == 0
    assert x.workspace_bytes(_dims(x, head_dim=96), 8, x.WS_SPARSE_LAYER) == 0
    assert x.workspace_bytes(dm, 0, x.WS_SPARSE_LAYER) == 0
    assert x.workspace_bytes(dm, 8, 99) == 0


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every call below fails validation first


def _layer(x):
    return x.Layer(FAKE, 0.0, 1.0, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, FAKE)


def test_sparse_layer_rejects_before_launch(x):
    L = _layer(x)
    dm = _dims(x)
    f = x.lib.xmod_sparse_layer_fwd
    args = lambda **o: [o.get("x", FAKE), ctypes.byref(o.get("L", L)), ctypes.byref(o.get("dm", dm)),
                        o.get("K", 8), None, 1.0, 0.05, None, None, o.get("ws", FAKE),
                        o.get("wsb", 1 << 40), None]
    assert f(*args(K=0)) == x.ERR_INVALID_ARG
    assert f(*args(K=5000)) == x.ERR_INVALID_ARG                  # floor(T/K) < 1
    assert f(*args(x=None)) == x.ERR_INVALID_ARG
    assert f(*args(dm=_dims(x, n_kv_heads=3))) == x.ERR_INVALID_ARG  # Hq % Hkv != 0
    assert f(*args(dm=_dims(x, head_dim=96))) == x.ERR_UNSUPPORTED
    assert f(*args(dm=_dims(x, d=2000))) == x.ERR_UNSUPPORTED
    assert f(*args(dm=_dims(x, T=70000))) == x.ERR_UNSUPPORTED
    assert f(*args(dm=_dims(x, B=0))) == x.ERR_INVALID_ARG
    assert f(*args(wsb=1024)) == x.ERR_WORKSPACE
    assert f(*args(ws=None)) == x.ERR_WORKSPACE
    bad = _layer(x)
    bad.w_router = None
    assert f(*args(L=bad)) == x.ERR_INVALID_ARG
    nan = _layer(x)
    nan.varsigma = float("nan")
    assert f(*args(L=nan)) == x.ERR_INVALID_ARG


def test_block_rejects_before_launch(x):
    dm = _dims(x)
    layers = (x.Layer * 5)(*[_layer(x) for _ in range(5)])
    f = x.lib.xmod_block_fwd
    call = lambda n, N0, N1, A, K: f(FAKE, layers, n, ctypes.byref(dm), N0, N1, A, K, FAKE, 1.0,
                                     0.05, FAKE, 1 << 40, None)
    assert call(4, 1, 2, 0.5, 2) == x.ERR_INVALID_ARG          # wrong layer count
    assert call(5, 1, 2, 0.3, 2) == x.ERR_INVALID_ARG          # A*K not an integer
    assert call(5, -1, 2, 0.5, 2) == x.ERR_INVALID_ARG
    nowr = (x.Layer * 5)(*[_layer(x) for _ in range(5)])
    nowr[1].w_router = None                                   # layer 1 is sparse: needs a router
    assert f(FAKE, nowr, 5, ctypes.byref(dm), 1, 2, 0.5, 2, FAKE, 1.0, 0.05, FAKE, 1 << 40,
             None) == x.ERR_INVALID_ARG


def test_stage_entry_points_reject_before_launch(x):
    L = x.lib
    f = L.xmod_topk_from_logits
    assert f(FAKE, 2, 100, 0, FAKE, None, None, 0.0, None, 0, None) == x.ERR_INVALID_ARG
    assert f(FAKE, 2, 100, 101, FAKE, None, None, 0.0, None, 0, None) == x.ERR_INVALID_ARG
    assert f(FAKE, 1, 70000, 5, FAKE, None, None, 0.0, None, 0, None) == x.ERR_UNSUPPORTED
    # the chunked select's workspace: per 4096-position chunk the counts of 2048 buckets and two
    # bases, per sequence the threshold; none for sequences of at most 8192 positions; large
    # batches run in groups of at most 4096 chunks
    n = L.xmod_topk_workspace_bytes
    assert n(1, 8192) == 0 and n(1, 70000) == 0 and n(0, 16384) == 0
    assert n(1, 8193) == 3 * 8192 + 3 * 8 + 8
    assert n(1, 32768) == 8 * 8192 + 8 * 8 + 8
    assert n(256, 65536) == 256 * (16 * 8192 + 16 * 8 + 8) == n(1000, 65536)
    assert f(FAKE, 1, 32768, 5, FAKE, None, None, 0.0, FAKE, n(1, 32768) - 1,
             None) == x.ERR_WORKSPACE
    dm = _dims(x, T=16384)
    assert x.workspace_bytes(dm, 4, x.WS_ROUTE_TOPK) == n(dm.B, dm.T) > 0
    assert L.xmod_pack(FAKE, FAKE, 2, 10, 100, 5, FAKE, None) == x.ERR_UNSUPPORTED
    assert L.xmod_pack(FAKE, None, 2, 10, 128, 5, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_scatter_gated(FAKE, FAKE, FAKE, float("inf"), FAKE, FAKE, 2, 10, 128, 5,
                                None) == x.ERR_INVALID_ARG
    assert L.xmod_gemm_bf16_nt(FAKE, 100, FAKE, 100, FAKE, 64, 10, 64, 100, None) == x.ERR_UNSUPPORTED
    assert L.xmod_gemm_bf16_nt(FAKE, 64, FAKE, 64, FAKE, 64, 0, 64, 64, None) == x.ERR_INVALID_ARG
    assert L.xmod_attention_fwd(FAKE, 384, FAKE, 128, 1, 10, 2, 1, 80, None) == x.ERR_UNSUPPORTED
    assert L.xmod_attention_fwd(FAKE, 384, FAKE, 128, 1, 10, 3, 2, 64, None) == x.ERR_INVALID_ARG
    assert L.xmod_route_topk(FAKE, FAKE, 0.0, None, 1.0, 0, ctypes.byref(_dims(x)), FAKE, FAKE,
                             FAKE, None, 0, None) == x.ERR_INVALID_ARG


def test_threshold_entry_points_reject_before_launch(x):
    L = x.lib
    dm = _dims(x)
    # threshold routing workspace: sized for every row (B*T), plus counts / offsets / total
    ws = x.workspace_bytes(dm, 1, x.WS_SPARSE_THRESHOLD)
    assert ws >= x.workspace_bytes(dm, 1, x.WS_DENSE_LAYER) + 8 * 4096 * 4 * 3
    f = L.xmod_threshold_select
    assert f(FAKE, 0, 10, FAKE, FAKE, FAKE, None, FAKE, None, 0.0, None) == x.ERR_INVALID_ARG
    assert f(FAKE, 2, 10, None, FAKE, FAKE, None, FAKE, None, 0.0, None) == x.ERR_INVALID_ARG
    assert f(FAKE, 2, 10, FAKE, FAKE, FAKE, None, None, None, 0.0, None) == x.ERR_INVALID_ARG
    assert f(FAKE, 1, 70000, FAKE, FAKE, FAKE, None, FAKE, None, 0.0, None) == x.ERR_UNSUPPORTED
    assert f(FAKE, 2, 10, FAKE, FAKE, FAKE, None, FAKE, FAKE, float("nan"), None) == x.ERR_INVALID_ARG
    g = L.xmod_sparse_layer_fwd_threshold
    lay = _layer(x)
    args = lambda **o: [o.get("x", FAKE), ctypes.byref(o.get("L", lay)),
                        ctypes.byref(o.get("dm", dm)), None, o.get("tau", 1.0), 0.05, None, None,
                        None, o.get("ws", FAKE), o.get("wsb", 1 << 40), None]
    assert g(*args(x=None)) == x.ERR_INVALID_ARG
    assert g(*args(tau=float("inf"))) == x.ERR_INVALID_ARG
    assert g(*args(dm=_dims(x, head_dim=80))) == x.ERR_UNSUPPORTED
    assert g(*args(wsb=ws - 1)) == x.ERR_WORKSPACE
    bad = _layer(x)
    bad.w_router = None
    assert g(*args(L=bad)) == x.ERR_INVALID_ARG
    h = L.xmod_mask_agreement
    assert h(FAKE, FAKE, 2, 10, 11, FAKE, None) == x.ERR_INVALID_ARG
    assert h(FAKE, FAKE, 2, 10, 5, None, None) == x.ERR_INVALID_ARG
    assert h(FAKE, FAKE, 1, 70000, 5, FAKE, None) == x.ERR_UNSUPPORTED


def test_training_entry_points_reject_before_launch(x):
    L = x.lib
    dm = _dims(x)
    saved = x.workspace_bytes(dm, 8, x.WS_TRAIN_SAVED)
    bwd = x.workspace_bytes(dm, 8, x.WS_BACKWARD)
    # the saved activations hold at least X, u, QKV, O, v, g, z = [zg | zu] (bf16), a and f
    # (fp32) of the 4096 routed rows
    M = 8 * 512
    assert saved >= M * (2048 * 2 * 3 + 6144 * 2 + 2048 * 2 + 5632 * 2 * 3 + 2048 * 4 * 2)
    assert bwd > 0
    assert x.workspace_bytes(dm, 0, x.WS_TRAIN_SAVED) == 0
    lay = _layer(x)
    f = L.xmod_sparse_layer_fwd_train
    args = lambda **o: [o.get("x", FAKE), ctypes.byref(o.get("L", lay)),
                        ctypes.byref(o.get("dm", dm)), o.get("K", 8), None, 1.0, 0.05, None, None,
                        o.get("saved", FAKE), o.get("sb", saved), None]
    assert f(*args(K=0)) == x.ERR_INVALID_ARG
    assert f(*args(x=None)) == x.ERR_INVALID_ARG
    assert f(*args(sb=saved - 1)) == x.ERR_WORKSPACE
    assert f(*args(saved=None)) == x.ERR_WORKSPACE
    for field, val in (("residual", 1), ("rope_theta", 1e4)):
        other = _layer(x)
        setattr(other, field, val)
        assert f(*args(L=other)) == x.ERR_UNSUPPORTED, field
    qn = _layer(x)
    qn.q_norm = FAKE
    assert f(*args(L=qn)) == x.ERR_UNSUPPORTED
    g = L.xmod_sparse_layer_bwd
    G = x.Grads(*[FAKE] * len(x.GRAD_FIELDS))
    bargs = lambda **o: [FAKE, o.get("dy", FAKE), FAKE, ctypes.byref(o.get("L", lay)),
                         ctypes.byref(dm), 8, o.get("coef", 1e-4), FAKE, o.get("sb", saved),
                         ctypes.byref(o.get("G", G)), None, FAKE, o.get("wsb", bwd), None]
    assert g(*bargs(dy=None)) == x.ERR_INVALID_ARG
    assert g(*bargs(coef=float("nan"))) == x.ERR_INVALID_ARG
    assert g(*bargs(sb=saved - 1)) == x.ERR_WORKSPACE
    assert g(*bargs(wsb=bwd - 1)) == x.ERR_WORKSPACE
    nog = x.Grads(*[FAKE] * len(x.GRAD_FIELDS))
    nog.w_o = None
    assert g(*bargs(G=nog)) == x.ERR_INVALID_ARG
    other = _layer(x)
    other.residual = 1
    assert g(*bargs(L=other)) == x.ERR_UNSUPPORTED


def test_layout_gemm_and_attention_backward_reject_before_launch(x):
    L = x.lib
    f = L.xmod_gemm_bf16
    # layout, A, lda, B, ldb, C, ldc, out_f32, M, N, K
    assert f(3, FAKE, 64, FAKE, 64, FAKE, 64, 1, 64, 64, 64, None) == x.ERR_INVALID_ARG
    assert f(x.GEMM_NN, FAKE, 64, FAKE, 32, FAKE, 64, 1, 64, 64, 64, None) == x.ERR_INVALID_ARG  # ldb < N
    assert f(x.GEMM_TN, FAKE, 32, FAKE, 64, FAKE, 64, 1, 64, 64, 64, None) == x.ERR_INVALID_ARG  # lda < M
    assert f(x.GEMM_TN, FAKE, 64, FAKE, 64, FAKE, 64, 0, 64, 64, 64, None) == x.ERR_UNSUPPORTED  # bf16 out
    assert f(x.GEMM_NN, FAKE, 96, FAKE, 64, FAKE, 64, 1, 64, 64, 96, None) == x.ERR_UNSUPPORTED  # K % 64
    assert f(x.GEMM_TN, FAKE, 68, FAKE, 64, FAKE, 64, 1, 60, 64, 64, None) == x.ERR_UNSUPPORTED  # M % 8
    assert f(x.GEMM_NN, FAKE, 64, FAKE, 64, FAKE, 64, 1, 0, 64, 64, None) == x.ERR_INVALID_ARG
    g = L.xmod_attention_bwd
    assert g(FAKE, 384, FAKE, 128, FAKE, FAKE, 128, FAKE, FAKE, 384, 1, 10, 2, 1, 80,
             None) == x.ERR_UNSUPPORTED
    assert g(FAKE, 384, FAKE, 128, None, FAKE, 128, FAKE, FAKE, 384, 1, 10, 2, 1, 64,
             None) == x.ERR_INVALID_ARG
    assert g(FAKE, 384, FAKE, 128, FAKE, FAKE, 128, FAKE, FAKE, 100, 1, 10, 2, 1, 64,
             None) == x.ERR_INVALID_ARG
    assert L.xmod_attention_fwd_lse(FAKE, 384, FAKE, 128, None, 1, 10, 2, 1, 64,
                                    None) == x.ERR_INVALID_ARG


def test_probes_reject_before_launch(x):
    L = x.lib
    assert L.xmod_probe_mfma(None, 10, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_mfma(FAKE, 0, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_mfma(FAKE, (1 << 18) + 1, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read(None, 64, 4, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read(FAKE, 0, 4, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read(FAKE, 24, 4, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read(FAKE, 64, 4, None, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read(FAKE, 64, 5, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read_chunked(None, 64, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read_chunked(FAKE, 0, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read_chunked(FAKE, 24, FAKE, None) == x.ERR_INVALID_ARG
    assert L.xmod_probe_read_chunked(FAKE, 64, None, None) == x.ERR_INVALID_ARG


def test_operand_size_limits_reject_before_launch(x):
    """The projections address their operands by 32-bit byte offsets: a layer whose activation
    or weight matrices would hold 2^31 elements or more is refused before any launch (it would
    otherwise read wrapped addresses)."""
    L = _layer(x)
    ws = (FAKE, 1 << 40)
    # top-k layer: 8 x 16384 routed rows of 2F = 28672 columns (3.8e9 elements)
    big = _dims(x, B=8, T=65536, d=4096, n_q_heads=32, n_kv_heads=8, ffn_hidden=14336)
    assert x.lib.xmod_sparse_layer_fwd(FAKE, ctypes.byref(L), ctypes.byref(big), 4, None, 1.0,
                                       0.05, None, None, *ws, None) == x.ERR_UNSUPPORTED
    assert x.lib.xmod_sparse_layer_fwd_noalloc(FAKE, ctypes.byref(L), ctypes.byref(big), 4, None,
                                               1.0, 0.05, None, None, None) == x.ERR_UNSUPPORTED
    # dense layer and block: every one of the B*T rows is projected
    dense = _dims(x, B=2, T=65536, d=4096, n_q_heads=32, n_kv_heads=8, ffn_hidden=14336)
    assert x.lib.xmod_dense_layer_fwd(FAKE, ctypes.byref(L), ctypes.byref(dense), *ws,
                                      None) == x.ERR_UNSUPPORTED
    layers = (x.Layer * 2)(*[_layer(x) for _ in range(2)])
    assert x.lib.xmod_block_fwd(FAKE, layers, 2, ctypes.byref(dense), 0, 1, 0.5, 2, FAKE, 1.0,
                                0.05, *ws, None) == x.ERR_UNSUPPORTED
    # a weight matrix of 2^31 elements (F x d = 262144 x 8192) on a tiny input
    wide = _dims(x, B=1, T=64, d=8192, n_q_heads=64, n_kv_heads=64, ffn_hidden=262144)
    assert x.lib.xmod_sparse_layer_fwd(FAKE, ctypes.byref(L), ctypes.byref(wide), 1, None, 1.0,
                                       0.05, None, None, *ws, None) == x.ERR_UNSUPPORTED
    # stage GEMM: A of 65536 x 32768 elements
    assert x.lib.xmod_gemm_bf16_nt(FAKE, 32768, FAKE, 32768, FAKE, 64, 65536, 64, 32768,
                                   None) == x.ERR_UNSUPPORTED
    assert x.lib.xmod_gemm_bf16(x.GEMM_NT, FAKE, 32768, FAKE, 32768, FAKE, 64, 0, 65536, 64,
                                32768, None) == x.ERR_UNSUPPORTED
