"""The Python binding's host checks (CPU): a tensor of the wrong dtype, device, layout or size
raises before the library is called, so no kernel ever reads or writes past a buffer that a
bare C pointer cannot describe. The library is replaced by a stub that records calls, and the
tensors are shape-only ("meta") tensors standing in for device tensors, so nothing here needs a
GPU."""
import pytest
import torch

xmod = pytest.importorskip("sparse_depth_token_amd.xmod")


class StubLib:
    def __init__(self):
        self.calls = []

    def __getattr__(self, name):
        def fn(*args):
            self.calls.append(name)
            return 0
        return fn


@pytest.fixture
def stub(monkeypatch):
    s = StubLib()
    monkeypatch.setattr(xmod, "lib", s)
    monkeypatch.setattr(xmod, "_DEVICE_TYPE", "meta")
    monkeypatch.setattr(xmod, "_stream", lambda stream=None: None)
    return s


def T(*shape, dtype=torch.bfloat16):
    return torch.empty(*shape, dtype=dtype, device="meta")


B, TT, D, HQ, HKV, HD, F, K = 2, 64, 128, 2, 1, 64, 256, 4
k = TT // K
DIMS = xmod.make_dims(B, TT, D, HQ, HKV, HD, F)
DQ, DKV = HQ * HD, HKV * HD


def layer(**change):
    w = {"w_router": T(D), "g_attn": T(D), "w_qkv": T(DQ + 2 * DKV, D), "w_o": T(D, DQ),
         "g_ffn": T(D), "w_gate": T(F, D), "w_up": T(F, D), "w_down": T(D, F)}
    w.update(change)
    L = xmod.make_layer({n: v for n, v in w.items() if v is not None})
    return L


def good_sparse_args():
    return dict(x=T(B, TT, D), layer=layer(), dims=DIMS, K=K,
                bias=T(B, TT, dtype=torch.float32), tau=1.0, delta=0.05,
                ws=T(1024, dtype=torch.uint8), idx_out=T(B, k, dtype=torch.int32),
                gate_out=T(B, k, dtype=torch.float32))


def test_good_arguments_reach_the_library(stub):
    xmod.sparse_layer_fwd(**good_sparse_args())
    assert stub.calls == ["xmod_sparse_layer_fwd"]


@pytest.mark.parametrize("change", [
    {"x": T(B, TT, D, dtype=torch.float16)},                # wrong dtype
    {"x": T(B, TT - 1, D)},                                 # wrong size
    {"x": T(B, D, TT).transpose(1, 2)},                     # not contiguous
    {"x": torch.empty(B, TT, D, dtype=torch.bfloat16)},     # host tensor
    {"bias": T(B, TT, dtype=torch.float64)},                # fp64 bias
    {"bias": T(B, TT - 1, dtype=torch.float32)},
    {"idx_out": T(B, k, dtype=torch.int64)},                # int64 indices
    {"idx_out": T(B, k - 1, dtype=torch.int32)},            # too small
    {"gate_out": T(B, k - 1, dtype=torch.float32)},
    {"ws": T(1024, dtype=torch.float32)},                   # workspace must be bytes
    {"layer": layer(w_qkv=T(DQ + DKV, D))},                 # weight of the wrong shape
    {"layer": layer(w_down=T(D, F, dtype=torch.float32))},  # weight of the wrong dtype
    {"layer": layer(w_router=None)},                        # a sparse layer needs its router
    {"K": TT + 1},                                          # floor(T/K) = 0
])
def test_bad_arguments_raise_before_the_library(stub, change):
    a = good_sparse_args()
    a.update(change)
    with pytest.raises((TypeError, ValueError)):
        xmod.sparse_layer_fwd(**a)
    assert stub.calls == []


def test_other_entry_points(stub):
    x = T(B, TT, D)
    ws = T(4096, dtype=torch.uint8)
    bias = T(B, TT, dtype=torch.float32)
    with pytest.raises(ValueError):
        xmod.block_fwd(x, [layer()] * 3, DIMS, 0, 1, 2 / K, K, None, 1.0, 0.05, ws)  # bias required
    with pytest.raises(TypeError):
        xmod.dense_layer_fwd(T(B, TT, D, dtype=torch.float32), layer(), DIMS, ws)
    with pytest.raises(ValueError):
        xmod.pack(x, T(B, k, dtype=torch.int32), T(B * k - 1, D))            # output too small
    with pytest.raises(TypeError):
        xmod.topk_from_logits(T(B, TT, dtype=torch.float32), k, T(B, k, dtype=torch.int64))
    with pytest.raises(ValueError):
        xmod.scatter_gated(x, T(B, k, dtype=torch.int32), T(B * k - 1, dtype=torch.float32), 1.0,
                           T(B * k, D), T(B * k, D))
    with pytest.raises(ValueError):                                        # qkv too narrow
        xmod.attention_fwd(T(B * k, (HQ + 2 * HKV) * HD - 8), T(B * k, DQ), B, k, HQ, HKV, HD)
    with pytest.raises(ValueError):                                        # C not row-major
        xmod.gemm_bf16_nt(T(64, 128), T(64, 128), T(64, 64).t())
    with pytest.raises(ValueError):
        xmod.threshold_select(T(B, TT, dtype=torch.float32), T(B, dtype=torch.int32),
                              T(B, dtype=torch.int32), T(B * TT - 1, dtype=torch.int32),
                              T(1, dtype=torch.int32))
    assert stub.calls == []
    xmod.block_fwd(x, [layer()] * 3, DIMS, 0, 1, 2 / K, K, bias, 1.0, 0.05, ws)
    xmod.dense_layer_fwd(x, layer(w_router=None), DIMS, ws)
    xmod.gemm_bf16_nt(T(64, 128), T(64, 128), T(64, 64))
    xmod.attention_fwd(T(B * k, (HQ + 2 * HKV) * HD), T(B * k, DQ), B, k, HQ, HKV, HD)
    assert stub.calls == ["xmod_block_fwd", "xmod_dense_layer_fwd", "xmod_gemm_bf16_nt",
                          "xmod_attention_fwd"]
