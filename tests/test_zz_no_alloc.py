"""xmod_sparse_layer_fwd_noalloc, the sparse layer for callers that cannot allocate: its
workspace is the library's static per-GPU array instead of a caller buffer. It runs the same
kernels as xmod_sparse_layer_fwd, so its results must be the same bits; checked through the C
ABI on two calls in a row, the second on a smaller input (the array keeps the first call's
contents). A layer too large for the array is refused before any launch."""
import ctypes

import numpy as np
import pytest
import torch

import workload as wl
from parity import dev_bf16, host_bits, layer_to_device, say

xmod = pytest.importorskip("sparse_depth_token_amd.xmod")

# the MoD-pairs workload's sparse layer (B4 x T4096, d 1536, K 8: 61 MB of workspace), then a
# ragged GQA layer with gains, a router bias, a carried bias and varsigma
CALLS = [
    wl.WORKLOADS["mod_pairs_k8_b4x4096_d1536"],
    wl.Workload("noalloc_small", 61, 3, 700, 512, 8, 2, 64, 1536, 3, bias_std=0.1,
                varsigma_range=(0.5, 1.5), gain_std=0.1, router_bias=0.2),
]


def _dims(w):
    return xmod.make_dims(w.B, w.T, w.d, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden,
                          w.rms_eps)


def test_too_large_for_the_array_is_refused_before_any_launch():
    w = wl.WORKLOADS["sparse_k8_b8x4096_d2048"]
    dims = _dims(w)
    assert xmod.workspace_bytes(dims, w.K, xmod.WS_SPARSE_LAYER) > xmod.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    L = xmod.Layer(fake, 0.0, 1.0, fake, fake, fake, fake, fake, fake, fake, 0, None, None, 0.0)
    st = xmod.lib.xmod_sparse_layer_fwd_noalloc(fake, ctypes.byref(L), ctypes.byref(dims), w.K,
                                                None, 1.0, 0.05, None, None, None)
    assert st == xmod.ERR_WORKSPACE
    for c in CALLS:
        assert xmod.workspace_bytes(_dims(c), c.K, xmod.WS_SPARSE_LAYER) <= xmod.NOALLOC_SCRATCH_BYTES


@pytest.mark.gpu
def test_noalloc_equals_workspace_entry_point():
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    for w in CALLS:
        say(f"[no-alloc sparse layer] {w.name}: B{w.B} T{w.T} d{w.d} K{w.K}")
        dims = _dims(w)
        xb, lay, bias = wl.make_x(w), wl.make_layer(w, 0), wl.make_bias(w)
        L = xmod.make_layer(layer_to_device(lay))
        outs = []
        for noalloc in (False, True):
            xt = dev_bf16(xb)
            bt = torch.from_numpy(bias.copy()).cuda()
            idx = torch.full((w.B, w.k), -1, dtype=torch.int32, device="cuda")
            gate = torch.full((w.B, w.k), -1.0, dtype=torch.float32, device="cuda")
            if noalloc:
                xmod.sparse_layer_fwd_noalloc(xt, L, dims, w.K, bt, w.tau, w.delta, idx, gate)
            else:
                ws = xmod.alloc_workspace(dims, w.K, xmod.WS_SPARSE_LAYER)
                xmod.sparse_layer_fwd(xt, L, dims, w.K, bt, w.tau, w.delta, ws, idx, gate)
            torch.cuda.synchronize()
            outs.append((host_bits(xt), idx.cpu().numpy(), gate.cpu().numpy(), bt.cpu().numpy()))
        ref, got = outs
        assert np.all(ref[1] >= 0) and not np.array_equal(ref[0], xb)
        for name, a, b in zip(("x", "idx", "gate", "bias"), ref, got):
            assert np.array_equal(a, b), f"{w.name}: {name} differs from the workspace entry point"
