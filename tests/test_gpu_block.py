"""Stacks of layers: [Dense]xN0 + ([Sparse(K)]xAK + [Dense])xN1 on the GPU.

* Lock-step: the oracle walks the whole stack on its own; every GPU layer is then fed the
  oracle's state at that layer's input (hidden state and carried bias) and compared with the
  oracle's output of that layer. No GPU value ever enters the oracle.
* The block entry point equals the same layers called one by one (bitwise), at full size.
* Free-running properties: with varsigma = 0 in the sparse layers (x frozen) and a bias step
  far above the logit range, the carried bias rotates the selection so each token is chosen
  exactly AK/K times per block; exactly k tokens are selected per sparse layer in any stack.
"""
import numpy as np
import pytest
import torch

import oracle
import workload as wl
from parity import (bf16_vals, check_values, compare_selection, dev_bf16, host_bits,
                    layer_to_device, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def x():
    from sparse_depth_token_amd import xmod
    assert torch.cuda.is_available(), "GPU tests need a ROCm device"
    return xmod


def _dims(x, w):
    return x.make_dims(w.B, w.T, w.d, w.n_q_heads, w.n_kv_heads, w.head_dim, w.ffn_hidden, w.rms_eps)


REDUCED = {
    "MoD pairs ([S(8)]+[D])x2, B2 T512 d256": wl.Workload(
        "mod_pairs_small", 31, 2, 512, 256, 4, 4, 64, 512, 8, N0=0, N1=2, AK=1),
    "A1.5K4 block: D + ([S(4)]x6 + D)x2, B2 T512 d256 GQA 4/2": wl.Workload(
        "xmod_small", 32, 2, 512, 256, 4, 2, 64, 512, 4, N0=1, N1=2, AK=6, delta=0.05),
}


@pytest.mark.parametrize("name", list(REDUCED))
def test_block_lockstep(x, name):
    w = REDUCED[name]
    kinds = w.layer_kinds()
    say(f"[lock-step] {name}: {''.join(kinds)}")
    xb = wl.make_x(w)
    layers = [wl.make_layer(w, l) for l in range(len(kinds))]
    _, trace = oracle.block_forward(xb, layers, w, kinds, w.K, tau=w.tau, delta=w.delta, record=True)
    dims = _dims(x, w)
    ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
    for l, (kind, e) in enumerate(zip(kinds, trace)):
        xin = oracle.f64_to_bf16_bits(e["x_in"])
        xt = dev_bf16(xin)
        dl = layer_to_device(layers[l])       # keeps the weight tensors alive during the call
        L = x.make_layer(dl)
        if kind == "D":
            x.dense_layer_fwd(xt, L, dims, ws)
            torch.cuda.synchronize()
            check_values(bf16_vals(host_bits(xt)), e["y"], f"layer {l} (dense)")
            continue
        bt = torch.from_numpy(e["bias_in"].copy()).cuda()
        idx = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
        x.sparse_layer_fwd(xt, L, dims, w.K, bt, w.tau, w.delta, ws, idx, None)
        torch.cuda.synchronize()
        idx_g = idx.cpu().numpy()
        first = compare_selection(idx_g, e["idx"], e["ell"])
        y = host_bits(xt)
        sel = np.zeros((w.B, w.T), bool)
        sel[np.arange(w.B)[:, None], idx_g] = True
        assert np.array_equal(y[~sel], xin[~sel]), f"layer {l}: unselected rows changed"
        same = first == w.k
        assert np.array_equal(bt.cpu().numpy()[same], e["bias_out"][same]), f"layer {l}: bias"
        for b in range(w.B):
            rows = idx_g[b, :first[b]]
            check_values(bf16_vals(y[b, rows]), e["y"][b, rows], f"layer {l} seq {b}")


def _gpu_layers(x, w, seed_shift=0):
    kinds = w.layer_kinds()
    host = [wl.make_layer(w, l + seed_shift) for l in range(len(kinds))]
    dev = [layer_to_device(h) for h in host]
    return kinds, host, dev, [x.make_layer(d) for d in dev]


def _composed(x, w, kinds, Ls, xt, bt, ws, dims):
    """The stack walked layer by layer through the single-layer entry points."""
    n_in_block = w.AK + 1
    for i, (kind, L) in enumerate(zip(kinds, Ls)):
        if i >= w.N0 and (i - w.N0) % n_in_block == 0:
            bt.zero_()
        if kind == "S":
            x.sparse_layer_fwd(xt, L, dims, w.K, bt, w.tau, w.delta, ws)
        else:
            x.dense_layer_fwd(xt, L, dims, ws)


@pytest.mark.parametrize("name", ["mod_pairs_k8_b4x4096_d1536", "a3k16_block_b4x4096_d1024"])
def test_block_entry_equals_composed_layers_full_size(x, name):
    w = wl.WORKLOADS[name]
    say(f"[block == composed] {name}")
    kinds, _, dev, Ls = _gpu_layers(x, w)
    dims = _dims(x, w)
    ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
    xb = wl.make_x(w)
    A = w.AK / w.K
    x1 = dev_bf16(xb)
    b1 = torch.empty((w.B, w.T), dtype=torch.float32, device="cuda")
    x.block_fwd(x1, Ls, dims, w.N0, w.N1, A, w.K, b1, w.tau, w.delta, ws)
    x2 = dev_bf16(xb)
    b2 = torch.empty((w.B, w.T), dtype=torch.float32, device="cuda")
    _composed(x, w, kinds, Ls, x2, b2, ws, dims)
    torch.cuda.synchronize()
    y1, y2 = host_bits(x1), host_bits(x2)
    assert np.all(np.isfinite(bf16_vals(y1)))
    assert np.array_equal(y1, y2)
    assert np.array_equal(b1.cpu().numpy(), b2.cpu().numpy())
    # The last block's bias counts its selections: each sparse layer picked exactly k tokens
    # per sequence, so the per-token counts sum to AK*k.
    if w.delta > 0 and w.AK > 0:
        steps = [np.float32(0.0)]
        for _ in range(w.AK):
            steps.append(np.float32(steps[-1] + np.float32(w.delta)))
        lut = {float(v): n for n, v in enumerate(steps)}
        bias = b1.cpu().numpy()
        counts = np.vectorize(lambda v: lut[float(v)])(bias)
        assert np.all(counts.sum(axis=1) == w.AK * w.k)


def test_bias_rotation_free_running(x):
    # varsigma = 0 in every sparse layer (x frozen), shared router weights, delta = 1000: the
    # carried bias forces a rotation; every token is chosen exactly AK/K = 2 times per block.
    w = wl.Workload("rot", 33, 2, 1024, 256, 4, 4, 64, 512, 4, N0=0, N1=1, AK=8, delta=1000.0)
    kinds = w.layer_kinds()
    say(f"[rotation] {''.join(kinds)}")
    host = [wl.make_layer(w, l) for l in range(len(kinds))]
    for h in host[:-1]:
        h["w_router"] = host[0]["w_router"]
        h["varsigma"] = 0.0
    dev = [layer_to_device(h) for h in host]
    Ls = [x.make_layer(d) for d in dev]
    dims = _dims(x, w)
    ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
    xb = wl.make_x(w)
    xt = dev_bf16(xb)
    bt = torch.empty((w.B, w.T), dtype=torch.float32, device="cuda")
    x.block_fwd(xt, Ls, dims, w.N0, w.N1, w.AK / w.K, w.K, bt, w.tau, w.delta, ws)
    torch.cuda.synchronize()
    assert np.all(bt.cpu().numpy() == np.float32(2000.0))
    # x after the sparse layers is the input, so only the anchor changed it: compare the
    # free-running block with the oracle's
    ref = oracle.block_forward(xb, host, w, kinds, w.K, tau=w.tau, delta=w.delta)
    check_values(bf16_vals(host_bits(xt)), ref, "rotation block output")
