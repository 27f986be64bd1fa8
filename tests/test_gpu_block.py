"""Stacks of layers: [Dense]xN0 + ([Sparse(K)]xAK + [Dense])xN1 on the GPU.

* Lock-step: the oracle walks the whole stack on its own; every GPU layer is then fed the
  oracle's state at that layer's input (hidden state and carried bias) and compared with the
  oracle's output of that layer. No GPU value ever enters the oracle. Small stacks are walked
  in full; the two stack workloads at their own shapes on one sequence (the oracle's cost),
  with the GPU running the whole batch in the launch configuration the benchmark times.
* A sequence's output does not depend on the batch it runs in (bitwise).
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
                    layer_to_device, max_swapped, say)

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


def check_lockstep_sparse(w, l, lay, e, seqs, y_bits, idx_g, bias_g, xin):
    """One GPU sparse layer fed the oracle's state e (x_in, bias_in) against the oracle's output
    of that layer, on sequences seqs (y_bits, idx_g, bias_g, xin: those sequences' rows). The
    selection follows the swap rule; a sequence holding a swap is compared in full against the
    oracle re-run on the GPU's selection (forced_idx), so every routed row is checked."""
    first = compare_selection(idx_g, e["idx"][seqs], e["ell"][seqs])
    assert int(np.sum(first < w.k)) <= max_swapped(len(seqs)), f"layer {l}: selection swaps"
    sel = np.zeros((len(seqs), w.T), bool)
    sel[np.arange(len(seqs))[:, None], idx_g] = True
    assert np.array_equal(y_bits[~sel], xin[~sel]), f"layer {l}: unselected rows changed"
    for i, b in enumerate(seqs):
        y_ref, b_ref, tag = e["y"][b], e["bias_out"][b], f"layer {l} seq {b}"
        if first[i] < w.k:
            r = oracle.sparse_layer(e["x_in"][b:b + 1], lay, w, w.K, bias=e["bias_in"][b:b + 1],
                                    tau=w.tau, delta=w.delta, forced_idx=idx_g[i:i + 1])
            y_ref, b_ref, tag = r["y"][0], r["bias_out"][0], tag + " (GPU selection)"
        assert np.array_equal(bias_g[i], b_ref), f"{tag}: carried bias"
        check_values(bf16_vals(y_bits[i, idx_g[i]]), y_ref[idx_g[i]], tag)


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
        check_lockstep_sparse(w, l, layers[l], e, np.arange(w.B), host_bits(xt),
                              idx.cpu().numpy(), bt.cpu().numpy(), xin)


FULL_STACKS = ["mod_pairs_k8_b4x4096_d1536", "a3k16_block_b4x4096_d1024"]


@pytest.mark.parametrize("name", FULL_STACKS)
def test_block_lockstep_full_shape(x, name):
    """Lock-step at the stack workloads' own shapes and launch configuration: the oracle walks
    sequence 0 of the workload's inputs through every layer; the GPU runs every layer on the
    whole batch, sequence 0 fed the oracle's hidden state and carried bias at that layer's
    input, the other sequences carrying the GPU's own state from layer to layer. Every layer's
    output for sequence 0 is compared with the oracle's (for the MoD pairs: after each sparse
    and each dense layer, so after each pair; for the A3K16 block: the dense prefix, all 48
    sparse layers and the anchor)."""
    w = wl.WORKLOADS[name]
    kinds = w.layer_kinds()
    say(f"[lock-step, full size] {name}: {''.join(kinds)}; oracle on sequence 0")
    xb = wl.make_x(w)
    layers = [wl.make_layer(w, l) for l in range(len(kinds))]
    _, trace = oracle.block_forward(xb[:1], layers, w, kinds, w.K, tau=w.tau, delta=w.delta,
                                    record=True)
    say(f"    oracle walk done ({len(trace)} layers)")
    dims = _dims(x, w)
    ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
    xt = dev_bf16(xb)
    bt = torch.zeros((w.B, w.T), dtype=torch.float32, device="cuda")
    idx = torch.empty((w.B, w.k), dtype=torch.int32, device="cuda")
    for l, (kind, e) in enumerate(zip(kinds, trace)):
        if l >= w.N0 and (l - w.N0) % (w.AK + 1) == 0:
            bt.zero_()                                   # start of a block (the library's rule)
        xin0 = oracle.f64_to_bf16_bits(e["x_in"])       # [1, T, d]
        xt[0].copy_(dev_bf16(xin0[0]))
        bt[0].copy_(torch.from_numpy(e["bias_in"][0].copy()))
        dl = layer_to_device(layers[l])
        L = x.make_layer(dl)
        if kind == "D":
            x.dense_layer_fwd(xt, L, dims, ws)
            torch.cuda.synchronize()
            check_values(bf16_vals(host_bits(xt[0])), e["y"][0], f"layer {l} (dense) seq 0")
        else:
            x.sparse_layer_fwd(xt, L, dims, w.K, bt, w.tau, w.delta, ws, idx, None)
            torch.cuda.synchronize()
            check_lockstep_sparse(w, l, layers[l], e, np.array([0]), host_bits(xt[:1]),
                                  idx.cpu().numpy()[:1], bt.cpu().numpy()[:1], xin0)
        assert np.all(np.isfinite(bf16_vals(host_bits(xt[1:])))), f"layer {l}: other sequences"
        del dl, L


@pytest.mark.parametrize("name", FULL_STACKS)
def test_block_sequence_independent_of_batch(x, name):
    """A sequence's block output does not depend on the batch it runs in (bitwise): sequence 0
    of the full-batch block equals the block on sequence 0 alone, although the two launch
    different grids (and, for the pairs' dense layers, a different attention work split). With
    the full-batch block equal to the layers called one by one (the next test), the per-sequence
    lock-step above covers every sequence of the full-size block."""
    w = wl.WORKLOADS[name]
    say(f"[batch independence] {name}")
    kinds, _, dev, Ls = _gpu_layers(x, w)
    xb = wl.make_x(w)
    A = w.AK / w.K
    outs = []
    for B in (w.B, 1):
        wb = wl.scaled(w, B=B)
        dims = _dims(x, wb)
        ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
        xt = dev_bf16(xb[:B])
        bt = torch.empty((B, w.T), dtype=torch.float32, device="cuda")
        x.block_fwd(xt, Ls, dims, w.N0, w.N1, A, w.K, bt, w.tau, w.delta, ws)
        torch.cuda.synchronize()
        outs.append((host_bits(xt[:1]), bt[:1].cpu().numpy()))
        del ws
    assert np.array_equal(outs[0][0], outs[1][0])
    assert np.array_equal(outs[0][1], outs[1][1])


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


@pytest.mark.parametrize("name", ["a3k16_block_b4x4096_d1024"])
def test_block_graph_replay_equals_eager(x, name):
    """xmod_block_fwd enqueues kernels only (the bias reset is a fill kernel, not a memset), so
    it can be captured in a HIP graph. Every one of several replays, with eager work and
    synchronisations between them, equals the eager block bit for bit."""
    w = wl.WORKLOADS[name]
    say(f"[graph replay] {name}")
    kinds, _, dev, Ls = _gpu_layers(x, w)
    dims = _dims(x, w)
    ws = x.alloc_workspace(dims, w.K, x.WS_BLOCK)
    xb = wl.make_x(w)
    A = w.AK / w.K
    x0 = dev_bf16(xb)
    xt = x0.clone()
    bt = torch.empty((w.B, w.T), dtype=torch.float32, device="cuda")
    x.block_fwd(xt, Ls, dims, w.N0, w.N1, A, w.K, bt, w.tau, w.delta, ws)
    torch.cuda.synchronize()
    y_eager, b_eager = host_bits(xt), bt.cpu().numpy()
    xt.copy_(x0)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        x.block_fwd(xt, Ls, dims, w.N0, w.N1, A, w.K, bt, w.tau, w.delta, ws)
    for rep in range(3):
        xt.copy_(x0)
        bt.fill_(float(rep + 7))                  # eager work between the replays
        x.sparse_layer_fwd(x0.clone(), Ls[w.N0], dims, w.K, None, w.tau, w.delta, ws)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(xt), y_eager), f"replay {rep}: hidden state"
        assert np.array_equal(bt.cpu().numpy(), b_eager), f"replay {rep}: carried bias"
    del graph
