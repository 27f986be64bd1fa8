"""Mechanism controls of the X-MoD review (section "mechanism controls: conditional capacity vs
attention context", Table 7) on the GPU vs the oracle: the Routed-FFN control's routed FFN
refinement and full-sequence attention block, and the Selected-Q/full-KV layer. Same bar as
the sparse layer (selection swaps only at oracle logit gaps < 1e-5; unselected rows
bit-identical; max |diff| <= 2e-2 + half a bf16 spacing, relative L2 <= 5e-3; a sequence
holding a swap is compared in full against the oracle re-run with the GPU's selection)."""
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


def _run(x, w, xb, lay, bias, entry, ws_id, K):
    dims = _dims(x, w)
    xt = dev_bf16(xb)
    bt = torch.from_numpy(bias.copy()).cuda() if bias is not None else None
    ws = x.alloc_workspace(dims, K, ws_id)
    ws.fill_(255)  # NaN bits: an intermediate the kernels leave unwritten poisons the output
    L = x.make_layer(layer_to_device(lay))
    if entry is None:
        x.attention_layer_fwd(xt, L, dims, ws)
        torch.cuda.synchronize()
        return host_bits(xt), None, None
    idx = torch.empty((w.B, w.T // K), dtype=torch.int32, device="cuda")
    entry(xt, L, dims, K, bt, w.tau, w.delta, ws, idx_out=idx)
    torch.cuda.synchronize()
    return host_bits(xt), idx.cpu().numpy(), None if bt is None else bt.cpu().numpy()


def _check_routed(w, xb, got, ref, what, rerun=None, sample=None):
    """rerun(b, idx_b, sample_b): the oracle on sequence b alone with the given selection; a
    sequence holding a selection swap is compared in full under the GPU's selection."""
    y_bits, idx_g, bias_g = got
    k = w.T // w.K
    first = compare_selection(idx_g, ref["idx"], ref["ell"])
    assert int(np.sum(first < k)) <= max_swapped(w.B)
    sel = np.zeros((w.B, w.T), bool)
    sel[np.arange(w.B)[:, None], idx_g] = True
    assert np.array_equal(y_bits[~sel], xb[~sel]), "unselected rows changed"
    yv = bf16_vals(y_bits)
    for b in range(w.B):
        r, bb, tag = ref, b, f"{what} seq {b}"
        if first[b] < k:
            sb = None if sample is None else {0: sample[b]} if b in sample else {}
            r, bb, tag = rerun(b, idx_g[b:b + 1], sb), 0, tag + " (GPU selection)"
        if bias_g is not None:
            assert np.array_equal(bias_g[b], r["bias_out"][bb]), f"{tag}: carried bias"
        if "rows" in r:
            if bb in r["rows"]:
                prow, pos, ysel = r["rows"][bb]
                assert np.array_equal(pos, idx_g[b, prow])
                check_values(yv[b, pos], ysel, tag + " sampled")
        else:
            check_values(yv[b, idx_g[b]], r["y"][bb, idx_g[b]], tag)


ROUTED = {
    "B2 T512 K2 d256": wl.Workload("rffn_a", 130, 2, 512, 256, 4, 4, 64, 1024, 2, bias_std=0.1,
                                   varsigma_range=(0.5, 1.5)),
    "B2 T2048 K8 d1024 F2816": wl.Workload("rffn_b", 131, 2, 2048, 1024, 8, 8, 128, 2816, 8,
                                           bias_std=0.1, gain_std=0.1),
    # 2000 routed rows x F 8256: 8 x 65 gate/up tiles of 256 x 256 (ragged rows; the last column
    # tile half full),
    # enough for the persistent walk (two or three tiles per workgroup on 256 CUs)
    "B1 T8000 K4 d256 F8256 (persistent SwiGLU tiles)": wl.Workload(
        "rffn_c", 140, 1, 8000, 256, 4, 4, 64, 8256, 4, bias_std=0.1, gain_std=0.1),
}


@pytest.mark.parametrize("name", list(ROUTED))
def test_routed_ffn(x, name):
    w = ROUTED[name]
    say(f"[routed FFN] {name}")
    xb = wl.make_x(w)
    lay = wl.make_layer(w, 0)
    bias = wl.make_bias(w)
    got = _run(x, w, xb, lay, bias, x.routed_ffn_fwd, x.WS_ROUTED_FFN, w.K)
    ref = oracle.routed_ffn_layer(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta)
    _check_routed(w, xb, got, ref, "routed FFN", rerun=lambda b, i, sb: oracle.routed_ffn_layer(
        xb[b:b + 1], lay, w, w.K, bias=bias[b:b + 1], tau=w.tau, delta=w.delta, forced_idx=i))


@pytest.mark.parametrize("w", [
    wl.Workload("attn_a", 132, 2, 300, 256, 4, 2, 64, 512, 1, gain_std=0.1),
    wl.Workload("attn_b", 133, 1, 1024, 1024, 8, 2, 128, 1024, 1)], ids=["B2 T300 d256 GQA", "B1 T1024 d1024 hd128"])
def test_attention_block(x, w):
    say(f"[attention block] {w.name}")
    xb = wl.make_x(w)
    lay = wl.make_layer(w, 0)
    y = _run(x, w, xb, lay, None, None, x.WS_ATTN_LAYER, 1)[0]
    ref = oracle.attention_layer(xb, lay, w)
    check_values(bf16_vals(y), ref, "attention block")


def test_attention_block_with_rope(x):
    w = wl.Workload("attn_r", 134, 2, 500, 512, 8, 2, 64, 1024, 1)
    rng = np.random.default_rng(135)
    lay = dict(wl.make_layer(w, 0), rope_theta=1e4,
               q_norm=wl.f32_to_bf16_bits((1 + 0.2 * rng.standard_normal(64)).astype(np.float32)),
               k_norm=wl.f32_to_bf16_bits((1 + 0.2 * rng.standard_normal(64)).astype(np.float32)))
    say("[attention block] QK-norm + RoPE")
    xb = wl.make_x(w)
    y = _run(x, w, xb, lay, None, None, x.WS_ATTN_LAYER, 1)[0]
    check_values(bf16_vals(y), oracle.attention_layer(xb, lay, w), "attention block + RoPE")


FULLKV = {
    "B2 T512 K2 d256": (wl.Workload("fkv_a", 136, 2, 512, 256, 4, 4, 64, 1024, 2, bias_std=0.1,
                                    varsigma_range=(0.5, 1.5)), {}),
    "B3 T700 K4 d512 GQA 8/2 hd64 (ragged)": (wl.Workload("fkv_b", 137, 3, 700, 512, 8, 2, 64, 1536,
                                                          4, bias_std=0.1, gain_std=0.1), {}),
    "B1 T2048 K8 d1024 GQA 8/2 hd128 + RoPE": (wl.Workload("fkv_c", 138, 1, 2048, 1024, 8, 2, 128,
                                                           2816, 8, bias_std=0.1), {"rope_theta": 1e4}),
    # 16 heads x 4 sequences x 5 q-tiles of 256: more workgroups than CUs (one tile each)
    "B4 T2100 K2 d1024 GQA 16/4 hd64 (ragged, one-tile split)": (
        wl.Workload("fkv_d", 139, 4, 2100, 1024, 16, 4, 64, 1024, 2, bias_std=0.1), {}),
}


@pytest.mark.parametrize("name", list(FULLKV))
def test_selected_q_full_kv(x, name):
    w, extra = FULLKV[name]
    say(f"[Selected-Q/full-KV] {name}")
    xb = wl.make_x(w)
    lay = dict(wl.make_layer(w, 0), **extra)
    bias = wl.make_bias(w)
    got = _run(x, w, xb, lay, bias, x.sparse_layer_fwd_fullkv, x.WS_SPARSE_FULLKV, w.K)
    ref = oracle.sparse_layer_fullkv(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta)
    _check_routed(w, xb, got, ref, "full KV", rerun=lambda b, i, sb: oracle.sparse_layer_fullkv(
        xb[b:b + 1], lay, w, w.K, bias=bias[b:b + 1], tau=w.tau, delta=w.delta, forced_idx=i))


def test_selected_q_full_kv_bench_shape_sampled(x):
    w = wl.WORKLOADS["sparse_k8_b8x4096_d2048"]
    say(f"[Selected-Q/full-KV, full size] {w.name}: oracle on sequences 2 and 7")
    xb = wl.make_x(w)
    lay = wl.make_layer(w, 0)
    bias = wl.make_bias(w)
    got = _run(x, w, xb, lay, bias, x.sparse_layer_fwd_fullkv, x.WS_SPARSE_FULLKV, w.K)
    k = w.T // w.K
    rows = np.concatenate([np.arange(24), np.arange(k - 24, k)])
    sample = {2: rows, 7: rows}
    ref = oracle.sparse_layer_fullkv(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta,
                                     sample=sample)
    _check_routed(w, xb, got, ref, "full KV", sample=sample, rerun=lambda b, i, sb:
                  oracle.sparse_layer_fullkv(xb[b:b + 1], lay, w, w.K, bias=bias[b:b + 1],
                                             tau=w.tau, delta=w.delta, sample=sb, forced_idx=i))
