"""The bf16-operand model (tests/bf16_model.py) against the oracle, on the CPU.

* Without its roundings the model is the oracle's sparse layer (same selection, same rows), so
  its arithmetic is pinned to the oracle's before its roundings are trusted.
* With them it measures how far bf16 operands alone move the output from the float64 result.
  At the bench layer (d 2048, F 5632) that distance stays inside the stated 2e-2 bar. At the
  long-context GQA layer (d 4096, F 14336, 8192 routed rows) it exceeds 2e-2 on the rows the
  GPU test samples: no implementation with bf16 matrix-core operands can meet 2e-2 there, so
  the GPU test compares that layer with this model at 2e-2 and with the oracle at the model's
  own distance plus 2e-2. The relative-L2 bar (5e-3) holds for the model at both shapes.
"""
import numpy as np
import pytest

import bf16_model
import oracle
import workload as wl

# The rows the long-context GPU test samples: the first 48 packed rows, 16 in the middle and
# the last 64 (which see every routed row as keys).
LONG_ROWS = np.concatenate([np.arange(0, 48), np.arange(4090, 4106), np.arange(8192 - 64, 8192)])


def test_model_without_rounding_is_the_oracle():
    w = wl.scaled(wl.WORKLOADS["sparse_k2_b2x512_d256"], seed=41, gain_std=0.2, router_bias=0.3,
                  bias_std=0.1, varsigma_range=(0.5, 1.5))
    xb, lay, bias = wl.make_x(w), wl.make_layer(w, 0), wl.make_bias(w)
    ref = oracle.sparse_layer(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta)
    mod = bf16_model.sparse_layer_rows(xb, lay, w, w.K, bias=bias, tau=w.tau, rounding=False,
                                       round_p=True)
    for b, (prow, pos, y) in mod.items():
        assert np.array_equal(pos, ref["idx"][b])
        assert np.max(np.abs(y - ref["y"][b, pos])) < 1e-12
    # with the roundings the model moves, but stays close at this small shape
    mod_r = bf16_model.sparse_layer_rows(xb, lay, w, w.K, bias=bias, tau=w.tau)
    ref_rows = {b: (np.arange(w.k), ref["idx"][b], ref["y"][b, ref["idx"][b]]) for b in range(w.B)}
    worst, rel = bf16_model.gap(mod_r, ref_rows)
    assert 0 < worst < 2e-2 and rel < 5e-3


@pytest.mark.slow
def test_bench_layer_model_within_stated_bar():
    w = wl.WORKLOADS["sparse_k8_b8x4096_d2048"]
    xb, lay, bias = wl.make_x(w), wl.make_layer(w, 0), wl.make_bias(w)
    sample = {0: np.arange(w.k)}
    ref = oracle.sparse_layer(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta, sample=sample)
    mod = bf16_model.sparse_layer_rows(xb, lay, w, w.K, bias=bias, tau=w.tau, sample=sample,
                                       round_p=True)
    worst, rel = bf16_model.gap(mod, ref["rows"])
    print(f"bench layer, sequence 0: bf16-operand model vs oracle max|diff| {worst:.4g}, "
          f"relL2 {rel:.3g}")
    assert worst < 2e-2 and rel < 5e-3


@pytest.mark.slow
def test_long_context_model_exceeds_stated_bar():
    w = wl.WORKLOADS["sparse_k4_gqa_b1x32768_d4096"]
    xb, lay = wl.make_x(w), wl.make_layer(w, 0)
    sample = {0: LONG_ROWS}
    ref = oracle.sparse_layer(xb, lay, w, w.K, sample=sample)
    for round_p in (False, True):
        mod = bf16_model.sparse_layer_rows(xb, lay, w, w.K, sample=sample, round_p=round_p)
        worst, rel = bf16_model.gap(mod, ref["rows"])
        print(f"long-context layer, {len(LONG_ROWS)} sampled rows, P rounded: {round_p}: "
              f"bf16-operand model vs oracle max|diff| {worst:.4g}, relL2 {rel:.3g}")
        assert 2e-2 < worst < 8e-2
        assert rel < 5e-3
