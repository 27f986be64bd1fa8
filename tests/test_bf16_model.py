"""The bf16-operand model (tests/bf16_model.py) against the oracle, on the CPU.

* Without its roundings the model is the oracle's sparse layer (same selection, same rows), so
  its arithmetic is pinned to the oracle's before its roundings are trusted.
* With them it measures how far bf16 operands alone move the output from the float64 result.
  At the bench layer (d 2048, F 5632) that distance stays inside the stated 2e-2 bar. At the
  long-context GQA layer (d 4096, F 14336, 8192 routed rows) it exceeds 2e-2 on the rows the
  GPU test samples: no implementation with bf16 matrix-core operands can meet 2e-2 there, so
  the GPU test holds that layer to the model's own distance from the oracle plus 2e-2. The
  same holds at the widest hidden state the library takes (d 8192). The relative-L2 bar (5e-3)
  holds for the model at every shape.
* Which values cross a bf16 rounding boundary depends on how the sums before it are taken: the
  same model accumulating in fp32 instead of float64 lands up to about 2e-2 from itself on the
  long-context rows (relative L2 about 1e-3). That is the spread between two bf16-operand
  computations that differ only in summation precision, and it is why the GPU is compared with
  the model in relative L2 only, not element by element at 2e-2.
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
    mods = {}
    for round_p, acc in ((False, np.float64), (True, np.float64), (True, np.float32)):
        mod = bf16_model.sparse_layer_rows(xb, lay, w, w.K, sample=sample, round_p=round_p,
                                           accumulate=acc)
        mods[(round_p, acc)] = mod
        worst, rel = bf16_model.gap(mod, ref["rows"])
        print(f"long-context layer, {len(LONG_ROWS)} sampled rows, P rounded: {round_p}, "
              f"{np.dtype(acc).name} sums: bf16-operand model vs oracle max|diff| {worst:.4g}, "
              f"relL2 {rel:.3g}")
        assert 2e-2 < worst < 8e-2
        assert rel < 5e-3
    a, b = mods[(True, np.float64)], mods[(True, np.float32)]
    spread, rel = bf16_model.gap(b, a)
    print(f"fp32 vs float64 sums in the model: max|diff| {spread:.4g}, relL2 {rel:.3g}")
    assert 1e-3 < spread < 4e-2 and rel < 2e-3


def test_widest_state_model_exceeds_stated_bar():
    """At the widest hidden state (d = 8192, 128 routed rows; the GPU test's workload) the
    bf16-operand roundings alone also move the outputs beyond 2e-2 from the oracle."""
    w = wl.Workload("wide", 28, 1, 256, 8192, 8, 8, 128, 512, 2, bias_std=0.1, gain_std=0.1)
    xb, lay, bias = wl.make_x(w), wl.make_layer(w, 0), wl.make_bias(w)
    sample = {0: np.arange(w.k)}
    ref = oracle.sparse_layer(xb, lay, w, w.K, bias=bias, tau=w.tau, delta=w.delta, sample=sample)
    mod = bf16_model.sparse_layer_rows(xb, lay, w, w.K, bias=bias, tau=w.tau, sample=sample,
                                       round_p=True)
    worst, rel = bf16_model.gap(mod, ref["rows"])
    print(f"widest state: bf16-operand model vs oracle max|diff| {worst:.4g}, relL2 {rel:.3g}")
    assert 2e-2 < worst < 8e-2 and rel < 5e-3
