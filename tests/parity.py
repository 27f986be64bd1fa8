"""Helpers for comparing the HIP path with the oracle (tests only).

Tolerances follow the stated bar for this layer: outputs within max |diff| <= 2e-2 plus half a
bf16 spacing of the expected value (the output format's own rounding), relative L2 <= 5e-3;
selection identical, except swaps between tokens whose oracle logits differ by < 1e-5.
"""
from __future__ import annotations

import numpy as np
import torch

import workload as wl

ABS_TOL = 2e-2
REL_L2_TOL = 5e-3
SWAP_GAP = 1e-5


def say(*a):
    print(*a, flush=True)


def dev_bf16(bits: np.ndarray, device="cuda") -> torch.Tensor:
    """Upload bf16 bit patterns as a torch.bfloat16 device tensor."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(device)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.detach().view(torch.int16).cpu().numpy().view(np.uint16)


def bf16_vals(bits: np.ndarray) -> np.ndarray:
    return wl.bf16_bits_to_f32(bits).astype(np.float64)


def ulp_bf16(v: np.ndarray) -> np.ndarray:
    """Spacing of bf16 numbers at |v| (8 significant bits)."""
    a = np.maximum(np.abs(np.asarray(v, dtype=np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def layer_to_device(lay: dict, device="cuda") -> dict:
    out = {}
    for k, v in lay.items():
        out[k] = dev_bf16(v, device) if isinstance(v, np.ndarray) else v
    return out


def check_values(got: np.ndarray, ref: np.ndarray, what: str, abs_tol=ABS_TOL, rel_tol=REL_L2_TOL):
    """got: GPU values (float64 of bf16); ref: oracle float64 values."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert got.shape == ref.shape, (what, got.shape, ref.shape)
    assert np.all(np.isfinite(got)), f"{what}: non-finite output"
    diff = np.abs(got - ref)
    bound = abs_tol + 0.5 * ulp_bf16(ref)
    worst = np.unravel_index(np.argmax(diff - bound), diff.shape)
    rel = np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-30)
    say(f"    {what}: max|diff| {diff.max():.4g}, worst excess over bound {np.max(diff - bound):.3g}, "
        f"relL2 {rel:.3g}")
    assert np.all(diff <= bound), (f"{what}: max|diff|={diff.max():.3g} exceeds bound at {worst}: "
                                   f"got {got[worst]} ref {ref[worst]}")
    assert rel <= rel_tol, f"{what}: relative L2 {rel:.3g} > {rel_tol}"
    return float(diff.max()), float(rel)


def max_swapped(B: int) -> int:
    """Most sequences of a batch that may hold a selection swap: near-ties within 1e-5 are rare
    (about 1-2 % of the synthetic sequences), so more than a quarter means a broken selection."""
    return max(1, B // 4)


def compare_selection(idx_gpu: np.ndarray, idx_ref: np.ndarray, ell_ref: np.ndarray):
    """Check the swap rule; return, per sequence, the first packed position whose selection
    (and therefore attention context) may differ (k if the selections agree)."""
    B, k = idx_ref.shape
    assert idx_gpu.shape == (B, k)
    first_diff = np.full(B, k, dtype=np.int64)
    for b in range(B):
        g, r = idx_gpu[b], idx_ref[b]
        assert np.all(np.diff(g) > 0), f"seq {b}: GPU idx not strictly ascending"
        if np.array_equal(g, r):
            continue
        dropped = np.setdiff1d(r, g)
        added = np.setdiff1d(g, r)
        assert len(dropped) == len(added)
        for i in dropped:
            for j in added:
                gap = abs(float(ell_ref[b, i]) - float(ell_ref[b, j]))
                assert gap < SWAP_GAP, f"seq {b}: swap {i}<->{j} with logit gap {gap:.3g}"
        first_diff[b] = int(np.argmax(g != r))
    return first_diff
