"""The gate/up GEMM's measured L2 fills equal what its tile order implies.

The SwiGLU product walks 256x256 tiles with one workgroup per CU (256 of them, tile
blockIdx + 256 i at step i). Workgroups reach the 8 XCDs round-robin, the kernel remaps them so
that each XCD owns a contiguous run of tile ids, and then orders those ids in groups of 8 row
blocks. Counting the distinct 256-row blocks of the activations and of the interleaved gate/up
weights each XCD touches per step, times the block's bytes, must reproduce the FETCH_SIZE
counter stored beside the profiles (scaled by the plain copy's factor), within 1 %: every block
is then fetched once per XCD and step and nothing more. The tile order restated here is that of
gemm_kernel's tile_origin; a change to it would show as a mismatch here.
"""
import json
import os

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
PROFILES = os.path.join(ROOT, "profiles")


def tile_origin(t, n_tiles, tiles_m, tiles_n, xcds=8, group=8):
    q, rem = n_tiles // xcds, n_tiles % xcds
    xcd, loc = t % xcds, t // xcds
    wg = xcd * q + min(xcd, rem) + loc
    per_group = group * tiles_n
    first_m = (wg // per_group) * group
    gsz = min(tiles_m - first_m, group)
    return first_m + (wg % per_group) % gsz, (wg % per_group) // gsz


def modelled_fill_bytes(M, F, K, cus=256, xcds=8):
    tiles_m, tiles_n = (M + 255) // 256, (F + 127) // 128  # 128 outputs = 256 B rows per tile
    n_tiles = tiles_m * tiles_n
    block = 256 * K * 2  # one 256-row block of either operand, bf16
    total = 0
    for s0 in range(0, n_tiles, cus):
        for x in range(xcds):
            rows, cols = set(), set()
            for t in range(s0 + x, min(s0 + cus, n_tiles), xcds):
                m, n = tile_origin(t, n_tiles, tiles_m, tiles_n, xcds)
                rows.add(m)
                cols.add(n)
            total += (len(rows) + len(cols)) * block
    return total


def test_tile_origin_is_a_bijection():
    tiles_m, tiles_n = 16, 44
    n = tiles_m * tiles_n
    seen = {tile_origin(t, n, tiles_m, tiles_n) for t in range(n)}
    assert seen == {(m, c) for m in range(tiles_m) for c in range(tiles_n)}


@pytest.mark.parametrize("workload,shape", [
    ("sparse_k4_gqa_b1x32768_d4096", (8192, 14336, 4096)),
    ("sparse_k8_b8x4096_d2048", (4096, 5632, 2048)),
])
def test_gateup_fetch_equals_per_xcd_block_count(workload, shape):
    with open(os.path.join(PROFILES, f"gateup_swiglu_gemm_{workload}_traffic.json")) as f:
        rec = json.load(f)
    measured = rec["fetch_kib_per_dispatch"] * 1024 * rec["fetch_scale"]
    model = modelled_fill_bytes(*shape)
    print(f"{workload}: modelled {model / 1e6:.1f} MB, measured {measured / 1e6:.1f} MB")
    assert abs(measured / model - 1) < 0.01
    # and far above the algorithmic reads: the reuse is per XCD, not per chip
    M, F, K = shape
    assert model > 2 * (M * K + 2 * F * K)
