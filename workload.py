"""Seeded synthetic inputs for the X-MoD sparse-depth layer.

This module only draws random tensors and stores them as bfloat16 bit patterns. It holds none
of the layer's arithmetic: the CPU oracle under ``oracle/`` and the HIP library both consume
the arrays it returns, and neither shares any other code.

Every tensor comes from NumPy's PCG64 seeded by ``SeedSequence([seed, layer, tensor_id])``.
fp32 draws are rounded to bf16 (round to nearest even) here, so both sides see identical bf16
values.

Workload shapes follow the layer the X-MoD review describes (Fig. 1(b) and Eq. (7)): hidden
states [B, T, d], a scalar router Linear(d -> 1), GQA attention and a bias-free SwiGLU FFN.
There is no dataset: the pages measure on FineWeb-Edu tokens through trained models, and these
synthetic draws stand in for them.
"""
from __future__ import annotations

import dataclasses
import numpy as np

# Tensor ids used in the seed sequence. Never renumber: stored fixtures depend on them.
T_X, T_BIAS, T_VARSIGMA, T_WR, T_GATTN, T_WQKV, T_WO, T_GFFN, T_WGATE, T_WUP, T_WDOWN, T_SKEW = range(12)
T_DY = 12


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shapes and draw recipe of one synthetic workload."""
    name: str
    seed: int
    B: int
    T: int
    d: int
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    ffn_hidden: int
    K: int                      # token sparsity: each sparse layer keeps floor(T/K) tokens
    N0: int = 0                 # dense prefix layers
    N1: int = 0                 # number of [Sparse(K)] x AK + [Dense] blocks (0: single layer)
    AK: int = 0                 # sparse layers per block (A*K)
    bias_std: float = 0.0       # carried per-token bias b ~ N(0, bias_std) (0: zeros)
    varsigma_range: tuple | None = None   # varsigma ~ U(lo, hi); None: varsigma = 1
    skew_frac: float = 0.0      # fraction of rows scaled by skew_mult (power of two: exact)
    skew_mult: float = 8.0
    weight_std: float = 0.02
    tau: float = 1.0
    delta: float = 0.05
    rms_eps: float = 1e-6
    gain_std: float = 0.0       # RMSNorm gains gamma = 1 + N(0, gain_std) (0: gamma = 1)
    router_bias: float = 0.0

    @property
    def k(self) -> int:
        return self.T // self.K

    @property
    def d_q(self) -> int:
        return self.n_q_heads * self.head_dim

    @property
    def d_kv(self) -> int:
        return self.n_kv_heads * self.head_dim

    @property
    def n_qkv(self) -> int:
        return self.d_q + 2 * self.d_kv

    def layer_kinds(self) -> list[str]:
        """'D'/'S' list of the stack [Dense]xN0 + ([Sparse(K)]xAK + [Dense])xN1; one 'S' if N1 == 0."""
        if self.N1 == 0:
            return ["S"]
        return ["D"] * self.N0 + (["S"] * self.AK + ["D"]) * self.N1


# The five workloads. Sizes are the ones the X-MoD review's hot path is measured on here.
WORKLOADS = {
    # Single Sparse(K=2) layer, small enough for the CPU oracle in seconds.
    "sparse_k2_b2x512_d256": Workload("sparse_k2_b2x512_d256", 1, 2, 512, 256, 4, 4, 64, 1024, 2),
    # Single Sparse(K=8) layer: 512 of 4096 tokens per sequence routed; the throughput workload.
    "sparse_k8_b8x4096_d2048": Workload("sparse_k8_b8x4096_d2048", 2, 8, 4096, 2048, 16, 16, 128,
                                        5632, 8, bias_std=0.1, varsigma_range=(0.5, 1.5)),
    # Original MoD alternation ([Sparse(8)] + [Dense]) x 4.
    "mod_pairs_k8_b4x4096_d1536": Workload("mod_pairs_k8_b4x4096_d1536", 3, 4, 4096, 1536, 12, 12,
                                           128, 4096, 8, N0=0, N1=4, AK=1),
    # X-MoD A3K16 block: Dense prefix x1, then 48 Sparse(16) layers and one Dense anchor.
    "a3k16_block_b4x4096_d1024": Workload("a3k16_block_b4x4096_d1024", 4, 4, 4096, 1024, 8, 8, 128,
                                          2816, 16, N0=1, N1=1, AK=48),
    # Long-context Sparse(K=4) with GQA 32/8, 1% of rows scaled x8 (skewed router).
    "sparse_k4_gqa_b1x32768_d4096": Workload("sparse_k4_gqa_b1x32768_d4096", 5, 1, 32768, 4096, 32,
                                             8, 128, 14336, 4, skew_frac=0.01),
}

# The workload of the benchmark's headline: the largest single-layer workload that fits one GPU.
BENCH_WORKLOAD = "sparse_k4_gqa_b1x32768_d4096"


def rng_for(seed: int, layer: int, tensor_id: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, layer, tensor_id])))


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to bf16 (nearest even) and return the 16-bit patterns (finite input)."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return u.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Widen bf16 bit patterns to fp32 values (exact)."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normal_bf16(seed, layer, tid, shape, std, chunk=1 << 24):
    g = rng_for(seed, layer, tid)
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.uint16)
    for s in range(0, n, chunk):
        e = min(n, s + chunk)
        v = g.standard_normal(e - s, dtype=np.float32) * np.float32(std)
        out[s:e] = f32_to_bf16_bits(v)
    return out.reshape(shape)


def make_x(w: Workload, B: int | None = None, T: int | None = None) -> np.ndarray:
    """Hidden states x ~ N(0,1) as bf16 bits [B, T, d]; a skewed fraction of rows is scaled.

    The scaling multiplies bf16 values by a power of two, so it stays exact.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    x = _normal_bf16(w.seed, 0, T_X, (B, T, w.d), 1.0)
    if w.skew_frac > 0:
        n_rows = int(round(w.skew_frac * B * T))
        rows = rng_for(w.seed, 0, T_SKEW).permutation(B * T)[:n_rows]
        flat = x.reshape(B * T, w.d)
        vals = bf16_bits_to_f32(flat[rows]) * np.float32(w.skew_mult)
        flat[rows] = f32_to_bf16_bits(vals)
    return x


def make_dy(w: Workload, B: int | None = None, T: int | None = None, std: float = 1.0) -> np.ndarray:
    """Upstream gradient of a layer's output, dy ~ N(0, std^2), as bf16 bits [B, T, d]."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    return _normal_bf16(w.seed, 0, T_DY, (B, T, w.d), std)


def make_bias(w: Workload, B: int | None = None, T: int | None = None) -> np.ndarray:
    """Carried per-token bias b as fp32 [B, T]."""
    B = w.B if B is None else B
    T = w.T if T is None else T
    if w.bias_std == 0.0:
        return np.zeros((B, T), dtype=np.float32)
    return (rng_for(w.seed, 0, T_BIAS).standard_normal((B, T), dtype=np.float32)
            * np.float32(w.bias_std)).astype(np.float32)


def make_layer(w: Workload, layer: int) -> dict:
    """Weights of one layer as bf16 bits, PyTorch Linear layout [out, in].

    w_qkv rows are ordered: query heads, then key heads, then value heads.
    """
    s = w.seed
    lay = {
        "w_router": _normal_bf16(s, layer, T_WR, (w.d,), w.weight_std),
        "w_qkv": _normal_bf16(s, layer, T_WQKV, (w.n_qkv, w.d), w.weight_std),
        "w_o": _normal_bf16(s, layer, T_WO, (w.d, w.d_q), w.weight_std),
        "w_gate": _normal_bf16(s, layer, T_WGATE, (w.ffn_hidden, w.d), w.weight_std),
        "w_up": _normal_bf16(s, layer, T_WUP, (w.ffn_hidden, w.d), w.weight_std),
        "w_down": _normal_bf16(s, layer, T_WDOWN, (w.d, w.ffn_hidden), w.weight_std),
        "router_bias": float(w.router_bias),
    }
    for name, tid in (("g_attn", T_GATTN), ("g_ffn", T_GFFN)):
        if w.gain_std == 0.0:
            lay[name] = f32_to_bf16_bits(np.ones(w.d, dtype=np.float32))
        else:
            g = 1.0 + rng_for(s, layer, tid).standard_normal(w.d, dtype=np.float32) * np.float32(w.gain_std)
            lay[name] = f32_to_bf16_bits(g.astype(np.float32))
    if w.varsigma_range is None:
        lay["varsigma"] = 1.0
    else:
        lo, hi = w.varsigma_range
        lay["varsigma"] = float(np.float32(rng_for(s, layer, T_VARSIGMA).uniform(lo, hi)))
    return lay


def scaled(w: Workload, **changes) -> Workload:
    """A copy of a workload with some fields replaced (e.g. smaller B, T for parity tests)."""
    return dataclasses.replace(w, **changes)
