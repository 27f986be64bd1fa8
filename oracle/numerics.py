"""bf16 helpers private to the oracle (test infrastructure only; see oracle/__init__.py).

The oracle computes in float64. The hidden state a layer hands to the next one is stored as
bf16, so the stack walk rounds each layer's output once, to nearest even.
"""
import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Value of each bf16 bit pattern, as float64 (exact)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def round_to_bf16(v) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits. For |v| in [2^(E-1), 2^E) the spacing is 2^(E-8); dividing
    by it is an exact power-of-two scaling, so np.rint (half to even) rounds correctly. The
    smallest normal bf16 exponent is that of fp32 (spacing floor 2^-133).
    """
    v = np.asarray(v, dtype=np.float64)
    assert np.all(np.isfinite(v)), "non-finite value reached bf16 rounding"
    _, e = np.frexp(v)                       # v = m * 2^e with 0.5 <= |m| < 1
    e = np.maximum(e, -125)                  # fp32/bf16 normal range floor
    ulp = np.ldexp(1.0, (e - 8).astype(np.int64))
    out = np.rint(v / ulp) * ulp
    assert np.all(np.abs(out) < 3.3895313892515355e38), "bf16 overflow"
    return out


def f64_to_bf16_bits(v) -> np.ndarray:
    """bf16 bit patterns of values that are already exactly representable in bf16."""
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    return (f.view(np.uint32) >> 16).astype(np.uint16)
