"""bf16 <-> fp64 conversions for the oracle (round-to-nearest-even, exact).

bf16 is IEEE binary32 with the low 16 fraction bits dropped: 8 exponent bits,
7 stored fraction bits. Rounding fp64 -> bf16 here is done in one step on the
exact fp64 value (no intermediate fp32), so it is the correctly rounded result.
"""
import numpy as np

_BF16_MAX = float.fromhex("0x1.fep127")


def bf16_bits_to_f64(u16: np.ndarray) -> np.ndarray:
    """uint16 bf16 bit patterns -> exact fp64 values."""
    u = np.asarray(u16, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def _quantum(x: np.ndarray) -> np.ndarray:
    # x = m * 2**e with m in [0.5, 1): normal bf16 spacing is 2**(e-8); below
    # the smallest normal (2**-126, i.e. e <= -125) the spacing stays 2**-133.
    _, e = np.frexp(x)
    e = np.maximum(e, -125)
    return np.ldexp(1.0, e - 8)


def round_bf16(x) -> np.ndarray:
    """Round fp64 values to the nearest bf16 value, ties to even; returns fp64."""
    x = np.asarray(x, dtype=np.float64)
    q = _quantum(np.where(x == 0, 1.0, x))
    r = np.rint(x / q) * q          # x/q is exact (power-of-two scaling); rint is half-to-even
    r = np.where(np.abs(r) > _BF16_MAX, np.copysign(np.inf, x), r)
    return np.where(np.isfinite(x), r, x)


def f64_to_bf16_bits(x) -> np.ndarray:
    """fp64 -> bf16 bit pattern (uint16), correctly rounded (RNE)."""
    r = round_bf16(x).astype(np.float32)  # exact: every bf16 value is an fp32 value
    return (r.view(np.uint32) >> 16).astype(np.uint16)


def ulp_bf16(x) -> np.ndarray:
    """Spacing of bf16 values at |x| (the unit in the last place)."""
    x = np.abs(np.asarray(x, dtype=np.float64))
    return _quantum(np.where(x == 0, float.fromhex("0x1p-126"), x))
