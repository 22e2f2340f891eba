"""bfloat16 codec for the oracle (its own; shares nothing with the HIP path).

bfloat16 is IEEE binary32 truncated to its top 16 bits: 1 sign bit, 8
exponent bits, 7 stored mantissa bits. Every conversion to bf16 in this
build rounds to nearest, ties to even, directly from the float64 value (no
intermediate float32 rounding, which could round twice).
"""
import numpy as np

_MAX_FINITE = (2.0 - 2.0 ** -7) * 2.0 ** 127      # 0x7F7F
_MIN_NORMAL = 2.0 ** -126
_SUBNORMAL_QUANTUM = 2.0 ** -133                  # 2^(-126-7)


def to_f64(bits) -> np.ndarray:
    """bf16 bit patterns (any integer dtype, low 16 bits used) -> float64, exact."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    f32 = (b.astype(np.uint32) << 16).view(np.float32)
    with np.errstate(invalid="ignore"):          # NaN patterns stay NaN
        return f32.astype(np.float64)


def from_f64(x) -> np.ndarray:
    """float64 -> bf16 bit patterns (uint16), round to nearest even.

    Normal range: keep 8 significant bits. frexp gives x = m * 2**e with
    0.5 <= |m| < 1, so m * 2**8 has 8 integer bits and rint (ties to even)
    rounds it exactly. Below the smallest normal the grid is the fixed
    subnormal quantum 2**-133. Overflow past the largest finite value rounds
    to infinity the way IEEE RNE does."""
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.float64)
    finite = np.isfinite(x)
    xf = np.where(finite, x, 0.0)
    m, e = np.frexp(xf)
    normal_val = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub_val = np.rint(xf / _SUBNORMAL_QUANTUM) * _SUBNORMAL_QUANTUM
    val = np.where(np.abs(xf) < _MIN_NORMAL, sub_val, normal_val)
    # a value whose rounding carries past the largest finite bf16 is infinite
    val = np.where(np.abs(val) > _MAX_FINITE, np.copysign(np.inf, xf), val)
    out[...] = np.where(finite, val, x)
    f32 = out.astype(np.float32)              # exact: val has <= 8 significant bits
    bits = (f32.view(np.uint32) >> 16).astype(np.uint16)
    # keep NaN a quiet NaN after truncation
    bits = np.where(np.isnan(x), np.uint16(0x7FC0), bits)
    return bits.astype(np.uint16)


def round_f64(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value, returned as float64."""
    return to_f64(from_f64(x))


def near_tie(x, abs_tol: float = 1e-12) -> np.ndarray:
    """Mask of float64 values within abs_tol of a bf16 rounding midpoint.

    Such a value rounds one way or the other depending on its last few
    float64 bits, so two correct float64 evaluations (different operation
    orders, or sin/cos one ulp apart) may round it to adjacent bf16 values.
    The midpoint on x's side of its nearest bf16 value v lies half a
    spacing from v, the spacing being the gap from v to the next bf16
    magnitude above (|x| > |v|) or below (|x| < |v|)."""
    x = np.asarray(x, dtype=np.float64)
    b = from_f64(x).astype(np.int64)
    v = to_f64(b)
    mag = b & 0x7FFF
    sign = b & 0x8000
    up = np.abs(to_f64(sign | np.minimum(mag + 1, 0x7F80)))
    down = np.abs(to_f64(sign | np.maximum(mag - 1, 0)))
    outward = np.abs(x) > np.abs(v)
    gap = np.where(outward, up - np.abs(v), np.abs(v) - down)
    with np.errstate(invalid="ignore"):
        dist = 0.5 * gap - np.abs(x - v)
        return np.isfinite(x) & (gap > 0) & (dist <= abs_tol)
