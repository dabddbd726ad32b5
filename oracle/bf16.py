"""bfloat16 storage rounding for the oracle's matched mode.

bfloat16 keeps float32's 8 exponent bits and 7 stored mantissa bits
[Megatron-LM：张量并行与大规模训练, §5.5 BF16 vs FP16]. The pages state only the
format; rounding is read as IEEE round-to-nearest, ties to even, applied to the
exact (float64) value — one rounding, as an ideal bf16 store would do.
"""
import numpy as np

_BF16_MAX_EXP = 128          # values >= 2**128 after rounding overflow to inf
_BF16_MIN_EXP = -125         # frexp exponent of the smallest normal, 2**-126


def round_to_bf16(x) -> np.ndarray:
    """Nearest bfloat16 value (ties to even) of each float64 entry, as float64.

    frexp gives x = m * 2**e with 0.5 <= |m| < 1; bf16 normals carry 8
    significant bits, so the spacing of representable values around x is
    2**(e-8). Below the normal range the spacing stays 2**(-125-8) (subnormals).
    Division by a power of two is exact, and numpy's rint rounds half to even.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, copy=True)
    fin = np.isfinite(x)
    xf = x[fin]
    _, e = np.frexp(xf)
    q = np.ldexp(1.0, np.maximum(e, _BF16_MIN_EXP) - 8)
    r = np.rint(xf / q) * q
    r = np.where(np.abs(r) >= 2.0 ** _BF16_MAX_EXP, np.copysign(np.inf, r), r)
    out[fin] = r
    return out


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Exact value of bfloat16 bit patterns. A bf16 pattern is the upper half of
    the float32 with the same sign, exponent and leading mantissa bits, so the
    value is read by placing the 16 bits in the top of a 32-bit word."""
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x) -> np.ndarray:
    """Bit pattern of round_to_bf16(x) (finite and infinite values; NaN -> 0x7FC0)."""
    r = round_to_bf16(x)
    out = np.zeros(r.shape, np.uint16)
    neg = np.signbit(r)
    a = np.abs(r)
    nan = np.isnan(r)
    inf = np.isinf(a)
    fin = ~(nan | inf)
    af = a[fin]
    m, e = np.frexp(af)                       # af = m*2**e, m in [0.5, 1)
    is_norm = af >= 2.0 ** -126
    expo = np.where(is_norm, e - 1 + 127, 0)
    mant = np.where(is_norm, np.rint((m * 2.0 - 1.0) * 128.0),
                    np.rint(af / 2.0 ** -133))
    mant = np.where(af == 0, 0, mant)
    bits = (expo.astype(np.int64) << 7) | mant.astype(np.int64)
    out[fin] = bits.astype(np.uint16)
    out[inf] = 0x7F80
    out[nan] = 0x7FC0
    out = np.where(neg & ~nan, out | 0x8000, out).astype(np.uint16)
    return out
