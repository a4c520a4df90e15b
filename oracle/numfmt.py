"""Exact number-format conversions used by the oracle (fp64 <-> bf16/fp16/fp32).

Storage formats named by the pages: row norms r' are kept in BF16 (OrbitQuant
page, Method); the int8 article stores per-group scales next to the int8
codes (its section 4 pseudo-code), read here as fp16.  All roundings are to
nearest, ties to even, taken directly from float64 (no double rounding).
"""
import numpy as np

_BF16_MAX = float(np.ldexp(255.0, 120))  # (2 - 2^-7) * 2^127


def bf16_bits_to_f64(b):
    """bfloat16 bit patterns (uint16) -> float64, exactly."""
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16
    return u.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """float64 -> bfloat16 bits, round to nearest even, straight from fp64.

    bfloat16 keeps 8 significant bits and float32's exponent range; below
    2^-126 the quantum stays 2^-133 (subnormals).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty(x.shape, dtype=np.uint16)
    flat_x, flat_o = x.reshape(-1), out.reshape(-1)
    nan = np.isnan(flat_x)
    fin = np.isfinite(flat_x)
    xf = np.where(fin, flat_x, 0.0)
    _, e = np.frexp(xf)                       # xf = m * 2^e, 0.5 <= |m| < 1
    q = np.maximum(e - 8, -133)               # exponent of one bf16 ulp
    y = np.ldexp(np.rint(np.ldexp(xf, -q)), q)  # rint rounds half to even
    y = np.where(np.abs(y) > _BF16_MAX, np.copysign(np.inf, xf), y)
    y = np.where(fin, y, flat_x)
    bits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    flat_o[:] = np.where(nan, np.uint16(0x7FC0), bits)
    return out


def f16_bits_to_f64(b):
    """IEEE binary16 bit patterns (uint16) -> float64, exactly."""
    return np.asarray(b, dtype=np.uint16).view(np.float16).astype(np.float64)


def f64_to_f16_bits(x):
    """float64 -> binary16 bits; numpy's double->half cast rounds to nearest even."""
    return np.asarray(x, dtype=np.float64).astype(np.float16).view(np.uint16)


def f64_to_f32(x):
    """float64 -> float32 (nearest even)."""
    return np.asarray(x, dtype=np.float64).astype(np.float32)
