"""Number formats used by the oracle, written from their definitions.

Test infrastructure only: the oracle is a slow, plain fp64 CPU reference.

bf16: 1 sign bit, 8 exponent bits (bias 127), 7 stored mantissa bits; it is
the top half of an IEEE binary32.  Rounding from a wider value is round to
nearest, ties to even, with overflow to infinity.

e4m3fn (OCP 8-bit floating point, "E4M3"): 1 sign bit, 4 exponent bits
(bias 7), 3 mantissa bits, no infinities; exponent 1111 with mantissa 111 is
NaN, so the largest finite value is 1.75 * 2^8 = 448.  Exponent 0000 encodes
subnormals m/8 * 2^-6.

The FP8 KV cache of the DeepSeek-V4-Flash recipe keeps FP8 storage and
converts to BF16 before attention in every phase (page "Finish RL Training
Faster" digest, section "让训练前向使用推理的数值" and its figure caption);
the format choice OCP e4m3fn is the reading for gfx950.
"""
from __future__ import annotations

import numpy as np

BF16_MAX = float(np.float32(3.3895313892515355e38))
E4M3_MAX = 448.0


def _round_to_precision(x: np.ndarray, sig_bits: int, min_normal_exp: int) -> np.ndarray:
    """Round float64 values to a binary format with ``sig_bits`` significant bits
    (implicit bit included) whose smallest normal is 2**min_normal_exp, ties to even.
    No overflow handling (callers do it)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.array(x, dtype=np.float64, copy=True)
    fin = np.isfinite(x) & (x != 0)
    if not np.any(fin):
        return out
    xf = x[fin]
    _, e = np.frexp(xf)               # xf = m * 2**e, 0.5 <= |m| < 1; leading bit 2**(e-1)
    lead = np.maximum(e - 1, min_normal_exp)
    ulp_exp = lead - (sig_bits - 1)
    scaled = np.ldexp(xf, -ulp_exp)    # exact: power-of-two scaling
    out[fin] = np.ldexp(np.rint(scaled), ulp_exp)   # np.rint rounds half to even
    return out


def bf16_round(x) -> np.ndarray:
    """Round-to-nearest-even to bf16, returned as float64 values."""
    y = _round_to_precision(x, 8, -126)
    big = np.isfinite(y) & (np.abs(y) > BF16_MAX)
    y[big] = np.copysign(np.inf, y[big])
    return y


def bf16_encode(x) -> np.ndarray:
    """float values -> uint16 bf16 bit patterns (round to nearest even)."""
    y = bf16_round(x)
    bits = (y.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    bits[np.isnan(y)] = 0x7FC0
    return bits


def bf16_decode(bits) -> np.ndarray:
    """uint16 bf16 bit patterns -> float64 (exact widening)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(np.float64)


def _e4m3_table() -> np.ndarray:
    vals = np.empty(256, dtype=np.float64)
    for code in range(256):
        s = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            vals[code] = np.nan
        elif e == 0:
            vals[code] = s * (m / 8.0) * 2.0 ** -6
        else:
            vals[code] = s * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return vals


E4M3_VALUES = _e4m3_table()


def e4m3_decode(codes) -> np.ndarray:
    """uint8 codes -> float64 values."""
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x) -> np.ndarray:
    """Values -> e4m3fn codes, round to nearest even, saturating at +-448.  NaN -> 0x7F."""
    x = np.asarray(x, dtype=np.float64)
    nan = np.isnan(x)
    xc = np.clip(np.where(nan, 0.0, x), -E4M3_MAX, E4M3_MAX)
    y = _round_to_precision(xc, 4, -6)
    a = np.abs(y)
    code = np.zeros(x.shape, dtype=np.int64)
    sub = (a > 0) & (a < 2.0 ** -6)
    code[sub] = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)        # m / 8 * 2^-6
    nrm = a >= 2.0 ** -6
    _, e = np.frexp(a[nrm])
    ex = e - 1                                                      # a = 1.m * 2**ex
    mant = np.rint((np.ldexp(a[nrm], -ex) - 1.0) * 8.0).astype(np.int64)
    code[nrm] = ((ex + 7) << 3) | mant
    code |= np.where(np.signbit(y), 0x80, 0)
    code[nan] = 0x7F
    return code.astype(np.uint8)
