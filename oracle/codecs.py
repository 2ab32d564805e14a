"""Storage codecs of the oracle (float64 results), from the format definitions.

bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits — the upper
half of an IEEE-754 binary32.  E4M3FN (OCP 8-bit floating point, the "FN"
variant): 1 sign bit, 4 exponent bits (bias 7), 3 fraction bits; exponent 0
holds subnormals m/8·2^-6; S.1111.111 is NaN; there is no infinity; the
largest finite magnitude is 448.  The pages only fix that an FP8 element is
one byte ("vLLM 高性能大语言模型推理引擎深度技术评估与分布式架构展望", the
memory formula under "物理分块与操作系统的分页类比", where S_elem is 1 byte for
FP8); the E4M3FN reading and the per-tensor scale come from the workload
definition of the fp8 cache.

Test infrastructure only (see the package docstring).
"""
from __future__ import annotations

import numpy as np


def bf16_to_f64(bits) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64, field by field."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    sign = np.where(u >> 15, -1.0, 1.0)  # applied with copysign: NaNs keep their sign
    e = (u >> 7) & 0xFF
    m = (u & 0x7F).astype(np.float64)
    with np.errstate(over="ignore", invalid="ignore"):
        normal = np.ldexp(1.0 + m / 128.0, (e - 127).astype(np.int64))
        sub = np.ldexp(m / 128.0, -126)
        val = np.where(e == 0, sub, normal)
        val = np.where(e == 255, np.where(m == 0, np.inf, np.nan), val)
    return np.copysign(val, sign)


def f32_to_f64(bits) -> np.ndarray:
    """Decode binary32 bit patterns (uint32) to float64 (exact)."""
    return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)


def e4m3fn_to_f64(bits) -> np.ndarray:
    """Decode OCP E4M3FN bytes (uint8) to float64, field by field."""
    u = np.asarray(bits, dtype=np.uint8).astype(np.int64)
    sign = np.where(u >> 7, -1.0, 1.0)  # applied with copysign: NaNs keep their sign
    e = (u >> 3) & 0xF
    m = (u & 0x7).astype(np.float64)
    normal = np.ldexp(1.0 + m / 8.0, (e - 7).astype(np.int64))
    sub = np.ldexp(m / 8.0, -6)
    val = np.where(e == 0, sub, normal)
    val = np.where((e == 15) & (m == 7), np.nan, val)
    return np.copysign(val, sign)


# All non-negative finite E4M3FN magnitudes, indexed by their code 0x00..0x7E.
_E4M3_POS = e4m3fn_to_f64(np.arange(0x7F, dtype=np.uint8))
E4M3_MAX = 448.0


def f32_to_e4m3fn(x) -> np.ndarray:
    """Encode float32 values to E4M3FN bytes: clamp to ±448, then round to the
    nearest representable value, ties to the even code (even mantissa).
    NaN encodes to 0x7F with the input's sign bit; ±inf saturates to ±448.

    The clamp-then-round order makes the encoder saturating: no finite input
    becomes NaN.
    """
    x = np.asarray(x, dtype=np.float32)
    neg = np.signbit(x)
    a = np.abs(x.astype(np.float64))
    nan = np.isnan(a)
    a = np.where(nan, 0.0, np.minimum(a, E4M3_MAX))
    # Candidates: the largest code <= a and the one above it.
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first code with value >= a
    hi = np.minimum(hi, len(_E4M3_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _E4M3_POS[lo]
    d_hi = _E4M3_POS[hi] - a
    exact = d_hi == 0
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(exact, hi, np.where(pick_hi, hi, lo)).astype(np.uint8)
    code = np.where(nan, np.uint8(0x7F), code)
    return (code | np.where(neg, np.uint8(0x80), np.uint8(0))).astype(np.uint8)


def quantize_e4m3fn(x_f32, scale_f32) -> np.ndarray:
    """The cache write's fp8 quantiser: the float32 quotient x / scale
    (correctly rounded, as IEEE binary32 division) encoded by ``f32_to_e4m3fn``."""
    x = np.asarray(x_f32, dtype=np.float32)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        qt = x / np.float32(scale_f32)
    return f32_to_e4m3fn(qt)


def decode(bits, dtype: str, scale: float = 1.0) -> np.ndarray:
    """Storage words of ``dtype`` ('f32' | 'bf16' | 'fp8') to float64 values;
    fp8 values are multiplied by their float32 per-tensor scale in float64."""
    if dtype == "f32":
        return f32_to_f64(bits)
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "fp8":
        return e4m3fn_to_f64(bits) * float(np.float32(scale))
    raise ValueError(dtype)
