"""Storage formats of the KV cache, decoded to float64 (oracle; test infrastructure).

KV-cache quantization stores keys and values in 8 bits with one float scale
per attention head and dequantises inside the attention kernel
("TensorRT-LLM框架解析与高性能推理优化实践", §7.2 KV Cache量化).  The pages name
FP8 without fixing the flavour; the scale "amax/448" of the workload implies
the OCP e4m3fn format (largest finite value 448, no infinities, NaN = S.1111.111).

bf16 is the upper half of an IEEE float32.  fp32 is exact in float64.
"""
from __future__ import annotations

import numpy as np


# ---------------------------------------------------------------- bf16 ------
def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> float64: the float32 whose top half they are."""
    u = np.asarray(bits).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return u.view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- fp8 -------
def e4m3fn_value(code: int) -> float:
    """Value of one OCP e4m3fn byte ``s eeee mmm`` (exponent bias 7).

    e == 0           : (-1)^s * 2^-6 * m/8          (zero and subnormals)
    e == 15, m == 7  : NaN                           (the only non-finite code)
    otherwise        : (-1)^s * 2^(e-7) * (1 + m/8)
    """
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    sign = -1.0 if s else 1.0
    if e == 0:
        return sign * (2.0 ** -6) * (m / 8.0)
    if e == 15 and m == 7:
        return float("nan")
    return sign * (2.0 ** (e - 7)) * (1.0 + m / 8.0)


E4M3FN_TABLE = np.array([e4m3fn_value(c) for c in range(256)], dtype=np.float64)
E4M3FN_MAX = 448.0
# Non-negative finite codes 0x00..0x7E in increasing order of value.
_POS_CODES = np.arange(0x7F, dtype=np.int64)
_POS_VALUES = E4M3FN_TABLE[:0x7F]


def e4m3fn_to_f64(codes: np.ndarray) -> np.ndarray:
    """fp8 e4m3fn bytes -> float64 by table lookup."""
    return E4M3FN_TABLE[np.asarray(codes, dtype=np.uint8).astype(np.int64)]


def f32_to_e4m3fn(x: np.ndarray) -> np.ndarray:
    """float32 -> e4m3fn bytes: nearest value, ties to the even code, saturating.

    Magnitudes at or above 448 become 448 (so rounding never overflows to NaN);
    NaN stays NaN (0x7F with the sign); the sign of zero and of values that
    round to zero is kept.  Nearest is found by searching the sorted table of
    the 127 non-negative finite values, which is the definition itself.
    """
    x = np.asarray(x, dtype=np.float32)
    a = np.abs(x.astype(np.float64))
    neg = np.signbit(x)
    nan = np.isnan(x)
    a_safe = np.where(nan, 0.0, np.minimum(a, E4M3FN_MAX))
    hi = np.searchsorted(_POS_VALUES, a_safe, side="left")      # first value >= a
    hi = np.clip(hi, 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a_safe - _POS_VALUES[lo]
    d_hi = _POS_VALUES[hi] - a_safe
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (_POS_CODES[hi] % 2 == 0))
    code = np.where(pick_hi, _POS_CODES[hi], _POS_CODES[lo])
    code = np.where(a_safe == _POS_VALUES[hi], _POS_CODES[hi], code)
    code = np.where(nan, 0x7F, code)
    code = code | np.where(neg, 0x80, 0)
    return code.astype(np.uint8)


# ------------------------------------------------------------------ int8 ----
# Symmetric INT8 KV codes with one scale per KV head
# ("TensorRT-LLM框架解析与高性能推理优化实践" §7.2: a scale per attention head, from
# the data's statistics; "4. TensorRT-LLM架构与核心组件…" §4.3: the KV-cache
# quantization plugin stores INT8 or FP8).  Reading: the code of a value x is
# the float32 quotient x / scale rounded to the nearest integer, ties to even,
# saturated to [-127, 127] (symmetric: -128 is never produced); NaN encodes
# as 0.  A code c stands for c * scale.
INT8_MAX = 127


def f32_to_int8_sym(q: np.ndarray) -> np.ndarray:
    """Code of float32 quotients q = x / scale (already divided)."""
    q = np.asarray(q, dtype=np.float32).astype(np.float64)     # exact widening
    r = np.clip(np.rint(q), -INT8_MAX, INT8_MAX)                # rint: ties to even
    return np.where(np.isnan(q), 0.0, r).astype(np.int8)


def int8_to_f64(codes: np.ndarray) -> np.ndarray:
    return np.asarray(codes, dtype=np.int8).astype(np.float64)
