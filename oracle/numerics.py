"""Element-wise numerics of the oracle, all in float64.

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages name the architecture only as a mixture-of-experts transformer
([TR] Experiment, architecture paragraph); the synthetic configurations add
"RMSNorm", "RoPE base 10000" and "SwiGLU".  Readings taken here:
  * RMSNorm: y = x / sqrt(mean(x^2) + eps) with unit gains, eps = 1e-6.
  * RoPE: rotate-half pairs (j, j + D/2), theta_j = base^(-2j/D), angle =
    absolute position * theta_j, applied to queries and keys.
  * SwiGLU: silu(g) * u with silu(x) = x / (1 + exp(-x)).
  * bf16 and OCP e4m3 rounding are round-to-nearest-even; e4m3 saturates at
    +-448 (the fp8 storage of the long-context configuration).
"""
from __future__ import annotations

import numpy as np


def round_bf16(x) -> np.ndarray:
    """Round float64 values to the nearest bfloat16 value (ties to even), returned as float64.

    bf16 keeps 8 significant bits and float32's exponent range (normal
    minimum 2^-126, subnormal step 2^-133, largest finite (2 - 2^-7) * 2^127).
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    a = np.abs(x)
    normal = a >= 2.0 ** -126
    m, e = np.frexp(x[normal])                      # x = m * 2^e, |m| in [0.5, 1)
    out[normal] = np.ldexp(np.rint(np.ldexp(m, 8)), e - 8)
    sub = ~normal
    out[sub] = np.ldexp(np.rint(np.ldexp(x[sub], 133)), -133)
    big = np.abs(out) > (2.0 - 2.0 ** -7) * 2.0 ** 127
    out[big] = np.copysign(np.inf, out[big])
    out[np.isnan(x)] = np.nan
    return out


E4M3_MAX = 448.0


def e4m3_round(x) -> np.ndarray:
    """Round to the nearest OCP e4m3 value (ties to even), saturating at +-448.

    e4m3: 3 mantissa bits, exponent bias 7, normal minimum 2^-6, subnormal
    step 2^-9, largest finite 1.75 * 2^8 = 448.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    _, e = np.frexp(a)                              # a = m * 2^e, m in [0.5, 1)
    e = np.maximum(e - 1, -6)                       # a = 1.f * 2^e for normals
    step = np.ldexp(1.0, e - 3)
    q = np.minimum(np.rint(a / step) * step, E4M3_MAX)
    return np.copysign(q, x)


def e4m3_value_of_code(codes) -> np.ndarray:
    """Decode e4m3 byte codes to float64 (NaN codes 0x7f / 0xff give NaN)."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.ldexp(1.0, e - 7))
    val = np.where((e == 0xF) & ((c & 7) == 7), np.nan, val)
    return sign * val


def e2m1_value_of_code(codes) -> np.ndarray:
    """Decode OCP E2M1 (FP4) codes 0..15 to float64: bit 3 the sign, bits 2-1 the exponent
    (bias 1), bit 0 the mantissa; exponent 0 is subnormal (0 or 0.5)."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    sign = np.where(c & 8, -1.0, 1.0)
    e = (c >> 1) & 3
    m = (c & 1).astype(np.float64)
    val = np.where(e == 0, 0.5 * m, (1.0 + 0.5 * m) * np.ldexp(1.0, e - 1))
    return sign * val


def mxfp4_dequant(codes, scales) -> np.ndarray:
    """Values of an OCP MX FP4 matrix [rows, cols]: codes [rows, cols / 2] (the even column
    in the low nibble), E8M0 scales [rows / 32, cols] (2^(s - 127), one per 32 rows)."""
    c = np.asarray(codes, dtype=np.uint8)
    rows, half = c.shape
    q = np.empty((rows, 2 * half), np.int64)
    q[:, 0::2] = c & 0xF
    q[:, 1::2] = c >> 4
    s = np.ldexp(1.0, np.asarray(scales, np.int64) - 127)            # [rows / 32, cols]
    return e2m1_value_of_code(q) * np.repeat(s, 32, axis=0)


def rmsnorm(x, eps: float = 1e-6) -> np.ndarray:
    """RMSNorm over the last axis with unit gains."""
    x = np.asarray(x, dtype=np.float64)
    return x / np.sqrt(np.mean(x * x, axis=-1, keepdims=True) + eps)


def rope(x, positions, base: float = 10000.0) -> np.ndarray:
    """Rotary embedding, rotate-half form, on the last axis of x [..., n, D]."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[-1]
    half = D // 2
    theta = base ** (-2.0 * np.arange(half, dtype=np.float64) / D)
    ang = np.asarray(positions, dtype=np.float64)[:, None] * theta[None, :]
    c, s = np.cos(ang), np.sin(ang)
    x1, x2 = x[..., :half], x[..., half:]
    return np.concatenate([x1 * c - x2 * s, x2 * c + x1 * s], axis=-1)


def softmax(z, axis: int = -1) -> np.ndarray:
    z = np.asarray(z, dtype=np.float64)
    m = np.max(z, axis=axis, keepdims=True)
    e = np.exp(z - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def silu(x) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    return x / (1.0 + np.exp(-x))
