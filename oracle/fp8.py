"""FP8 E4M3 quantisation of the windowed branches' Q and K.

Source: the Kairos project page (zhaifeiyue.github.io, "Kairos: A Native
World Model Stack for Physical AI", Sec. 1 TL;DR and Sec. 2 Q2) names FP8/INT4 attention
quantisation without details; the workload fixes e4m3 with one absmax scale
per 64-token block.

Readings:

* Format: OCP FP8 E4M3 ("fn"): 1 sign, 4 exponent bits (bias 7), 3 mantissa
  bits, subnormals, no infinities, largest finite 448.
* Rounding: round to nearest, ties to even; values beyond 448 saturate to 448.
* Scale per (b, h, block of 64 consecutive tokens of the call, all d):
  s = amax / 448 computed in fp32 (s = 1 when amax = 0), not rounded to a
  power of two.  The quantised code is e4m3(fp32(x / s)); the division is an
  fp32 IEEE division (this decides the code, so both sides use fp32).
* Dequantised value x_hat = e4m3_value * s (exact in fp64).
"""
from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
_MIN_NORMAL_EXP = -6          # 2^-6 smallest normal
_MANT_BITS = 3


def e4m3_round(x) -> np.ndarray:
    """Nearest e4m3 value (ties to even), saturating at +-448; fp64 result."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    # exponent of the binade (ax = m 2^E with m in [0.5, 1), so e = E - 1),
    # clamped below at the subnormal range
    _, E = np.frexp(np.where(ax > 0, ax, 1.0))
    e = np.maximum(E.astype(np.float64) - 1.0, _MIN_NORMAL_EXP)
    quantum = np.exp2(e - _MANT_BITS)            # spacing of representable values
    # float64 division by a power of two is exact; np.rint is ties-to-even
    qv = np.rint(ax / quantum) * quantum
    qv = np.minimum(qv, E4M3_MAX)
    return np.copysign(qv, x)          # keeps the sign of zero, as the format does


def e4m3_encode(vals) -> np.ndarray:
    """Bit patterns (uint8) of values already on the e4m3 grid."""
    vals = np.asarray(vals, dtype=np.float64)
    sign = (np.signbit(vals)).astype(np.uint8) << 7
    av = np.abs(vals)
    _, E = np.frexp(np.where(av > 0, av, 1.0))
    e = E.astype(np.int64) - 1
    normal = av >= 2.0 ** _MIN_NORMAL_EXP
    exp_field = np.where(normal, e + 7, 0)
    mant = np.where(normal, av / np.exp2(e.astype(np.float64)) - 1.0, av / 2.0 ** _MIN_NORMAL_EXP) * 8.0
    mant = np.rint(mant).astype(np.int64)
    code = (exp_field << 3) | mant
    code = np.where(av == 0, 0, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e4m3_decode(codes) -> np.ndarray:
    """Values of e4m3 bit patterns (0x7F / 0xFF are NaN in this format)."""
    c = np.asarray(codes, dtype=np.int64)
    s = (c >> 7) & 1
    e = (c >> 3) & 0xF
    m = c & 7
    v = np.where(e == 0, m / 8.0 * 2.0 ** _MIN_NORMAL_EXP, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    v = np.where((c & 0x7F) == 0x7F, np.nan, v)
    return np.where(s == 1, -v, v)


def fp8_quantize_blocks(x, block=64):
    """Quantise ``x`` ``[B, T, H, d]`` (fp32 values) per (b, h, 64-token block).

    Returns ``(codes uint8 [B, T, H, d], scales float32 [B, H, nblk],
    xhat float64 [B, T, H, d])`` with nblk = ceil(T / 64).
    """
    x = np.asarray(x, dtype=np.float32)
    B, T, H, d = x.shape
    nblk = -(-T // block)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    xhat = np.empty(x.shape, dtype=np.float64)
    for bi in range(nblk):
        s0, s1 = bi * block, min((bi + 1) * block, T)
        xb = x[:, s0:s1]                                    # [B, n, H, d]
        amax = np.max(np.abs(xb), axis=(1, 3))              # [B, H] (exact: a max)
        s = np.where(amax > 0, amax / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, :, bi] = s
        ratio = (xb / s[:, None, :, None]).astype(np.float32)   # fp32 IEEE division
        qv = e4m3_round(ratio)
        codes[:, s0:s1] = e4m3_encode(qv)
        xhat[:, s0:s1] = qv * s[:, None, :, None].astype(np.float64)
    return codes, scales, xhat
