"""4-bit (FP4 E2M1) quantisation of the windowed branches' Q and K.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: the Kairos project page (Sec. 2, Q2) names FP8 and INT4 attention
quantisation without details.

Readings:

* Format.  The 4-bit path uses OCP FP4 E2M1 codes: 1 sign bit, 2 exponent
  bits (bias 1), 1 mantissa bit; magnitudes 0, 0.5 (subnormal), 1, 1.5, 2, 3,
  4, 6; no infinities or NaN.  The pages say INT4; gfx950's matrix
  instructions take 4-bit floating-point operands but no 4-bit integers, and
  an integer path would need the codes widened to 8 bits in the vector unit
  for every block.  E2M1 keeps the 4-bit storage and the per-block absmax
  scale.
* Scale per (b, h, block of 64 consecutive tokens of the call, all d):
  s = amax / 6 in fp32 (1 when amax = 0), so the block's largest magnitude
  maps to the largest code.  The code is E2M1(fp32(x / s)), round to nearest
  with ties to the even code (mantissa bit 0), saturating at 6.
* Dequantised value x_hat = e2m1_value * s (exact in fp64).
* Packing (for the GPU's byte layout): feature 2i in the low nibble of byte
  i, feature 2i + 1 in the high nibble.
"""
from __future__ import annotations

import numpy as np

E2M1_MAX = 6.0
_MANT_BITS = 1
_MIN_NORMAL_EXP = 0            # smallest normal 2^0; subnormal spacing 2^-1


def e2m1_round(x) -> np.ndarray:
    """Nearest E2M1 value (ties to even code), saturating at +-6; fp64 result."""
    x = np.asarray(x, dtype=np.float64)
    ax = np.abs(x)
    _, E = np.frexp(np.where(ax > 0, ax, 1.0))              # ax = m 2^E, m in [0.5, 1)
    e = np.maximum(E.astype(np.float64) - 1.0, _MIN_NORMAL_EXP)
    quantum = np.exp2(e - _MANT_BITS)                         # spacing inside the binade
    qv = np.rint(ax / quantum) * quantum                      # rint: ties to even multiple
    qv = np.minimum(qv, E2M1_MAX)
    return np.copysign(qv, x)


def e2m1_encode(vals) -> np.ndarray:
    """4-bit codes (uint8, 0..15) of values already on the E2M1 grid."""
    vals = np.asarray(vals, dtype=np.float64)
    sign = np.signbit(vals).astype(np.uint8) << 3
    av = np.abs(vals)
    _, E = np.frexp(np.where(av > 0, av, 1.0))
    e = E.astype(np.int64) - 1
    normal = av >= 1.0
    exp_field = np.where(normal, e + 1, 0)
    # mantissa bit: normal (1 + m/2) 2^e -> m; subnormal m * 0.5 -> m
    mant = np.where(normal, (av / np.exp2(e.astype(np.float64)) - 1.0) * 2.0, av / 0.5)
    code = (exp_field << 1) | np.rint(mant).astype(np.int64)
    code = np.where(av == 0, 0, code)
    return (code.astype(np.uint8) | sign).astype(np.uint8)


def e2m1_decode(codes) -> np.ndarray:
    """Values of 4-bit E2M1 codes."""
    c = np.asarray(codes, dtype=np.int64) & 0xF
    s = (c >> 3) & 1
    e = (c >> 1) & 3
    m = c & 1
    v = np.where(e == 0, m * 0.5, (1.0 + m / 2.0) * np.exp2(e - 1.0))
    return np.where(s == 1, -v, v)


def fp4_pack(codes) -> np.ndarray:
    """[..., d] codes 0..15 -> [..., d/2] bytes (even feature in the low nibble)."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def fp4_unpack(packed) -> np.ndarray:
    p = np.asarray(packed, dtype=np.uint8)
    out = np.empty(p.shape[:-1] + (2 * p.shape[-1],), dtype=np.uint8)
    out[..., 0::2] = p & 0xF
    out[..., 1::2] = p >> 4
    return out


def fp4_quantize_blocks(x, block=64):
    """Quantise ``x`` ``[B, T, H, d]`` (fp32 values) per (b, h, 64-token block).

    Returns ``(codes uint8 [B, T, H, d] (one code per element, unpacked),
    scales float32 [B, H, nblk], xhat float64 [B, T, H, d])``.
    """
    x = np.asarray(x, dtype=np.float32)
    B, T, H, d = x.shape
    nblk = -(-T // block)
    scales = np.empty((B, H, nblk), dtype=np.float32)
    codes = np.empty(x.shape, dtype=np.uint8)
    xhat = np.empty(x.shape, dtype=np.float64)
    for bi in range(nblk):
        s0, s1 = bi * block, min((bi + 1) * block, T)
        xb = x[:, s0:s1]
        amax = np.max(np.abs(xb), axis=(1, 3))
        s = np.where(amax > 0, amax / np.float32(E2M1_MAX), np.float32(1.0)).astype(np.float32)
        scales[:, :, bi] = s
        ratio = (xb / s[:, None, :, None]).astype(np.float32)    # fp32 IEEE division
        qv = e2m1_round(ratio)
        codes[:, s0:s1] = e2m1_encode(qv)
        xhat[:, s0:s1] = qv * s[:, None, :, None].astype(np.float64)
    return codes, scales, xhat
