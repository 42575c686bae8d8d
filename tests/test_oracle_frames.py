"""Pins of the oracle's frame-aligned quantisation blocks (oracle.quantize_frames,
the "frames" reading of the FP8 / 4-bit 64-token blocks that a streamed
rollout needs), checked without reusing the function's own slicing:

* every scale equals amax / 448 (or / 6) over exactly the tokens of its block,
  found by brute force from the explicit partition (frame f, block i) ->
  rows [f L + 64 i, min(f L + 64 i + 64, (f + 1) L, T));
* with L a multiple of 64 the partition is the token-order one, so the result
  is the token-order quantiser's bit for bit;
* values on the code grid scaled so that each block's maximum maps to the
  largest code come back exactly (so a block that straddled a frame end, or
  leaked a neighbour frame's maximum, would not);
* a large value at the end of one frame leaves the next frame's first scale
  unchanged (it does change it in token order when the block straddles);
* the layer in the "frames" reading equals one call per frame with its
  quantisation done on that frame alone (the streamed form), the windowed
  branches seeing earlier frames' dequantised keys."""
import numpy as np
import pytest

import oracle


def _brute_scales(x, L, qmax):
    B, T, H, d = x.shape
    out = []
    for f0 in range(0, T, L):
        f1 = min(f0 + L, T)
        for b0 in range(f0, f1, 64):
            b1 = min(b0 + 64, f1)
            amax = np.max(np.abs(x[:, b0:b1]), axis=(1, 3))
            out.append(np.where(amax > 0, amax / np.float32(qmax), np.float32(1.0)).astype(np.float32))
    return np.stack(out, axis=2)


@pytest.mark.parametrize("fmt,qmax", [("fp8", 448.0), ("fp4", 6.0)])
@pytest.mark.parametrize("T,L", [(300, 100), (1560 * 2 + 7, 1560), (130, 40), (192, 64)])
def test_frame_scales_brute_force(fmt, qmax, T, L):
    x = np.random.default_rng(T + L).standard_normal((2, T, 3, 32)).astype(np.float32)
    x[:, ::7] *= 30.0
    codes, scales, xhat = oracle.quantize_frames(x, L, fmt)
    np.testing.assert_array_equal(scales, _brute_scales(x, L, qmax))
    assert codes.shape == x.shape and xhat.shape == x.shape


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_frames_equal_tokens_when_64_divides_L(fmt):
    x = np.random.default_rng(7).standard_normal((1, 3 * 128 + 64, 2, 32)).astype(np.float32)
    quant = oracle.fp8_quantize_blocks if fmt == "fp8" else oracle.fp4_quantize_blocks
    a, b = oracle.quantize_frames(x, 128, fmt), quant(x)
    for u, v in zip(a, b):
        np.testing.assert_array_equal(u, v)


def test_frame_blocks_lossless_on_grid():
    """Grid values x = c * s with each block's largest |c| = 448: exact."""
    rng = np.random.default_rng(3)
    T, L = 250, 90
    grid = oracle.e4m3_round(rng.uniform(-400, 400, (1, T, 2, 16)).astype(np.float32))
    for f0 in range(0, T, L):
        for b0 in range(f0, min(f0 + L, T), 64):
            grid[:, b0, :, 0] = 448.0                          # each block's maximum
    s = np.float32(0.125)
    x = (grid * s).astype(np.float32)
    _, scales, xhat = oracle.quantize_frames(x, L, "fp8")
    np.testing.assert_array_equal(scales, np.full(scales.shape, s, np.float32))
    np.testing.assert_array_equal(xhat, x.astype(np.float64))


def test_no_scale_leak_across_frames():
    L, T = 100, 200                                           # block 64..127 straddles in token order
    x = np.ones((1, T, 1, 8), np.float32)
    x[0, 99, 0, 0] = 1000.0                                   # last token of frame 0
    _, s_frames, _ = oracle.quantize_frames(x, L, "fp8")
    _, s_tokens, _ = oracle.fp8_quantize_blocks(x)
    assert s_frames[0, 0, 2] == np.float32(1.0 / 448)         # frame 1, first block: ones only
    assert s_tokens[0, 0, 1] == np.float32(1000.0 / 448)      # token order: the straddling block


@pytest.mark.parametrize("fmt", ["fp8", "fp4"])
def test_layer_frames_reading_equals_per_frame_calls(fmt):
    """Windowed branches of the layer in the "frames" reading, against a
    streamed form built from per-frame quantisation: frame f's queries attend
    over keys whose dequantised values come from quantising each frame alone."""
    B, F, L, H, d, w, dil = 1, 5, 40, 2, 32, 70, 2
    T = F * L
    rng = np.random.default_rng(11)
    q, k, v = (rng.standard_normal((B, T, H, d)).astype(np.float32) for _ in range(3))
    gates = np.array([[30.0] * H, [-30.0] * H, [-30.0] * H])   # SWA only
    alpha = np.full((B, T, H), 0.9, np.float32)
    beta = np.full((B, T, H), 0.5, np.float32)
    y, _ = oracle.hlta(q, k, v, alpha, beta, gates, L, w, dil, window_qk=fmt, qk_blocks="frames")
    quant = oracle.fp8_quantize_blocks if fmt == "fp8" else oracle.fp4_quantize_blocks
    qh = np.concatenate([quant(q[:, f * L:(f + 1) * L])[2] for f in range(F)], axis=1)
    kh = np.concatenate([quant(k[:, f * L:(f + 1) * L])[2] for f in range(F)], axis=1)
    o_gdn, _ = oracle.gdn_recurrent(q, k, v, alpha, beta)
    s = oracle.sigmoid(gates)
    o = oracle.windowed_attention(qh, kh, v, L, w, 1)
    ref = s[0][None, None, :, None] * o + s[2][None, None, :, None] * o_gdn + \
        s[1][None, None, :, None] * oracle.windowed_attention(qh, kh, v, L, w, dil)
    np.testing.assert_allclose(y, ref, rtol=1e-12, atol=1e-12)
