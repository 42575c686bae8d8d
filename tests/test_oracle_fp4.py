"""Pins of the oracle's 4-bit (OCP FP4 E2M1) quantiser.

The rounding is compared with a brute-force nearest-value search over the
format's representable values (ties to the code with mantissa bit 0) on a
dense set of inputs that contains every midpoint; the code table with the
values the format defines; the block quantiser with its structural
properties (the block maximum maps to the top code, zero blocks, lossless
re-quantisation of its own output) and with the unquantised layer on inputs
that already lie on the grid.
"""
import numpy as np
import pytest

from oracle import (e2m1_round, e2m1_encode, e2m1_decode, fp4_pack, fp4_unpack,
                    fp4_quantize_blocks, hlta)

GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])      # E2M1 magnitudes (OCP MX)


def _brute_round(x):
    """Nearest of +-GRID; ties to the value whose code has mantissa bit 0."""
    vals = np.concatenate([GRID, -GRID[1:]])
    codes = np.concatenate([np.arange(8), 8 + np.arange(1, 8)])
    out = np.empty_like(x)
    for i, xi in enumerate(x):
        if abs(xi) >= 6.0:
            out[i] = np.copysign(6.0, xi)
            continue
        dist = np.abs(vals - xi)
        best = np.flatnonzero(dist == dist.min())
        if len(best) > 1:
            best = [b for b in best if codes[b] % 2 == 0]
        out[i] = vals[best[0]]
    return out


def test_code_table():
    np.testing.assert_array_equal(e2m1_decode(np.arange(8)), GRID)
    np.testing.assert_array_equal(e2m1_decode(np.arange(8, 16)), -GRID)
    np.testing.assert_array_equal(e2m1_encode(GRID), np.arange(8))
    np.testing.assert_array_equal(e2m1_encode(-GRID[1:]), 8 + np.arange(1, 8))


def test_round_matches_bruteforce_including_every_midpoint():
    mids = (GRID[1:] + GRID[:-1]) / 2
    x = np.concatenate([np.linspace(-8, 8, 4001), mids, -mids, np.nextafter(mids, 0),
                        np.nextafter(mids, 10), np.nextafter(-mids, 0), np.nextafter(-mids, -10),
                        [6.0, 6.5, 7.0, 100.0, -7.0, 0.25, -0.25]])
    np.testing.assert_array_equal(e2m1_round(x), _brute_round(x))


def test_round_keeps_sign_of_zero_and_saturates():
    assert np.signbit(e2m1_round(-0.1)) and e2m1_round(-0.1) == 0.0
    assert e2m1_round(1e30) == 6.0 and e2m1_round(-1e30) == -6.0


def test_pack_roundtrip():
    c = np.random.default_rng(1).integers(0, 16, size=(3, 7, 128)).astype(np.uint8)
    p = fp4_pack(c)
    assert p.shape == (3, 7, 64)
    assert p[0, 0, 0] == (c[0, 0, 0] | (c[0, 0, 1] << 4))
    np.testing.assert_array_equal(fp4_unpack(p), c)


def test_block_quantiser_properties():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal((2, 150, 3, 32)) * 5).astype(np.float32)
    x[0, :64, 1] = 0.0                                   # an all-zero block
    codes, scales, xhat = fp4_quantize_blocks(x)
    assert scales.shape == (2, 3, 3)
    assert scales[0, 1, 0] == 1.0 and np.all(codes[0, :64, 1] == 0)
    for b in range(2):
        for h in range(3):
            for bi in range(3):
                blk = x[b, 64 * bi:64 * bi + 64, h]
                amax = np.abs(blk).max()
                if amax == 0:
                    continue
                assert scales[b, h, bi] == np.float32(amax) / np.float32(6.0)
                # the block maximum sits on the top code, within fp32 division
                assert abs(abs(e2m1_decode(codes[b, 64 * bi:64 * bi + 64, h])).max() - 6.0) < 1e-6
    # decoded codes times scales are the dequantised values; re-quantising them is lossless
    deq = e2m1_decode(codes) * np.repeat(np.moveaxis(scales, 2, 1), 64, axis=1)[:, :150, :, None]
    np.testing.assert_array_equal(deq, xhat)
    _, _, xhat2 = fp4_quantize_blocks(xhat.astype(np.float32))
    np.testing.assert_array_equal(xhat2, xhat)


def test_layer_is_lossless_on_grid_inputs():
    """q, k whose blocks are already scaled E2M1 grid values (block max on 6 s):
    the 4-bit layer equals the bf16 layer."""
    rng = np.random.default_rng(3)
    B, T, H, d, L = 1, 128, 2, 16, 32
    def on_grid():
        v = rng.choice(np.concatenate([GRID, -GRID[1:]]), size=(B, T, H, d))
        v[:, ::64, :, 0] = 6.0                          # every block reaches the top code
        return v * 0.25
    q, k = on_grid(), on_grid()
    v = rng.standard_normal((B, T, H, d))
    a = np.full((B, T, H), 0.95)
    b = np.full((B, T, H), 0.5)
    gates = rng.standard_normal((3, H))
    y4, _ = hlta(q, k, v, a, b, gates, L, 40, 2, window_qk="fp4")
    y16, _ = hlta(q, k, v, a, b, gates, L, 40, 2)
    np.testing.assert_allclose(y4, y16, rtol=1e-12, atol=1e-12)
