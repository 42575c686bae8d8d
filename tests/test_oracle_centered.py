"""Pins of the oracle's centred windows (Eq. 7 as printed, radius
floor(w / 2) on both sides, itself included) for SWA and DSWA.

Each check compares with a library routine (torch scaled-dot-product
attention, unmasked or with an explicit band mask), a symmetry of the
definition (reversing the sequence), the scalar brute force, or the literal
rearrange of Eq. 8.  Source: Kairos paper (arXiv 2606.16533, HTML v3),
Sec. 2.2.2, Eq. 7-8; dilations 6 and 12 as named there.
"""
import math

import numpy as np
import pytest
import torch

from oracle import windowed_attention, windowed_attention_rows, window_bruteforce, dswa_reshape, hlta

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _qkv(rng, B, T, H, d):
    return (rng.standard_normal((B, T, H, d)) for _ in range(3))


def _sdpa(q, k, v, mask=None):
    t = lambda x: torch.from_numpy(np.ascontiguousarray(np.moveaxis(x, 2, 1)))   # [B, H, T, d]
    m = None if mask is None else torch.from_numpy(mask)
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), attn_mask=m)
    return np.moveaxis(o.numpy(), 1, 2)


def test_centered_wide_window_is_full_attention():
    """Radius >= T: every query sees every key (bidirectional attention)."""
    rng = np.random.default_rng(1)
    q, k, v = _qkv(rng, 2, 40, 2, 16)
    got = windowed_attention(q, k, v, 10, 80, centered=True)
    np.testing.assert_allclose(got, _sdpa(q, k, v), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("w", [2, 7, 10, 31])
def test_centered_band_matches_masked_library_attention(w):
    """The band |i - j| <= floor(w/2) as an explicit boolean mask for torch's attention."""
    rng = np.random.default_rng(w)
    T = 53
    q, k, v = _qkv(rng, 1, T, 3, 8)
    i = np.arange(T)
    band = np.abs(i[:, None] - i[None, :]) <= w // 2
    got = windowed_attention(q, k, v, 11, w, centered=True)
    np.testing.assert_allclose(got, _sdpa(q, k, v, band), rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("w", [0, 1])
def test_centered_zero_radius_returns_values(w):
    rng = np.random.default_rng(3)
    q, k, v = _qkv(rng, 1, 20, 2, 8)
    np.testing.assert_allclose(windowed_attention(q, k, v, 5, w, dil=3, centered=True), v,
                               rtol=1e-14, atol=1e-14)


@pytest.mark.parametrize("L,F,w,dil", [(6, 12, 9, 1), (6, 12, 14, 6), (4, 12, 9, 12), (5, 8, 12, 4)])
def test_centered_reversal_symmetry(L, F, w, dil):
    """Reversing the token order (F divisible by dil keeps every group's
    positions reversed) maps a centred window onto itself, so the output is
    the reversed output.  A one-sided error in the band fails this."""
    rng = np.random.default_rng(L + F + w)
    q, k, v = _qkv(rng, 1, F * L, 2, 8)
    o = windowed_attention(q, k, v, L, w, dil, centered=True)
    rev = lambda x: x[:, ::-1]
    o_rev = windowed_attention(rev(q), rev(k), rev(v), L, w, dil, centered=True)
    np.testing.assert_allclose(rev(o_rev), o, rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("T,L,w,dil,fo", [(23, 4, 5, 1, 0), (30, 3, 4, 6, 0), (26, 2, 3, 12, 5),
                                          (21, 3, 6, 4, 2)])
def test_centered_blocked_equals_bruteforce(T, L, w, dil, fo):
    """Blocked evaluation == scalar loops, including ragged groups, a partial
    last frame and a non-zero absolute frame offset."""
    rng = np.random.default_rng(T * w)
    q, k, v = _qkv(rng, 1, T, 2, 4)
    np.testing.assert_allclose(windowed_attention(q, k, v, L, w, dil, fo, centered=True),
                               window_bruteforce(q, k, v, L, w, dil, fo, centered=True),
                               rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("F,dil,fo", [(12, 6, 0), (24, 12, 0), (21, 6, 0), (14, 6, 3)])
def test_centered_dswa_equals_literal_rearrange(F, dil, fo):
    """Mask form of DSWA == Eq. 8's gather-into-groups then centred SWA."""
    rng = np.random.default_rng(F + dil)
    L, w = 4, 7
    q, k, v = _qkv(rng, 1, F * L, 2, 8)
    np.testing.assert_allclose(windowed_attention(q, k, v, L, w, dil, fo, centered=True),
                               dswa_reshape(q, k, v, L, w, dil, fo, centered=True),
                               rtol=1e-11, atol=1e-12)


def test_centered_dilation_one_is_swa():
    rng = np.random.default_rng(9)
    q, k, v = _qkv(rng, 1, 30, 2, 8)
    a = windowed_attention(q, k, v, 5, 9, 1, centered=True)
    b = windowed_attention(q, k, v, 30, 9, 1, centered=True)     # frame length is irrelevant
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-14)


def test_centered_rows_equal_full():
    rng = np.random.default_rng(10)
    q, k, v = _qkv(rng, 2, 60, 2, 8)
    rows = np.array([0, 1, 17, 29, 30, 59])
    full = windowed_attention(q, k, v, 10, 13, 6, centered=True)
    np.testing.assert_allclose(windowed_attention_rows(q, k, v, rows, 10, 13, 6, centered=True),
                               full[:, rows], rtol=1e-13, atol=1e-14)


def test_centered_sees_the_future_causal_does_not():
    """Changing the last token's value changes centred outputs within the
    radius before it and no causal output before it."""
    rng = np.random.default_rng(11)
    q, k, v = _qkv(rng, 1, 30, 1, 8)
    v2 = v.copy()
    v2[0, -1] += 1.0
    c1 = windowed_attention(q, k, v, 10, 8, centered=True)
    c2 = windowed_attention(q, k, v2, 10, 8, centered=True)
    changed = np.abs(c1 - c2).max(axis=(0, 2, 3)) > 0
    assert changed.tolist() == [t >= 30 - 1 - 4 for t in range(30)]
    k1 = windowed_attention(q, k, v, 10, 8)
    k2 = windowed_attention(q, k, v2, 10, 8)
    assert np.array_equal(k1[:, :-1], k2[:, :-1])


def test_centered_layer_gate_isolation():
    """The hybrid layer with z = (+40, -40, -40) is the centred SWA branch."""
    rng = np.random.default_rng(12)
    B, T, H, d, L = 1, 24, 2, 8, 4
    q, k, v = _qkv(rng, B, T, H, d)
    a = np.full((B, T, H), 0.9)
    b = np.full((B, T, H), 0.5)
    gates = np.array([[40.0] * H, [-40.0] * H, [-40.0] * H])
    y, _ = hlta(q, k, v, a, b, gates, L, 6, 6, centered=True)
    np.testing.assert_allclose(y, windowed_attention(q, k, v, L, 6, 1, centered=True),
                               rtol=1e-12, atol=1e-12)
