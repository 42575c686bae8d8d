"""Pins of the oracle's RoPE and of its use in the windowed branches.

Each check compares with a second formulation (complex multiplication by
e^{i p theta}, numpy's complex exponential), a property of the published
definition (theta_0 = 1 and a geometric progression; rotations preserve norms
and invert with -p; scores depend on position differences only), or a
structural identity of the branches (SWA outputs do not move when every
position shifts; DSWA with RoPE equals Eq. 8's literal rearrange followed by
RoPE at the sub-sequence's own positions 0..n-1).  Source: Kairos paper
(arXiv 2606.16533, HTML v3), Sec. 2.2.2; RoFormer (Su et al.), Eq. 13-15.
"""
import numpy as np
import pytest

from oracle import (rope, rope_angles, branch_positions, windowed_attention, dswa_reshape,
                    hlta, frame_index_maps)

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_rope_is_complex_rotation_of_adjacent_pairs():
    rng = np.random.default_rng(1)
    d, base = 16, 10000.0
    x = rng.standard_normal((2, 9, 3, d))
    pos = rng.integers(-50, 5000, 9)
    got = rope(x, pos, base)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    theta = base ** (-np.arange(0, d, 2) / d)
    zr = z * np.exp(1j * pos[None, :, None, None] * theta)
    np.testing.assert_allclose(got[..., 0::2], zr.real, rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(got[..., 1::2], zr.imag, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d,base", [(128, 10000.0), (64, 500.0), (32, 1e6)])
def test_rope_frequencies(d, base):
    """theta_0 = 1 and theta_{i+1} / theta_i = base^(-2/d) (read off position 1)."""
    th = rope_angles(np.array([1]), d, base)[0]
    assert th[0] == 1.0
    np.testing.assert_allclose(th[1:] / th[:-1], base ** (-2.0 / d), rtol=1e-13)
    assert th.shape == (d // 2,)


def test_rope_preserves_pair_norms_and_inverts():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((1, 20, 2, 32))
    pos = np.arange(20) * 37 + 5
    y = rope(x, pos, 10000.0)
    np.testing.assert_allclose(np.hypot(y[..., 0::2], y[..., 1::2]), np.hypot(x[..., 0::2], x[..., 1::2]),
                               rtol=1e-13)
    np.testing.assert_allclose(rope(y, -pos, 10000.0), x, rtol=1e-12, atol=1e-12)
    np.testing.assert_array_equal(rope(x, np.zeros(20, dtype=int), 10000.0), x)


def test_rope_scores_depend_on_position_difference_only():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((1, 1, 1, 64))
    k = rng.standard_normal((1, 1, 1, 64))
    base = 10000.0
    s = lambda m, n: float(np.sum(rope(q, [m], base) * rope(k, [n], base)))
    for m, n, c in [(10, 3, 1000), (0, 7, 12345), (500, 500, -77)]:
        np.testing.assert_allclose(s(m + c, n + c), s(m, n), rtol=1e-9)
        np.testing.assert_allclose(s(m, n), float(np.sum(q * rope(k, [n - m], base))), rtol=1e-9)


def test_branch_positions():
    """SWA positions are absolute token indices; DSWA positions count inside the group."""
    T, L = 12, 3
    np.testing.assert_array_equal(branch_positions(T, L, 1, 2), np.arange(T) + 2 * L)
    np.testing.assert_array_equal(branch_positions(T, L, 2, 0), [0, 1, 2, 0, 1, 2, 3, 4, 5, 3, 4, 5])


@pytest.mark.parametrize("centered", [False, True])
def test_swa_with_rope_ignores_frame_offset(centered):
    """Every SWA position moves by the same amount when the frame offset changes."""
    rng = np.random.default_rng(4)
    q, k, v = (rng.standard_normal((1, 30, 2, 16)) for _ in range(3))
    a = windowed_attention(q, k, v, 5, 9, 1, 0, centered, rope_base=10000.0)
    b = windowed_attention(q, k, v, 5, 9, 1, 7, centered, rope_base=10000.0)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)
    c = windowed_attention(q, k, v, 5, 9, 1, 0, centered)
    assert np.max(np.abs(a - c)) > 1e-3                # RoPE does change the output


@pytest.mark.parametrize("F,dil,fo", [(12, 6, 0), (21, 6, 0), (14, 6, 3), (24, 12, 5)])
@pytest.mark.parametrize("centered", [False, True])
def test_dswa_rope_uses_subsequence_positions(F, dil, fo, centered):
    """DSWA with RoPE == gather each residue group (Eq. 8), then SWA with RoPE
    at the gathered sequence's own positions 0..n-1 (frame offset 0, dil 1)."""
    rng = np.random.default_rng(F + dil + fo)
    L, w, base = 4, 9, 10000.0
    q, k, v = (rng.standard_normal((1, F * L, 2, 16)) for _ in range(3))
    got = windowed_attention(q, k, v, L, w, dil, fo, centered, rope_base=base)

    def swa(qq, kk, vv):
        return windowed_attention(qq, kk, vv, L, w, 1, 0, centered, rope_base=base)
    np.testing.assert_allclose(got, dswa_reshape(q, k, v, L, w, dil, fo, swa=swa), rtol=1e-9,
                               atol=1e-11)


def test_dswa_rope_shift_by_whole_groups():
    """Shifting the frame offset by a multiple of the dilation keeps every
    group and shifts its positions uniformly: the output does not change."""
    rng = np.random.default_rng(5)
    q, k, v = (rng.standard_normal((1, 48, 2, 16)) for _ in range(3))
    a = windowed_attention(q, k, v, 4, 10, 6, 1, rope_base=500.0)
    b = windowed_attention(q, k, v, 4, 10, 6, 13, rope_base=500.0)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-11)


def test_layer_rope_gate_isolation():
    """The hybrid layer with RoPE and gates isolating DSWA is the DSWA branch with RoPE."""
    rng = np.random.default_rng(6)
    B, T, H, d, L = 1, 36, 2, 16, 3
    q, k, v = (rng.standard_normal((B, T, H, d)) for _ in range(3))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    a = np.full((B, T, H), 0.9)
    b = np.full((B, T, H), 0.5)
    gates = np.array([[-800.0] * H, [800.0] * H, [-800.0] * H])    # sigma: exactly 0, 1, 0
    y, _ = hlta(q, k, v, a, b, gates, L, 7, 6, frame_offset=2, rope_base=1000.0)
    np.testing.assert_allclose(y, windowed_attention(q, k, v, L, 7, 6, 2, rope_base=1000.0),
                               rtol=1e-12, atol=1e-12)
