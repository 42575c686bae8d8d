"""Pins of the oracle's input prologue (key/query L2 normalisation, sigmoid
gates of Eq. 1 and Eq. 4, and the rescaling that turns the printed Eq. 6 into
the canonical recurrence).

Each check compares the oracle with a library routine (torch's normalize,
scipy's expit), an invariant of the definition (unit norm, direction, scale
invariance, sigma(x) + sigma(-x) = 1), a closed form, or a second
formulation (the printed Eq. 6 evaluated token by token).  Source: Kairos
paper (arXiv 2606.16533, HTML v3), Sec. 2.2.1, Eq. 1-6.
"""
import math

import numpy as np
import pytest
import scipy.special
import torch

from oracle import gdn_prologue, l2_normalize, gdn_recurrent, gdn_literal_eq6
from oracle.prologue import sigmoid

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def test_l2_normalize_matches_torch_normalize():
    rng = np.random.default_rng(11)
    x = rng.standard_normal((3, 5, 2, 16)) * rng.uniform(0.1, 10.0, size=(3, 5, 2, 1))
    ref = torch.nn.functional.normalize(torch.from_numpy(x), dim=-1).numpy()
    np.testing.assert_allclose(l2_normalize(x), ref, rtol=1e-14, atol=1e-15)


def test_l2_normalize_unit_norm_and_direction():
    """||y|| = 1 and y . x = ||x|| (equality case of Cauchy-Schwarz: y is x's direction)."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((7, 64))
    y = l2_normalize(x)
    np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-14)
    np.testing.assert_allclose(np.sum(y * x, axis=-1), np.linalg.norm(x, axis=-1), rtol=1e-13)


@pytest.mark.parametrize("c", [1e-200, 1e-30, 3.0, 1e30, 1e200, -2.5])
def test_l2_normalize_scale_invariance(c):
    """normalize(c x) = sign(c) normalize(x), also where the plain sum of
    squares would underflow (1e-200) or overflow (1e200) in fp64."""
    rng = np.random.default_rng(13)
    x = rng.standard_normal((4, 32))
    np.testing.assert_allclose(l2_normalize(c * x), math.copysign(1.0, c) * l2_normalize(x),
                               rtol=1e-13, atol=1e-15)


def test_l2_normalize_special_rows():
    x = np.zeros((3, 8))
    x[1, 3] = -5.0                                 # one non-zero: a signed basis vector
    x[2] = 1.0                                     # all equal: 1/sqrt(d) each
    y = l2_normalize(x)
    assert np.all(y[0] == 0.0)                     # zero stays zero
    assert y[1, 3] == -1.0 and np.count_nonzero(y[1]) == 1
    np.testing.assert_allclose(y[2], 1.0 / math.sqrt(8), rtol=1e-15)


def test_sigmoid_values():
    z = np.linspace(-30, 30, 601)
    np.testing.assert_allclose(sigmoid(z), scipy.special.expit(z), rtol=1e-14)
    np.testing.assert_allclose(sigmoid(z) + sigmoid(-z), 1.0, rtol=1e-14)
    assert sigmoid(0.0) == 0.5
    np.testing.assert_allclose(sigmoid(math.log(3.0)), 0.75, rtol=1e-15)
    assert sigmoid(-800.0) == 0.0 and sigmoid(800.0) == 1.0


def test_decay_from_softplus_parameterisation():
    """exp(-softplus(x)) is the same decay as sigma(-x): the workload's alpha
    parameterisation and Eq. 4's sigmoid agree when z_alpha = -x."""
    x = np.random.default_rng(14).normal(-4.0, 1.0, size=1000)
    np.testing.assert_allclose(np.exp(-np.logaddexp(0.0, x)), gdn_prologue(
        np.ones((1, 1000, 1, 2)), -x.reshape(1, 1000, 1), np.zeros((1, 1000, 1)))["alpha"].ravel(),
        rtol=1e-14)


def _raw(rng, B, T, H, d):
    q = rng.standard_normal((B, T, H, d)) * 3.0
    k = rng.standard_normal((B, T, H, d)) * 3.0
    v = rng.standard_normal((B, T, H, d))
    za = rng.normal(4.0, 1.0, size=(B, T, H))      # sigma(za) mostly 0.9 .. 0.999
    zb = rng.normal(0.0, 1.0, size=(B, T, H))
    return q, k, v, za, zb


def test_literal_prologue_reproduces_printed_eq6():
    """The canonical recurrence on the literal prologue's outputs is Eq. 6 as
    printed, evaluated token by token on (sigma(za), sigma(zb), v)."""
    rng = np.random.default_rng(15)
    q, k, v, za, zb = _raw(rng, 2, 50, 3, 8)
    S0 = rng.standard_normal((2, 3, 8, 8))
    p = gdn_prologue(k, za, zb, q=q, v=v, literal=True)
    o1, S1 = gdn_recurrent(p["q"], p["k"], p["v"], p["alpha"], p["beta"], S0)
    kn = k / np.linalg.norm(k, axis=-1, keepdims=True)
    qn = q / np.linalg.norm(q, axis=-1, keepdims=True)
    o2, S2 = gdn_literal_eq6(qn, kn, v, scipy.special.expit(za), scipy.special.expit(zb), S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=1e-10, atol=1e-12)


def test_literal_prologue_one_token_closed_form():
    """From a zero memory one token writes S_1 = sigma(zb) v khat^T in both
    forms (the rescalings cancel)."""
    rng = np.random.default_rng(16)
    q, k, v, za, zb = _raw(rng, 1, 1, 1, 6)
    p = gdn_prologue(k, za, zb, v=v, literal=True)
    _, S = gdn_recurrent(q, p["k"], p["v"], p["alpha"], p["beta"])
    khat = k[0, 0, 0] / np.linalg.norm(k[0, 0, 0])
    expect = scipy.special.expit(zb[0, 0, 0]) * np.outer(v[0, 0, 0], khat)
    np.testing.assert_allclose(S[0, 0], expect, rtol=1e-13, atol=1e-15)


def test_literal_equals_canonical_without_decay():
    """alpha -> 1 (large z_alpha): the printed and canonical forms coincide, so
    both prologue modes give the same outputs."""
    rng = np.random.default_rng(17)
    q, k, v, _, zb = _raw(rng, 1, 30, 2, 8)
    za = np.full(zb.shape, 60.0)                   # sigma(60) == 1 in fp64
    pc = gdn_prologue(k, za, zb, v=v)
    pl = gdn_prologue(k, za, zb, v=v, literal=True)
    oc, Sc = gdn_recurrent(q, pc["k"], v, pc["alpha"], pc["beta"])
    ol, Sl = gdn_recurrent(q, pl["k"], pl["v"], pl["alpha"], pl["beta"])
    np.testing.assert_array_equal(oc, ol)
    np.testing.assert_array_equal(Sc, Sl)


def test_literal_differs_from_canonical_with_decay():
    """With alpha < 1 and a non-zero memory the two readings differ (the switch
    matters), so a prologue that ignored it would fail the test above it."""
    rng = np.random.default_rng(18)
    q, k, v, za, zb = _raw(rng, 1, 20, 1, 8)
    S0 = rng.standard_normal((1, 1, 8, 8))
    pc = gdn_prologue(k, za, zb, v=v)
    pl = gdn_prologue(k, za, zb, v=v, literal=True)
    oc, _ = gdn_recurrent(q, pc["k"], v, pc["alpha"], pc["beta"], S0)
    ol, _ = gdn_recurrent(q, pl["k"], pl["v"], pl["alpha"], pl["beta"], S0)
    assert np.max(np.abs(oc - ol)) > 1e-3


def test_query_untouched_unless_asked():
    rng = np.random.default_rng(19)
    q, k, v, za, zb = _raw(rng, 1, 4, 1, 8)
    assert "q" not in gdn_prologue(k, za, zb)
    with pytest.raises(ValueError):
        gdn_prologue(k, za, zb, literal=True)
