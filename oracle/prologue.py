"""Input side of the gated delta rule, fp64: key (and optionally query) L2
normalisation, the two sigmoid gates, and the printed-Eq.-6 rescaling.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: Kairos paper (arXiv 2606.16533, HTML v3), Sec. 2.2.1 "Global Pathway":

* Eq. 1 -- the write strength is a sigmoid of a per-token projection,
  beta_t = sigma(z_beta);
* Eq. 4 -- the decay is a sigmoid of a per-token projection,
  alpha_t = sigma(z_alpha);
* Eq. 2-3 -- the delta-rule write and retrieval assume unit keys; the keys
  enter L2-normalised per (token, head).
* Eq. 6 as printed erases with the un-decayed retrieval S_{t-1} k_t.  It is the
  canonical recurrence with rescaled inputs (b' = b / a, v' = a v); the
  ``literal`` switch returns those rescaled inputs.

Readings (the paper is silent on these):

* A zero vector has no direction; it normalises to the zero vector.
* The projections that produce the logits are outside this operator: it
  takes the logits z themselves.
* The query is not normalised unless asked (the read-out of step 4 applies no
  scale to q); normalising it is offered because common gated-delta-rule
  layers normalise both q and k.
"""
from __future__ import annotations

import numpy as np


def l2_normalize(x):
    """x / ||x||_2 over the last axis in fp64; rows that are all zero stay zero.

    The norm is taken after dividing by the row's largest magnitude, so rows
    whose squares would under- or overflow still normalise correctly.
    """
    x = np.asarray(x, dtype=np.float64)
    m = np.max(np.abs(x), axis=-1, keepdims=True)
    safe = np.where(m > 0, m, 1.0)
    y = x / safe
    n = np.sqrt(np.sum(y * y, axis=-1, keepdims=True))
    return np.where(m > 0, y / np.where(n > 0, n, 1.0), 0.0)


def sigmoid(z):
    """1 / (1 + e^{-z}) in fp64 (0 and 1 at the extremes, no NaN)."""
    z = np.asarray(z, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def gdn_prologue(k, alpha_logits, beta_logits, q=None, v=None, literal=False):
    """Prepare the inputs of the canonical gated delta rule.

    k [B, T, H, d] raw keys; alpha_logits, beta_logits [B, T, H] (z of Eq. 4
    and Eq. 1); q [B, T, H, d] raw queries or None (None: not normalised);
    v [B, T, H, d] (needed when ``literal``).

    Returns a dict with ``k`` (unit rows), ``alpha`` = sigma(z_alpha),
    ``beta`` = sigma(z_beta), ``q`` (unit rows, only if q was given) and, when
    ``literal`` is set, ``beta`` = sigma(z_beta) / sigma(z_alpha) and
    ``v`` = sigma(z_alpha) v, so that the canonical recurrence on the returned
    tensors is the printed Eq. 6 on (alpha, beta, v).
    """
    out = {"k": l2_normalize(k)}
    a = sigmoid(alpha_logits)
    b = sigmoid(beta_logits)
    if q is not None:
        out["q"] = l2_normalize(q)
    if literal:
        if v is None:
            raise ValueError("the literal form rescales v: pass v")
        out["beta"] = b / a
        out["v"] = a[..., None] * np.asarray(v, dtype=np.float64)
    else:
        out["beta"] = b
    out["alpha"] = a
    return out
