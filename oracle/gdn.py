"""Gated delta rule (GatedDeltaNet) forward, fp64, token by token.

Source: Kairos paper (arXiv 2606.16533, HTML v3), Sec. 2.2.1 "Global Pathway:
Gated Linear Attention as Persistent Causal Memory", Eq. 1-6 and step 4
(output generation from the *updated* memory).

Layouts: q, k, v ``[B, T, H, d]``; alpha, beta ``[B, T, H]``; the memory
``S`` is ``[B, H, dv, dk]`` (the paper's S_t lives in R^{dv x dk}, Eq. 2).

Readings (the paper is ambiguous or silent on these):

* Decay placement.  The canonical gated delta rule used throughout this
  project is ``S_t = a_t S_{t-1} (I - b_t k_t k_t^T) + b_t v_t k_t^T``: the
  retrieval that is erased is taken from the *decayed* memory.  Eq. 5/6 as
  printed erase with the un-decayed retrieval ``S_{t-1} k_t``;
  ``gdn_literal_eq6`` implements that form, and the two are related by the
  exact identity literal(a, b, v) == canonical(a, b/a, a v) (tested).
* Read-out: ``o_t = S_t q_t`` with the updated state, no scaling of q.
* Keys arrive L2-normalised; nothing here renormalises them.
* alpha, beta arrive as the gate values themselves (Eq. 1 and Eq. 4 apply a
  sigmoid to a projection; the projections are outside this operator).
"""
from __future__ import annotations

import numpy as np


def _f64(x):
    return np.asarray(x, dtype=np.float64)


def gdn_recurrent(q, k, v, alpha, beta, state_in=None):
    """Canonical gated delta rule, one token at a time.

    For every (b, h) and t = 0..T-1::

        S <- a_t * (S - b_t * (S k_t) k_t^T) + b_t * v_t k_t^T
        o_t = S q_t

    which is ``a_t S (I - b_t k_t k_t^T) + b_t v_t k_t^T`` written with the
    matrix product associated to the right.

    Returns ``(o, S_T)`` in fp64: o ``[B, T, H, dv]``, S_T ``[B, H, dv, dk]``.
    """
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if state_in is None else _f64(state_in).copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        kt = k[:, t]                                  # [B, H, dk]
        at = a[:, t][..., None, None]                 # [B, H, 1, 1]
        bt = b[:, t][..., None, None]
        retrieved = np.einsum("bhvk,bhk->bhv", S, kt)  # S k_t, [B, H, dv]
        S = at * (S - bt * retrieved[..., :, None] * kt[..., None, :]) \
            + bt * v[:, t][..., :, None] * kt[..., None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, q[:, t])
    return o, S


def gdn_literal_eq6(q, k, v, alpha, beta, state_in=None):
    """Eq. 2 + Eq. 6 exactly as printed: ``v_old = S_{t-1} k_t`` (un-decayed),
    ``S_t = a_t S_{t-1} + b_t (v_t - v_old) k_t^T``, ``o_t = S_t q_t``.

    Not the contract of the kernels; kept so that the tests can show how the
    printed form relates to the canonical one.
    """
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if state_in is None else _f64(state_in).copy()
    o = np.empty((B, T, H, dv))
    for t in range(T):
        kt = k[:, t]
        v_old = np.einsum("bhvk,bhk->bhv", S, kt)
        S = a[:, t][..., None, None] * S \
            + b[:, t][..., None, None] * (v[:, t] - v_old)[..., :, None] * kt[..., None, :]
        o[:, t] = np.einsum("bhvk,bhk->bhv", S, q[:, t])
    return o, S


def gdn_chunked(q, k, v, alpha, beta, state_in=None, chunk=64):
    """The same recurrence evaluated chunk by chunk (WY / UT form), fp64.

    Within a chunk of C tokens that starts from state S0, with
    g_t = sum_{s<=t} log a_s (cumulative inside the chunk) and
    delta_t = b_t (v_t - a_t S_{t-1} k_t), unrolling the recurrence gives
    S_t = e^{g_t} S0 + sum_{i<=t} e^{g_t - g_i} delta_i k_i^T, hence

        (I + A) Delta = diag(b) V - diag(b e^{g}) K S0^T,
            A[t, i] = b_t e^{g_t - g_i} (k_t . k_i)        for i < t
        O      = diag(e^{g}) Q S0^T + P Delta,
            P[t, i] = e^{g_t - g_i} (q_t . k_i)            for i <= t
        S_C    = e^{g_C} S0 + Delta^T diag(e^{g_C - g}) K

    The triangular system is solved with numpy.linalg.solve.  This is only a
    re-association of ``gdn_recurrent`` (equal up to rounding for any chunk
    size); the tests check that by brute force.
    """
    q, k, v, a, b = map(_f64, (q, k, v, alpha, beta))
    B, T, H, dk = k.shape
    dv = v.shape[-1]
    S = np.zeros((B, H, dv, dk)) if state_in is None else _f64(state_in).copy()
    o = np.empty((B, T, H, dv))
    for s in range(0, T, chunk):
        e = min(s + chunk, T)
        n = e - s
        # per (b, h) tensors with the token axis next to the feature axis
        K = np.moveaxis(k[:, s:e], 1, 2)           # [B, H, n, dk]
        Q = np.moveaxis(q[:, s:e], 1, 2)
        V = np.moveaxis(v[:, s:e], 1, 2)           # [B, H, n, dv]
        la = np.log(np.moveaxis(a[:, s:e], 1, 2))  # [B, H, n]
        bb = np.moveaxis(b[:, s:e], 1, 2)
        g = np.cumsum(la, axis=-1)
        decay = np.exp(g[..., :, None] - g[..., None, :])          # e^{g_t - g_i}
        strict = np.tril(np.ones((n, n)), -1)
        incl = np.tril(np.ones((n, n)))
        A = bb[..., :, None] * decay * (K @ np.swapaxes(K, -1, -2)) * strict
        P = decay * (Q @ np.swapaxes(K, -1, -2)) * incl
        rhs = bb[..., :, None] * V - (bb * np.exp(g))[..., :, None] * (K @ np.swapaxes(S, -1, -2))
        Delta = np.linalg.solve(np.eye(n) + A, rhs)                # [B, H, n, dv]
        O = np.exp(g)[..., :, None] * (Q @ np.swapaxes(S, -1, -2)) + P @ Delta
        w = np.exp(g[..., -1:] - g)                                # e^{g_C - g_i}
        S = np.exp(g[..., -1])[..., None, None] * S \
            + np.swapaxes(Delta, -1, -2) @ (w[..., :, None] * K)
        o[:, s:e] = np.moveaxis(O, 2, 1)
    return o, S
