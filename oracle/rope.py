"""Rotary position embedding (RoPE) of the windowed branches' queries and
keys, fp64.

TEST INFRASTRUCTURE ONLY (see the package header).

Source: Kairos paper (arXiv 2606.16533, HTML v3), Sec. 2.2.2 (every
sliding-window attention block, SWA and DSWA, uses RoPE-based relative
positional encoding; global position is left to the linear-attention path),
and Fig. 5's summary (RoPE handles local positional reasoning).  The paper
does not define the variant; the definition used is the one published with
the name, RoFormer (Su et al., "RoFormer: Enhanced Transformer with Rotary
Position Embedding", Eq. 13-15 there): feature pairs (2i, 2i+1) of a token at
position p are rotated by the angle p * theta_i, theta_i = base^(-2i/d).

Readings (the paper is silent on these):

* The base is a parameter (10000 in RoFormer).
* The position of a token is its position in the sequence its branch attends
  over: the absolute token index for SWA, and for DSWA the position in its
  residue group's sub-sequence (the rearranged sequence of Eq. 8),
  p = (f div dil) * L + (t mod L) with f the absolute frame index.  Since the
  rotation makes every score depend on position differences only, the origin
  does not matter; absolute frames keep calls of a rollout consistent.
* RoPE acts on q and k of the windowed branches only (not on v, not on the
  gated delta rule).  With FP8 windows the rotated values are quantised.
"""
from __future__ import annotations

import numpy as np

from .window import frame_index_maps


def rope_angles(pos, d, base):
    """Angles p * theta_i, shape [len(pos), d/2], fp64."""
    i = np.arange(d // 2, dtype=np.float64)
    theta = np.power(float(base), -2.0 * i / d)
    return np.asarray(pos, dtype=np.float64)[:, None] * theta[None, :]


def rope(x, pos, base):
    """Rotate feature pairs (2i, 2i+1) of x [B, T, H, d] by pos[t] * theta_i."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    ang = rope_angles(pos, d, base)                 # [T, d/2]
    c = np.cos(ang)[None, :, None, :]
    s = np.sin(ang)[None, :, None, :]
    x0, x1 = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = x0 * c - x1 * s
    out[..., 1::2] = x0 * s + x1 * c
    return out


def branch_positions(T, L, dil, frame_offset=0):
    """RoPE positions of a branch: the group positions p (dil = 1: absolute token index)."""
    _, _, p = frame_index_maps(T, L, dil, frame_offset)
    return p
