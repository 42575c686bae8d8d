"""Sliding-window (SWA) and dilated sliding-window (DSWA) softmax attention, fp64.

Source: Kairos paper (arXiv 2606.16533, HTML v3), Sec. 2.2.2 "Local and
Mid-Range Pathways", Eq. 7 (SWA over a token window w = L x window_size on a
sequence of F frames of L tokens) and Eq. 8 (DSWA = SWA on the input
rearranged from (B, F*L, D) to (B*d, F/d*L, D)).

Readings (the paper is ambiguous or silent on these):

* Causal windows by default.  Eq. 7 prints a centred band; the workloads
  here are causal, and streaming needs causality.  Query i sees the w keys
  ``i - w < j <= i`` (itself included).
* Centred windows (``centered=True``): Eq. 7's band ``[i - w/2, i + w/2]``
  read with the radius rounded down, r = floor(w / 2), both ends included:
  query i sees ``|j - i| <= r`` (2r + 1 keys away from the sequence ends;
  w + 1 for even w, w for odd w).  Keys exist only inside the call.
* Dilation groups frames by residue: frame f belongs to group f mod d (the
  rearrange keeps the frame's tokens contiguous and strides frames by d).
  Frames are counted from an absolute index ``frame_offset`` of the first
  frame of the call, so that a rollout cut into calls groups frames the same
  way as one long call.  F need not be divisible by d (groups may differ in
  size); the window counts sub-sequence positions.
* Softmax scale 1/sqrt(d), d the head dimension.  No positional encoding is
  applied (q and k are taken as already position-encoded).
* Keys exist only inside the call's sequence (no keys before token 0).

For every query i (token index inside the call), with
f(t) = t // L + frame_offset, r(t) = f(t) mod dil and
p(t) = (f(t) // dil) * L + t mod L, the key set is

    J(i) = { j : r(j) = r(i) and p(i) - w < p(j) <= p(i) }

and the output is sum_{j in J(i)} softmax_j(q_i . k_j / sqrt(d)) v_j.  With
dil = 1 this is exactly SWA's set {i - w < j <= i}.  Centred windows use

    J(i) = { j : r(j) = r(i) and |p(j) - p(i)| <= floor(w / 2) }.
"""
from __future__ import annotations

import math

import numpy as np


def frame_index_maps(T, L, dil, frame_offset=0):
    """Per-token absolute frame f, residue r and sub-sequence position p."""
    t = np.arange(T, dtype=np.int64)
    f = t // L + frame_offset
    r = f % dil
    p = (f // dil) * L + t % L
    return f, r, p


def _candidate_keys(i_lo, i_hi, T, L, w, dil, frame_offset):
    """Token indices that can hold keys of queries i_lo..i_hi (all in one frame)."""
    if dil == 1:
        return np.arange(max(0, i_lo - w + 1), i_hi + 1)
    f_loc = i_lo // L                       # frame index inside the call
    frames = []
    fl = f_loc
    # sub-sequence frames back needed to cover w positions: ceil(w / L) + 1 is enough
    for _ in range(w // L + 2):
        if fl < 0:
            break
        frames.append(fl)
        fl -= dil
    idx = [np.arange(fr * L, min((fr + 1) * L, T)) for fr in reversed(frames)]
    idx = np.concatenate(idx)
    return idx[idx <= i_hi]


def _in_window(p_key, p_query, w, centered):
    """Window test on sub-sequence positions (broadcasting)."""
    if centered:
        return np.abs(p_key - p_query) <= w // 2
    return (p_key > p_query - w) & (p_key <= p_query)


def windowed_attention_rows(q, k, v, rows, L, w, dil=1, frame_offset=0, centered=False,
                            rope_base=None):
    """Outputs of the windowed branch for the query tokens ``rows`` only.

    ``rope_base``: when given, q and k are first rotated by RoPE at the
    branch's positions (``oracle.rope``: group positions of this dilation).

    q, k, v: ``[B, T, H, d]``.  Returns ``[B, len(rows), H, d]`` fp64.
    Naive masked softmax: scores materialised, max subtracted, exponentiated,
    normalised, then multiplied by V.
    """
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, d = q.shape
    if rope_base:
        from .rope import rope, branch_positions
        pos = branch_positions(T, L if L else T, dil, frame_offset)
        q, k = rope(q, pos, rope_base), rope(k, pos, rope_base)
    rows = np.asarray(rows, dtype=np.int64)
    out = np.empty((B, len(rows), H, v.shape[-1]))
    f, r, p = frame_index_maps(T, L if L else T, dil, frame_offset)
    scale = 1.0 / math.sqrt(d)
    Lf = L if L else T
    # group the requested rows by frame, then in blocks of <= 256 rows
    order = np.argsort(rows, kind="stable")
    srt = rows[order]
    start = 0
    while start < len(srt):
        fr = srt[start] // Lf
        end = start
        while end < len(srt) and srt[end] // Lf == fr and end - start < 256:
            end += 1
        qi = srt[start:end]
        if centered:
            # every token of the rows' group within reach of the rows' positions
            rad = w // 2
            cand = np.nonzero((r == r[qi[0]]) & (p >= p[qi].min() - rad) & (p <= p[qi].max() + rad))[0]
        else:
            cand = _candidate_keys(qi[0], qi[-1], T, Lf, w, dil, frame_offset)
        mask = (r[cand][None, :] == r[qi][:, None]) \
            & _in_window(p[cand][None, :], p[qi][:, None], w, centered)
        for b in range(B):
            for h in range(H):
                s = (q[b, qi, h] @ k[b, cand, h].T) * scale
                s = np.where(mask, s, -np.inf)
                s = s - s.max(axis=1, keepdims=True)
                e = np.exp(s)
                e = e / e.sum(axis=1, keepdims=True)
                out[b, order[start:end], h] = e @ v[b, cand, h]
        start = end
    return out


def windowed_attention(q, k, v, L, w, dil=1, frame_offset=0, centered=False, rope_base=None):
    """Windowed branch for every query token: ``[B, T, H, d]`` fp64."""
    T = np.asarray(q).shape[1]
    return windowed_attention_rows(q, k, v, np.arange(T), L, w, dil, frame_offset, centered,
                                   rope_base)


def window_bruteforce(q, k, v, L, w, dil=1, frame_offset=0, centered=False):
    """Scalar loops straight from the key-set definition; tiny inputs only."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, d = q.shape
    out = np.zeros((B, T, H, v.shape[-1]))
    Lf = L if L else T
    for b in range(B):
        for h in range(H):
            for i in range(T):
                fi = i // Lf + frame_offset
                pi = (fi // dil) * Lf + i % Lf
                keys = []
                for j in range(T):
                    fj = j // Lf + frame_offset
                    pj = (fj // dil) * Lf + j % Lf
                    if centered:
                        inside = abs(pj - pi) <= w // 2
                    else:
                        inside = pi - w < pj <= pi
                    if fj % dil == fi % dil and inside:
                        keys.append(j)
                sc = [sum(q[b, i, h, c] * k[b, j, h, c] for c in range(d)) / math.sqrt(d)
                      for j in keys]
                m = max(sc)
                ex = [math.exp(x - m) for x in sc]
                z = sum(ex)
                for jj, j in enumerate(keys):
                    out[b, i, h] += ex[jj] / z * v[b, j, h]
    return out


def dswa_reshape(q, k, v, L, w, dil, frame_offset=0, swa=None, centered=False):
    """Eq. 8 taken literally: gather each residue group's frames into one
    contiguous sub-sequence (the rearrange), run SWA with window w (causal or
    centred) on it, and scatter the outputs back to their tokens.  ``swa`` is
    the SWA routine to use (defaults to ``windowed_attention`` with dil = 1)."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    B, T, H, d = q.shape
    if swa is None:
        def swa(qq, kk, vv):
            return windowed_attention(qq, kk, vv, L, w, 1, 0, centered)
    out = np.empty_like(v)
    F = -(-T // L)
    for res in range(dil):
        frames = [fr for fr in range(F) if (fr + frame_offset) % dil == res]
        if not frames:
            continue
        idx = np.concatenate([np.arange(fr * L, min((fr + 1) * L, T)) for fr in frames])
        out[:, idx] = swa(q[:, idx], k[:, idx], v[:, idx])
    return out
