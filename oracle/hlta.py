"""The hybrid layer: SWA, DSWA and gated-delta-rule branches combined by
per-head sigmoid gates.

Source: Kairos paper (arXiv 2606.16533, HTML v3), Sec. 2.2 and Fig. 5 (the
three temporal pathways: SWA for local, DSWA for mid-range, GLA implemented
as GatedDeltaNet for global memory), Sec. 2.2.1 (Eq. 1-6), Sec. 2.2.2 (Eq.
7-8) and "Long-Horizon Generation" (recurrent state passing).

Readings:

* The paper stacks the pathways as separate blocks; the layer here runs them
  as parallel branches on one shared q, k, v and mixes them per head:
  ``y = sigmoid(z_swa) o_swa + sigmoid(z_dswa) o_dswa + sigmoid(z_gdn) o_gdn``
  with z of shape [3, H] and no normalisation of the gates.
* With FP8 (or 4-bit) windows the SWA/DSWA branches use the dequantised
  q_hat, k_hat (per-64-token-block absmax E4M3, or E2M1); the GDN branch uses
  the unquantised q, k.
* A streamed rollout (frames fed call by call, state carried) is defined to
  equal one call over the whole sequence; the oracle is that single call.
* ``centered=True`` gives both windowed branches Eq. 7's centred band (see
  ``window``); such a layer sees future frames and has no streamed form.
* ``rope_base``: RoPE (``rope``) on each windowed branch's q and k at that
  branch's positions, before the FP8 quantisation when there is one.
* ``qk_blocks``: the 64-token quantisation blocks of the FP8 / 4-bit paths
  run over the call's tokens in order ("tokens", blocks may straddle frames
  when 64 does not divide L) or restart at every frame ("frames": a frame's
  last block may be short).  Only the second makes a rollout fed one frame
  per call quantise exactly as one run over the whole sequence, since no
  block then mixes tokens of two calls.
"""
from __future__ import annotations

import numpy as np

from .gdn import gdn_recurrent
from .window import windowed_attention_rows
from .fp8 import fp8_quantize_blocks
from .fp4 import fp4_quantize_blocks
from .rope import rope, branch_positions


def sigmoid(z):
    z = np.asarray(z, dtype=np.float64)
    return 1.0 / (1.0 + np.exp(-z))


def _branch_inputs(q, k, L, dil, frame_offset, window_qk, rope_base, qk_blocks="tokens"):
    """q, k as one windowed branch consumes them: rotated (RoPE at the
    branch's positions) when rope_base is given, then quantised for FP8."""
    if rope_base:
        T = np.asarray(q).shape[1]
        pos = branch_positions(T, L, dil, frame_offset)
        q, k = rope(q, pos, rope_base), rope(k, pos, rope_base)
    return _window_inputs(q, k, window_qk, L if qk_blocks == "frames" else None)


def quantize_frames(x, L, window_qk):
    """The block quantiser of ``window_qk`` ("fp8" or "fp4") applied to each
    frame of L tokens of ``x`` [B, T, H, d] on its own (the last frame may be
    partial): 64-token blocks restart at every frame.  Returns ``(codes,
    scales [B, H, sum over frames of ceil(len / 64)], xhat)`` with each
    frame's scales after the previous frame's."""
    quant = fp8_quantize_blocks if window_qk == "fp8" else fp4_quantize_blocks
    x = np.asarray(x, dtype=np.float32)
    T = x.shape[1]
    parts = [quant(x[:, f0:min(f0 + L, T)]) for f0 in range(0, T, L)]
    return (np.concatenate([p[0] for p in parts], axis=1), np.concatenate([p[1] for p in parts], axis=2),
            np.concatenate([p[2] for p in parts], axis=1))


def _window_inputs(q, k, window_qk, frame_len=None):
    if window_qk not in ("fp8", "fp4"):
        return q, k
    if frame_len is not None:
        return quantize_frames(q, frame_len, window_qk)[2], quantize_frames(k, frame_len, window_qk)[2]
    quant = fp8_quantize_blocks if window_qk == "fp8" else fp4_quantize_blocks
    return quant(q)[2], quant(k)[2]


def hlta_rows(q, k, v, alpha, beta, gates, L, w, dil, rows, frame_offset=0,
              state_in=None, window_qk="bf16", o_gdn=None, centered=False, rope_base=None,
              qk_blocks="tokens"):
    """Layer output for the query tokens ``rows`` (all heads) and final state.

    The GDN branch needs every token before the last requested row; it is
    computed over the full sequence (or taken from ``o_gdn`` when given).
    Returns ``(y_rows [B, n, H, d], S_T or None)``.
    """
    S = None
    if o_gdn is None:
        o_gdn, S = gdn_recurrent(q, k, v, alpha, beta, state_in)
    qw, kw = _branch_inputs(q, k, L, 1, frame_offset, window_qk, rope_base, qk_blocks)
    o_swa = windowed_attention_rows(qw, kw, v, rows, L, w, 1, frame_offset, centered)
    qw, kw = _branch_inputs(q, k, L, dil, frame_offset, window_qk, rope_base, qk_blocks)
    o_dswa = windowed_attention_rows(qw, kw, v, rows, L, w, dil, frame_offset, centered)
    g = sigmoid(gates)                                        # [3, H]
    y = g[0][None, None, :, None] * o_swa + g[1][None, None, :, None] * o_dswa \
        + g[2][None, None, :, None] * np.asarray(o_gdn, np.float64)[:, rows]
    return y, S


def hlta(q, k, v, alpha, beta, gates, L, w, dil, frame_offset=0, state_in=None,
         window_qk="bf16", centered=False, rope_base=None, qk_blocks="tokens"):
    """Layer output for every token ``[B, T, H, d]`` and the final GDN state."""
    T = np.asarray(q).shape[1]
    return hlta_rows(q, k, v, alpha, beta, gates, L, w, dil, np.arange(T), frame_offset,
                     state_in, window_qk, centered=centered, rope_base=rope_base,
                     qk_blocks=qk_blocks)
