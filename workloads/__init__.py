"""Seeded synthetic inputs shaped like the video-token workloads of the hybrid
linear temporal attention layer.

This module holds input generation only: random draws, the L2 normalisation
of keys that the inputs are specified to arrive with, bf16 rounding, and the
named workload shapes.  It contains none of the method's arithmetic and is
shared by the oracle side (tests, CPU baseline) and the GPU side (tests,
bench) alike.

Recipe (per workload index i): NumPy PCG64 seeded with ``1000 + i``; a
SeedSequence is spawned into six child streams used in the fixed order
q, k, v, alpha-source, beta-source, gates.  q, k, v are standard normal fp32
in C order ``[B, T, H, d]``, drawn in consecutive chunks of 2^22 elements,
chunk j from child j of the tensor's stream (so chunks can be drawn in
parallel and the result does not depend on the thread count); k is
L2-normalised per (token, head) in fp64 and then rounded; bf16 workloads
round q, k, v to bf16 (round to nearest even).
alpha and beta stay fp32, shape ``[B, T, H]``; gate logits are fp32 ``[3, H]``
in the order (swa, dswa, gdn).
"""
from __future__ import annotations

import dataclasses
import os
from typing import Optional

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "workload", "make_inputs", "make_custom", "make_raw",
    "to_bf16_bits", "bf16_bits_to_f32", "round_bf16",
]


@dataclasses.dataclass(frozen=True)
class Workload:
    """Shape and distribution recipe of one synthetic workload."""
    name: str
    B: int
    T: int
    H: int
    d: int
    io: str                      # "f32" or "bf16"
    alpha_kind: str              # "uniform" (U(0.9,0.999)) or "softplus" (exp(-softplus(N(-4,1))))
    beta_kind: str               # "uniform" (U(0.05,1)) or "sigmoid" (sigmoid(N(0,1)))
    L: int = 0                   # tokens per frame (0: no frames, GDN only)
    window: int = 0
    dilation: int = 1
    window_qk: str = "bf16"      # "bf16" or "fp8"
    stream_frames: int = 0       # >0: rolled out one frame per call with a KV ring
    ring_frames: int = 0
    seed: int = 1000

    @property
    def frames(self) -> int:
        return self.T // self.L if self.L else 0


# The five workloads: the fp32 gated delta rule on a tiny shape, the chunked
# bf16 gated delta rule, the bf16 hybrid layer over 21 frames of 1560 tokens,
# its 61-frame streamed rollout, and the FP8 hybrid layer over 16 frames of
# 3600 tokens.
WORKLOADS = [
    Workload("gdn_f32_B1H2T64d32", 1, 64, 2, 32, "f32", "uniform", "uniform", seed=1000),
    Workload("gdn_bf16_B2H16T4096d128", 2, 4096, 16, 128, "bf16", "softplus", "sigmoid", seed=1001),
    Workload("hlta_bf16_B1H24F21L1560", 1, 21 * 1560, 24, 128, "bf16", "softplus", "sigmoid",
             L=1560, window=1560, dilation=4, seed=1002),
    Workload("hlta_stream_B1H24F61L1560", 1, 61 * 1560, 24, 128, "bf16", "softplus", "sigmoid",
             L=1560, window=1560, dilation=4, stream_frames=61, ring_frames=4, seed=1003),
    Workload("hlta_fp8_B4H24F16L3600", 4, 16 * 3600, 24, 128, "bf16", "softplus", "sigmoid",
             L=3600, window=3600, dilation=4, window_qk="fp8", seed=1004),
]


def workload(i: int) -> Workload:
    return WORKLOADS[i]


# --------------------------------------------------------------------------- bf16

def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even.  Inputs are
    finite, so the 32-bit sum cannot wrap (largest pattern 0xFF7FFFFF)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    r = (u >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(to_bf16_bits(x))


# --------------------------------------------------------------------------- draws

def _l2_normalise_rows(k: np.ndarray, block: int = 1 << 16) -> np.ndarray:
    """Normalise the last axis to unit L2 norm in fp64 (in place, slices in
    parallel); the result is rounded to fp32 once."""
    import concurrent.futures as cf
    flat = k.reshape(-1, k.shape[-1])

    def norm(s):
        x = flat[s:s + block].astype(np.float64)
        n = np.sqrt(np.einsum("ij,ij->i", x, x))[:, None]
        np.divide(x, n, out=x)
        flat[s:s + block] = x
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
        list(pool.map(norm, range(0, flat.shape[0], block)))
    return k


_CHUNK = 1 << 22


def _normal_chunked(ss: np.random.SeedSequence, shape, pool) -> np.ndarray:
    """Standard normal fp32 array; chunk j drawn from child j of ss."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nchunks = max(1, -(-n // _CHUNK))
    children = ss.spawn(nchunks)

    def fill(j):
        g = np.random.Generator(np.random.PCG64(children[j]))
        s0 = j * _CHUNK
        out[s0:min(n, s0 + _CHUNK)] = g.standard_normal(min(n, s0 + _CHUNK) - s0, dtype=np.float32)
    list(pool.map(fill, range(nchunks)))
    return out.reshape(shape)


def _draw(seqs, B, T, H, d, alpha_kind, beta_kind):
    import concurrent.futures as cf
    sq, sk, sv, sa, sb, sg = seqs
    ra, rb, rg = (np.random.Generator(np.random.PCG64(x)) for x in (sa, sb, sg))
    shape = (B, T, H, d)
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
        q = _normal_chunked(sq, shape, pool)
        k = _l2_normalise_rows(_normal_chunked(sk, shape, pool))
        v = _normal_chunked(sv, shape, pool)
    if alpha_kind == "uniform":
        alpha = ra.uniform(0.9, 0.999, size=(B, T, H)).astype(np.float32)
    elif alpha_kind == "softplus":
        x = ra.standard_normal((B, T, H), dtype=np.float32).astype(np.float64) - 4.0
        alpha = (1.0 / (1.0 + np.exp(x))).astype(np.float32)      # exp(-softplus(x))
    else:
        raise ValueError(alpha_kind)
    if beta_kind == "uniform":
        beta = rb.uniform(0.05, 1.0, size=(B, T, H)).astype(np.float32)
    elif beta_kind == "sigmoid":
        x = rb.standard_normal((B, T, H), dtype=np.float32).astype(np.float64)
        beta = (1.0 / (1.0 + np.exp(-x))).astype(np.float32)
    else:
        raise ValueError(beta_kind)
    gates = rg.standard_normal((3, H), dtype=np.float32)
    return q, k, v, alpha, beta, gates


def make_custom(B: int, T: int, H: int, d: int, io: str = "bf16", seed: int = 0,
                alpha_kind: str = "softplus", beta_kind: str = "sigmoid") -> dict:
    """Inputs of arbitrary shape with a workload's distributions.

    Returns a dict of fp32 arrays (q, k, v hold exactly representable bf16
    values when ``io == "bf16"``) plus ``q_bits``/``k_bits``/``v_bits`` uint16
    bf16 patterns for bf16 io.
    """
    seqs = np.random.SeedSequence(seed).spawn(6)
    q, k, v, alpha, beta, gates = _draw(seqs, B, T, H, d, alpha_kind, beta_kind)
    out = dict(alpha=alpha, beta=beta, gates=gates)
    if io == "bf16":
        import concurrent.futures as cf

        def conv(x):
            bits = to_bf16_bits(x)
            return bits, bf16_bits_to_f32(bits)
        with cf.ThreadPoolExecutor(3) as ex:
            res = list(ex.map(conv, (q, k, v)))
        for name, (bits, vals) in zip(("q", "k", "v"), res):
            out[name + "_bits"] = bits
            out[name] = vals
    elif io == "f32":
        out.update(q=q, k=k, v=v)
    else:
        raise ValueError(io)
    return out


def make_raw(B: int, T: int, H: int, d: int, io: str = "bf16", seed: int = 0) -> dict:
    """Raw per-token inputs of the gated delta rule's input prologue.

    q, k, v standard normal fp32 ``[B, T, H, d]`` (keys NOT normalised),
    decay logits ``za = -x`` with x ~ N(-4, 1) (so sigmoid(za) is the
    softplus workloads' decay exp(-softplus(x))), write-strength logits
    ``zb`` ~ N(0, 1), both fp32 ``[B, T, H]``.  Seeded like make_custom
    (SeedSequence(seed) spawned into five streams: q, k, v, za, zb).  For
    ``io == "bf16"`` q, k, v are rounded to bf16 and ``*_bits`` hold the
    patterns.
    """
    import concurrent.futures as cf
    sq, sk, sv, sa, sb = np.random.SeedSequence(seed).spawn(5)
    shape = (B, T, H, d)
    with cf.ThreadPoolExecutor(min(16, os.cpu_count() or 1)) as pool:
        q = _normal_chunked(sq, shape, pool)
        k = _normal_chunked(sk, shape, pool)
        v = _normal_chunked(sv, shape, pool)
    ra, rb = (np.random.Generator(np.random.PCG64(x)) for x in (sa, sb))
    za = -(ra.standard_normal((B, T, H), dtype=np.float32) - np.float32(4.0))
    zb = rb.standard_normal((B, T, H), dtype=np.float32)
    out = dict(za=za, zb=zb)
    for name, x in (("q", q), ("k", k), ("v", v)):
        if io == "bf16":
            out[name + "_bits"] = to_bf16_bits(x)
            out[name] = bf16_bits_to_f32(out[name + "_bits"])
        elif io == "f32":
            out[name] = x
        else:
            raise ValueError(io)
    return out


def make_inputs(w: Workload | int, T: Optional[int] = None) -> dict:
    """Inputs of a named workload (optionally truncated to the first T tokens,
    which keeps every draw of the full workload's prefix only when T equals
    the full length; truncated draws are a different, smaller sample)."""
    if isinstance(w, int):
        w = WORKLOADS[w]
    return make_custom(w.B, T if T is not None else w.T, w.H, w.d, w.io, w.seed,
                       w.alpha_kind, w.beta_kind)


def make_device_inputs(w: Workload | int, device="cuda:0", seed_offset: int = 0, T: Optional[int] = None) -> dict:
    """The workload's distributions drawn on the device with torch's generator
    (seeded with the workload's seed; a different stream of numbers than the
    NumPy recipe, used where only shapes and distributions matter, e.g. for
    timing).  q, k, v bf16 (k L2-normalised in fp32 before rounding);
    alpha, beta, gates fp32."""
    import torch
    if isinstance(w, int):
        w = WORKLOADS[w]
    T = w.T if T is None else T
    gen = torch.Generator(device=device)
    gen.manual_seed(w.seed + seed_offset)
    shape = (w.B, T, w.H, w.d)
    out = {}
    dt = torch.bfloat16 if w.io == "bf16" else torch.float32
    q = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    out["q"] = q.to(dt)
    del q
    k = torch.randn(shape, generator=gen, device=device, dtype=torch.float32)
    k /= torch.linalg.vector_norm(k, dim=-1, keepdim=True)
    out["k"] = k.to(dt)
    del k
    out["v"] = torch.randn(shape, generator=gen, device=device, dtype=torch.float32).to(dt)
    if w.alpha_kind == "softplus":
        x = torch.randn((w.B, T, w.H), generator=gen, device=device) - 4.0
        out["alpha"] = torch.sigmoid(-x)                      # exp(-softplus(x))
    else:
        out["alpha"] = torch.rand((w.B, T, w.H), generator=gen, device=device) * 0.099 + 0.9
    if w.beta_kind == "sigmoid":
        out["beta"] = torch.sigmoid(torch.randn((w.B, T, w.H), generator=gen, device=device))
    else:
        out["beta"] = torch.rand((w.B, T, w.H), generator=gen, device=device) * 0.95 + 0.05
    out["gates"] = torch.randn((3, w.H), generator=gen, device=device)
    return out
