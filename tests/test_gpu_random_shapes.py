"""GPU parity on seeded random configurations of the hybrid layer.

Each case draws, from one fixed seed, a shape (batch, heads, frame length,
frame count, a partial last frame), a window (length, causal or centred,
dilation, frame offset), the windowed operands (bf16, E4M3 or E2M1; token or
frame quantisation blocks; RoPE or none) and whether a context runs part of
the call on its side stream, and compares y and the final GDN state with the
CPU oracle.  The rollout cases feed a random sequence through the ring in
calls of one to three frames and compare with one full-length oracle run.
The gated delta rule cases draw fp32 or bf16 inputs, the head dimension,
ragged lengths (long ones with few heads, where the scan splits over time)
and an incoming state.  Tolerances as in the other parity tests (fp32
gated delta rule: 1e-4).
"""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import host, inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3
FMT = {"bf16": K.BF16, "fp8": K.FP8_E4M3, "fp4": K.FP4_E2M1}


def _assert_close(got, ref, what, tmax=TOL_MAX, tmean=TOL_MEAN):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= tmax and rmean <= tmean, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


def _layer_cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        L = int(rng.choice([1, 7, 24, 40, 63, 64, 65, 100, 128, 150, 200, 257]))
        f_max = max(1, min(40 if L < 64 else 6, 1400 // L - 1))
        F = int(rng.integers(1, f_max + 1))
        extra = int(rng.integers(1, L)) if L > 1 and rng.random() < 0.5 else 0
        cases.append(dict(
            B=int(rng.integers(1, 3)), H=int(rng.integers(1, 4)), L=L, T=F * L + extra,
            w=int(rng.integers(1, 3 * L + 2)), dil=int(rng.integers(1, 6)), fo=int(rng.integers(0, 8)),
            centered=bool(rng.random() < 0.3), fmt=str(rng.choice(["bf16", "fp8", "fp4"])),
            blocks=str(rng.choice(["tokens", "frames"])), rope=float(rng.choice([0.0, 0.0, 1e4, 500.0])),
            ctx=bool(rng.random() < 0.5), seed=int(rng.integers(0, 1 << 30))))
    return cases


def _stream_cases(n=6, seed=20261204):
    rng = np.random.default_rng(seed)
    cases = []
    for _ in range(n):
        L = int(rng.choice([40, 64, 96, 100, 130]))
        fmt = str(rng.choice(["bf16", "fp8", "fp4"]))
        cases.append(dict(
            B=int(rng.integers(1, 3)), H=int(rng.integers(1, 3)), L=L, F=int(rng.integers(5, 10)),
            w=int(rng.integers(1, int(2.5 * L) + 1)), dil=int(rng.integers(1, 5)), fmt=fmt,
            blocks="frames" if fmt != "bf16" else str(rng.choice(["tokens", "frames"])),
            rope=float(rng.choice([0.0, 1e4])), seed=int(rng.integers(0, 1 << 30)),
            calls_seed=int(rng.integers(0, 1 << 30))))
    return cases


def _gdn_cases(n=10, seed=20261205):
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        io = str(rng.choice(["f32", "bf16"]))
        d = int(rng.choice([32, 64, 128] if io == "f32" else [64, 128]))
        long_seq = i % 3 == 0                    # few heads, long sequence: the split scan
        B, H = (1, int(rng.integers(1, 3))) if long_seq else (int(rng.integers(1, 4)), int(rng.integers(1, 6)))
        T = int(rng.integers(2000, 6001)) if long_seq else int(rng.choice([int(rng.integers(0, 1500)), 64 * int(rng.integers(1, 20))]))
        cases.append(dict(io=io, d=d, B=B, H=H, T=T, state=bool(rng.random() < 0.5),
                          alpha=str(rng.choice(["softplus", "uniform"])), seed=int(rng.integers(0, 1 << 30))))
    return cases


LAYER_CASES = _layer_cases()
STREAM_CASES = _stream_cases()
GDN_CASES = _gdn_cases()


@pytest.mark.parametrize("i", range(len(LAYER_CASES)))
def test_random_layer_matches_oracle(i):
    c = LAYER_CASES[i]
    print(f"random layer {i}: {c}", flush=True)
    B, T, H, L = c["B"], c["T"], c["H"], c["L"]
    inp = make_custom(B, T, H, 128, "bf16", seed=c["seed"])
    dv = inputs_to_dev(inp)
    qb = K.QK_BLOCKS_FRAMES if c["blocks"] == "frames" else K.QK_BLOCKS_TOKENS
    ctx = K.Context() if c["ctx"] else None
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, c["w"],
                             c["dil"], frame_offset=c["fo"], window_qk=FMT[c["fmt"]], qk_blocks=qb,
                             centered=c["centered"], rope_base=c["rope"], ctx=ctx)
    torch.cuda.synchronize()
    if ctx is not None:
        ctx.close()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"], L,
                               c["w"], c["dil"], frame_offset=c["fo"], window_qk=c["fmt"],
                               centered=c["centered"], rope_base=c["rope"] or None, qk_blocks=c["blocks"])
    _assert_close(host(y), y_ref, "y")
    _assert_close(host(S), S_ref, "S")


@pytest.mark.parametrize("i", range(len(STREAM_CASES)))
def test_random_rollout_matches_full_run(i):
    c = STREAM_CASES[i]
    print(f"random rollout {i}: {c}", flush=True)
    B, H, L, F, w, dil = c["B"], c["H"], c["L"], c["F"], c["w"], c["dil"]
    T = F * L
    inp = make_custom(B, T, H, 128, "bf16", seed=c["seed"])
    dv = inputs_to_dev(inp)
    wq = FMT[c["fmt"]]
    qb = K.QK_BLOCKS_FRAMES if c["blocks"] == "frames" else K.QK_BLOCKS_TOKENS
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))
    k_ring, v_ring = K.alloc_rings(B, L, H, 128, w, dil, R, wq, c["rope"], qb)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    rng = np.random.default_rng(c["calls_seed"])
    ys, f = [], 0
    while f < F:
        nf = min(int(rng.integers(1, 4)), F - f)
        sl = slice(f * L, (f + nf) * L)
        y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                 dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                 dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                 frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                 k_ring=k_ring, v_ring=v_ring, rope_base=c["rope"], window_qk=wq,
                                 qk_blocks=qb)
        ys.append(y)
        f += nf
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=c["fmt"], qk_blocks=c["blocks"],
                               rope_base=c["rope"] or None)
    _assert_close(np.concatenate([host(y) for y in ys], axis=1), y_ref, "rollout y")
    _assert_close(host(state), S_ref, "rollout S")


@pytest.mark.parametrize("i", range(len(GDN_CASES)))
def test_random_gdn_matches_oracle(i):
    c = GDN_CASES[i]
    print(f"random gdn {i}: {c}", flush=True)
    B, T, H, d = c["B"], c["T"], c["H"], c["d"]
    inp = make_custom(B, T, H, d, c["io"], seed=c["seed"], alpha_kind=c["alpha"])
    dv = inputs_to_dev(inp, c["io"])
    s0 = None
    if c["state"]:
        s0 = np.random.default_rng(c["seed"] + 1).standard_normal((B, H, d, d)).astype(np.float32) * 0.1
    out, S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"],
                              state_in=None if s0 is None else torch.from_numpy(s0).to("cuda:0"))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], state_in=s0)
    tol = (1e-4, 1e-4) if c["io"] == "f32" else (TOL_MAX, TOL_MEAN)
    if T > 0:
        _assert_close(host(out), o_ref, "o", *tol)
    _assert_close(host(S), S_ref, "S", *tol)
