"""GPU checks that need no oracle.

* Closed forms of the gated delta rule on the kernels: a key written twice
  (alpha = beta = 1, orthonormal keys) maps to its second value; with
  beta = 0 a non-zero state only decays, S_T = (prod alpha) S0 and
  o_t = (prod_{s<=t} alpha_s) S0 q_t.
* Runs into outputs, state and workspace filled with NaN bit patterns give
  results bit-identical to runs into zeroed buffers, and repeated runs are
  bit-identical (every output element is written, nothing reads an
  unwritten workspace byte, the kernels are deterministic).  The layer cases
  cover both schedules of the layer call: small calls run the GDN branch
  beside the window kernel, the larger ones before it.
"""
import numpy as np
import pytest
import torch

import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import dev_f32, host, inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu


def test_gdn_key_collision_fp32():
    rng = np.random.default_rng(21)
    d, n = 128, 64
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = Qm[:, :n].T                                   # n orthonormal rows
    T = 2 * n
    k = np.concatenate([keys, keys])[None, :, None, :].astype(np.float32)
    v = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    q = rng.standard_normal((1, T, 1, d)).astype(np.float32)
    ones = np.ones((1, T, 1), np.float32)
    _, S = K.kairos_gdn_fwd(dev_f32(q), dev_f32(k), dev_f32(v), dev_f32(ones), dev_f32(ones))
    torch.cuda.synchronize()
    Sk = (host(S)[0, 0] @ k[0, :n, 0].astype(np.float64).T).T   # row j = S k_j
    err = np.max(np.abs(Sk - v[0, n:, 0]))
    print(f"collision: max |S k_j - v'_j| = {err:.2e}", flush=True)
    assert err <= 1e-4


@pytest.mark.parametrize("io", ["f32", "bf16"])
def test_gdn_beta_zero_decays_the_state(io):
    B, T, H, d = 1, 150, 2, 128
    inp = make_custom(B, T, H, d, io, seed=23, alpha_kind="uniform")
    S0 = np.random.default_rng(22).standard_normal((B, H, d, d)).astype(np.float32)
    dv = inputs_to_dev(inp, io)
    out, S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], torch.zeros_like(dv["beta"]),
                              dev_f32(S0))
    torch.cuda.synchronize()
    cum = np.cumprod(inp["alpha"].astype(np.float64), axis=1)          # [B, T, H]
    o_ref = cum[..., None] * np.einsum("bhij,bthj->bthi", S0.astype(np.float64),
                                       inp["q"].astype(np.float64))
    S_ref = cum[:, -1][:, :, None, None] * S0.astype(np.float64)
    tol = 1e-4 if io == "f32" else 1e-2
    for got, ref, what in ((host(out), o_ref, "o"), (host(S), S_ref, "S")):
        rmax, rmean = rel_errors(got, ref)
        print(f"beta = 0 ({io}) {what}: rel_max={rmax:.2e} rel_mean={rmean:.2e}", flush=True)
        assert rmax <= tol


def _runs(call, bufs):
    """call() three times, into buffers zeroed / NaN-filled / zeroed."""
    res = []
    for fill in (0x00, 0xFF, 0x00):
        for t in bufs:
            t.view(torch.uint8).fill_(fill)
        call()
        torch.cuda.synchronize()
        res.append([t.clone() for t in bufs])
    return res


def _assert_same(res, names):
    for i, name in enumerate(names):
        if res[0][i].dtype != torch.uint8:
            assert torch.isfinite(res[0][i].float()).all(), f"{name}: non-finite values"
        for r in res[1:]:
            assert torch.equal(r[i], res[0][i]), f"{name}: differs between runs"


def test_gdn_poisoned_buffers_and_determinism():
    B, T, H = 2, 300, 4
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=601))
    nws = K.kairos_gdn_workspace_size(K.gdn_desc(B, T, H, 128))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    S = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    res = _runs(lambda: K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], out=out,
                                         state_out=S, workspace=ws), [out, S])
    _assert_same(res, ["o", "S"])


@pytest.mark.parametrize("use_ctx", [False, True])
@pytest.mark.parametrize("F,L,H,w,qk", [(6, 200, 2, 300, "bf16"), (6, 200, 2, 300, "fp8"),
                                         (8, 1024, 8, 1000, "bf16"), (8, 1024, 8, 1000, "fp8")])
def test_layer_poisoned_buffers_and_determinism(F, L, H, w, qk, use_ctx):
    """Single-stream calls, and with a context both of its schedules (the GDN
    beside the window kernel for the small calls, the operand pre-passes
    beside the scan for the larger ones)."""
    B, dil = 1, 4
    T = F * L
    print(f"layer F{F} L{L} H{H} {qk} ctx={use_ctx}", flush=True)
    ctx = K.Context() if use_ctx else None
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=600 + L + H))
    wq = K.FP8_E4M3 if qk == "fp8" else K.BF16
    nws = K.kairos_hlta_workspace_size(K.hlta_desc(B, T, H, 128, L, w, dil, window_qk=wq))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    S = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    res = _runs(lambda: K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"],
                                          L, w, dil, window_qk=wq, out=out, state_out=S, workspace=ws,
                                          ctx=ctx),
                [ws, out, S])
    _assert_same([r[1:] for r in res], ["y", "S"])
    if ctx is not None:
        ctx.close()


def test_window_stage_poisoned_buffers_and_determinism():
    B, F, L, H, w, dil = 1, 7, 150, 3, 200, 4
    T = F * L
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=602))
    o_gdn = dv["v"].flip(1).contiguous()                  # any bf16 tensor of the shape
    ws = torch.empty(4 * B * T * H * 129, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    res = _runs(lambda: K.kairos_hlta_window_fwd(dv["q"], dv["k"], dv["v"], o_gdn, dv["gates"], L, w, dil,
                                                 out=out, workspace=ws), [ws, out])
    _assert_same([r[1:] for r in res], ["y"])


@pytest.mark.parametrize("fmt,rope", [("bf16", 0.0), ("fp8", 1e4)])
def test_streaming_resume_from_host(fmt, rope):
    """Checkpoint and resume of a streamed rollout: after frame 4 the GDN state
    and both rings (with FP8: key codes and block scales; with RoPE: both
    branches' rotated keys) go to host memory, every device buffer is freed,
    fresh buffers are filled from the host copies and the rollout continues.
    Outputs and final state are bit-identical to an uninterrupted rollout:
    state, rings and the absolute frame index are the rollout's whole state."""
    B, F, L, H, w, dil = 1, 9, 96, 2, 150, 2
    T = F * L
    print(f"resume {fmt} rope={rope}", flush=True)
    wq = K.FP8_E4M3 if fmt == "fp8" else K.BF16
    qb = K.QK_BLOCKS_FRAMES if fmt == "fp8" else K.QK_BLOCKS_TOKENS
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=77))
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))

    def frame(f, state, kr, vr):
        sl = slice(f * L, (f + 1) * L)
        y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                 dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                 dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                 frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                 k_ring=kr, v_ring=vr, rope_base=rope, window_qk=wq, qk_blocks=qb)
        return y

    kr, vr = K.alloc_rings(B, L, H, 128, w, dil, R, wq, rope, qb)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ref = [frame(f, state, kr, vr).clone() for f in range(F)]
    torch.cuda.synchronize()
    ref_state = state.clone()

    kr, vr = K.alloc_rings(B, L, H, 128, w, dil, R, wq, rope, qb)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    got = [frame(f, state, kr, vr).clone() for f in range(5)]
    torch.cuda.synchronize()
    saved = [t.to("cpu", copy=True) for t in (state, kr, vr)]     # host copies
    del state, kr, vr
    torch.cuda.empty_cache()
    state, kr, vr = (t.to("cuda:0", copy=True) for t in saved)
    got += [frame(f, state, kr, vr).clone() for f in range(5, F)]
    torch.cuda.synchronize()
    for f in range(F):
        assert torch.equal(got[f], ref[f]), f"frame {f} differs after the resume"
    assert torch.equal(state, ref_state)
