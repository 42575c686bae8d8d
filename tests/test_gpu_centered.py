"""GPU parity of the centred windows (Eq. 7's band as printed, radius
floor(w / 2) on both sides) for SWA and DSWA with the paper's dilations 6
and 12, alone and inside the hybrid layer, bf16 and FP8 E4M3 Q/K, against the
oracle (``centered=True``).

Tolerances as for the causal windows: rel_max <= 2e-2, rel_mean <= 5e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import dev_bf16, host, inputs_to_dev
from workloads import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3


def _assert_close(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= TOL_MAX and rmean <= TOL_MEAN, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


CASES = [
    # B, T, L, H, w, dil, frame_offset
    (1, 6 * 128, 128, 2, 200, 1, 0),          # SWA, several query tiles per frame
    (1, 12 * 100, 100, 2, 300, 6, 0),         # DSWA dilation 6, two frames per group
    (1, 13 * 64, 64, 1, 130, 12, 5),          # dilation 12, groups of 1-2 frames, absolute offset
    (2, 7 * 200, 200, 2, 401, 6, 0),          # odd window
    (1, 40 * 24, 24, 2, 50, 6, 0),            # frames shorter than a key block
    (1, 5 * 130 + 37, 130, 2, 260, 6, 2),     # partial last frame
    (1, 4 * 96, 96, 1, 100000, 6, 0),         # window wider than every group
    (1, 3 * 64, 64, 1, 1, 12, 0),             # radius 0: o = v
]


@pytest.mark.parametrize("B,T,L,H,w,dil,fo", CASES)
def test_centered_single_branch(B, T, L, H, w, dil, fo):
    print(f"centred window B={B} T={T} L={L} H={H} w={w} dil={dil} fo={fo}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=T + w + dil)
    dv = inputs_to_dev(inp)
    for dl in sorted({1, dil}):
        out = K.kairos_window_fwd(dv["q"], dv["k"], dv["v"], L, w, dl, frame_offset=fo, centered=True)
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(inp["q"], inp["k"], inp["v"], L, w, dl, fo, centered=True)
        _assert_close(host(out), ref, f"centred window dil={dl}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("dil", [6, 12])
def test_centered_layer(fp8, dil):
    B, L, H, w = 2, 150, 2, 300
    T = 13 * L
    print(f"centred layer fp8={fp8} dil={dil}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=900 + dil + fp8)
    dv = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w,
                             dil, window_qk=K.FP8_E4M3 if fp8 else K.BF16, centered=True)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk="fp8" if fp8 else "bf16", centered=True)
    _assert_close(host(y), y_ref, "centred y")
    _assert_close(host(S), S_ref, "centred S")


def test_centered_rejects_ring():
    inp = make_custom(1, 64, 1, 128, "bf16", seed=1)
    dv = inputs_to_dev(inp)
    ring = torch.zeros((1, 4, 64, 1, 128), dtype=torch.bfloat16, device="cuda:0")
    with pytest.raises(K.KairosError):
        K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], 64, 64, 4,
                          ring_frames=4, k_ring=ring, v_ring=ring, centered=True)


def _rows(T, L, dil, rad, seed):
    """Query rows at the edges a centred band treats specially: sequence ends,
    frame boundaries, 128-query tile edges, rows within the radius of the end
    of their group, plus seeded random rows."""
    r = {0, 1, 127, 128, T - 1, T - 2, T - 1 - rad, T - rad}
    for f in (0, 1, dil - 1, dil, T // L - dil - 1, T // L - 1):
        for off in (0, 1, 127, 128, L - 1, L - 2, L // 2):
            t = f * L + off
            if 0 <= t < T:
                r.add(t)
    r.update(np.random.default_rng(seed).integers(0, T, 24).tolist())
    return np.array(sorted(x for x in r if 0 <= x < T))


@pytest.mark.slow
def test_centered_layer_full_size_sampled():
    """B1 H24 21 x 1560 bf16 layer with centred windows and dilation 6 (the
    pages' DSWA dilation), sampled rows of every kind against the oracle."""
    w = WORKLOADS[2]
    dil = 6
    inp = make_inputs(2)
    d = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L,
                             w.window, dil, centered=True)
    torch.cuda.synchronize()
    hs = [0, 23]
    rows = _rows(w.T, w.L, dil, w.window // 2, seed=6)
    sub = {k: inp[k][:1][:, :, hs] for k in ("q", "k", "v", "alpha", "beta")}
    y_ref, S_ref = oracle.hlta_rows(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"],
                                    inp["gates"][:, hs], w.L, w.window, dil, rows, centered=True)
    y_got = host(y[:, torch.as_tensor(rows, device=y.device)][:, :, hs])
    _assert_close(y_got, y_ref, f"centred layer y ({len(rows)} rows x {len(hs)} heads)")
    _assert_close(host(S[:, hs]), S_ref, "centred layer S")


@pytest.mark.slow
def test_centered_fp8_dswa_full_size_sampled():
    """B4 H24 16 x 3600 (the FP8 layer workload's shape): centred DSWA with
    dilation 12 on E4M3 Q/K, one branch, sampled rows against the oracle with
    the same quantisation."""
    w = WORKLOADS[4]
    dil = 12
    print("centred fp8 DSWA full size", flush=True)
    inp = make_inputs(4)
    d = inputs_to_dev(inp)
    q8, qs = K.kairos_fp8_quantize(d["q"])
    k8, ks = K.kairos_fp8_quantize(d["k"])
    out = K.kairos_window_fwd(q8, k8, d["v"], w.L, w.window, dil, q_scales=qs, k_scales=ks,
                              centered=True)
    torch.cuda.synchronize()
    bs, hs = [0, 3], [0, 23]
    rows = _rows(w.T, w.L, dil, w.window // 2, seed=12)
    sel = lambda x: x[bs][:, :, hs]
    _, _, qh = oracle.fp8_quantize_blocks(sel(inp["q"]))
    _, _, kh = oracle.fp8_quantize_blocks(sel(inp["k"]))
    ref = oracle.windowed_attention_rows(qh, kh, sel(inp["v"]), rows, w.L, w.window, dil,
                                         centered=True)
    got = host(out[bs][:, torch.as_tensor(rows, device=out.device)][:, :, hs])
    _assert_close(got, ref, f"centred fp8 DSWA ({len(rows)} rows x {len(bs)}x{len(hs)} heads)")
