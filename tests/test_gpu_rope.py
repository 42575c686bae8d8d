"""GPU parity of RoPE on the windowed branches (kairos_rope, and inside
kairos_hlta_fwd) against the oracle (oracle.rope, oracle.hlta with
rope_base).

Bounds derived from the arithmetic:
* rotated bf16 values: fp32 rotation (angle reduced in fp64; cos/sin within a
  few fp32 ulp: error per element below 1e-6 of the pair's norm) then one
  round to nearest even to bf16 (<= 2^-8 relative), so
  |got - ref| <= 2^-8 |ref| + 2e-6 |pair|.
* rotated E4M3 values: the codes are decided on fp32 rotated values that
  differ from the oracle's fp64 ones by ~1e-7, so a value next to a rounding
  boundary may take the neighbouring code; dequantised values are compared
  within one code step (2^-3 relative for normals, 2^-9 s for subnormals),
  the scales to 1e-6, and flips must stay rare.
* attention outputs: the bf16 / fp8 path tolerances (rel_max <= 2e-2,
  rel_mean <= 5e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import host, inputs_to_dev
from workloads import WORKLOADS, make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3
BASE = 10000.0


def _assert_close(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= TOL_MAX and rmean <= TOL_MEAN, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


def _pair_norm(x):
    n = np.hypot(x[..., 0::2], x[..., 1::2])
    return np.repeat(n, 2, axis=-1)


@pytest.mark.parametrize("T,L,dil,fo", [(300, 100, 1, 0), (64 * 7 + 5, 64, 6, 3), (1000, 40, 12, 0),
                                        (257, 128, 1, 700), (200, 50, 4, 100000)])
def test_rope_bf16_matches_oracle(T, L, dil, fo):
    """Large frame offsets put positions near 1e5-1e7: the fp64 angle reduction is exercised."""
    print(f"rope bf16 T={T} L={L} dil={dil} fo={fo}", flush=True)
    inp = make_custom(2, T, 3, 128, "bf16", seed=T + dil)
    dv = inputs_to_dev(inp)
    out = K.kairos_rope(dv["q"], L, dil, BASE, frame_offset=fo)
    torch.cuda.synchronize()
    pos = oracle.branch_positions(T, L, dil, fo)
    ref = oracle.rope(inp["q"], pos, BASE)
    got = host(out)
    bound = 2.0 ** -8 * np.abs(ref) + 2e-6 * _pair_norm(inp["q"])
    err = np.abs(got - ref)
    print(f"max err/bound {np.max(err / np.maximum(bound, 1e-30)):.3f}", flush=True)
    assert np.all(err <= bound)


def test_rope_bf16_in_place():
    inp = make_custom(1, 333, 2, 128, "bf16", seed=5)
    dv = inputs_to_dev(inp)
    ref = K.kairos_rope(dv["k"], 111, 6, BASE, frame_offset=2)
    K.kairos_rope(dv["k"], 111, 6, BASE, frame_offset=2, out=dv["k"])
    torch.cuda.synchronize()
    assert torch.equal(ref, dv["k"])


@pytest.mark.parametrize("T,L,dil", [(300, 100, 1), (64 * 9 + 17, 64, 6)])
def test_rope_fp8_matches_oracle(T, L, dil):
    print(f"rope fp8 T={T} L={L} dil={dil}", flush=True)
    inp = make_custom(2, T, 3, 128, "bf16", seed=T * dil)
    dv = inputs_to_dev(inp)
    codes, scales = K.kairos_rope(dv["k"], L, dil, BASE, fp8=True)
    torch.cuda.synchronize()
    pos = oracle.branch_positions(T, L, dil, 0)
    rot = oracle.rope(inp["k"], pos, BASE)
    c_ref, s_ref, x_ref = oracle.fp8_quantize_blocks(rot)
    s_got = scales.cpu().numpy()
    np.testing.assert_allclose(s_got, s_ref, rtol=1e-6)
    deq = oracle.e4m3_decode(codes.cpu().numpy()) * np.repeat(
        np.moveaxis(s_got, 2, 1), 64, axis=1)[:, :T, :, None]
    s_tok = np.repeat(np.moveaxis(s_ref, 2, 1), 64, axis=1)[:, :T, :, None].astype(np.float64)
    bound = 2.0 ** -3 * np.abs(rot) + 2.0 ** -9 * s_tok + 1e-6 * np.abs(rot)
    assert np.all(np.abs(deq - rot) <= bound)
    flips = np.mean(codes.cpu().numpy() != c_ref)
    print(f"code flips vs the fp64 oracle: {flips:.2e}", flush=True)
    assert flips < 1e-3


@pytest.mark.parametrize("centered", [False, True])
def test_rope_then_window_branch(centered):
    """kairos_rope + kairos_window_fwd == the oracle's branch with RoPE."""
    B, F, L, H, w, dil, fo = 1, 12, 100, 2, 250, 6, 1
    T = F * L
    inp = make_custom(B, T, H, 128, "bf16", seed=77 + centered)
    dv = inputs_to_dev(inp)
    for dl in (1, dil):
        qr = K.kairos_rope(dv["q"], L, dl, BASE, frame_offset=fo)
        kr = K.kairos_rope(dv["k"], L, dl, BASE, frame_offset=fo)
        out = K.kairos_window_fwd(qr, kr, dv["v"], L, w, dl, frame_offset=fo, centered=centered)
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(inp["q"], inp["k"], inp["v"], L, w, dl, fo, centered,
                                        rope_base=BASE)
        _assert_close(host(out), ref, f"rope branch dil={dl} centred={centered}")


@pytest.mark.parametrize("fp8,centered,dil,fo", [(False, False, 4, 0), (False, True, 6, 2),
                                                 (True, False, 6, 0), (True, True, 12, 5),
                                                 (False, False, 1, 3)])
def test_rope_layer(fp8, centered, dil, fo):
    B, F, L, H, w = 2, 13, 120, 2, 250
    T = F * L
    print(f"rope layer fp8={fp8} centred={centered} dil={dil} fo={fo}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=31 + dil + fo)
    dv = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w,
                             dil, frame_offset=fo, window_qk=K.FP8_E4M3 if fp8 else K.BF16,
                             centered=centered, rope_base=BASE)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, frame_offset=fo, window_qk="fp8" if fp8 else "bf16",
                               centered=centered, rope_base=BASE)
    _assert_close(host(y), y_ref, "rope layer y")
    _assert_close(host(S), S_ref, "rope layer S (RoPE does not touch the gated delta rule)")


def _rows(T, L, seed):
    r = {0, 1, 63, 64, 127, 128, T - 1, T - 2}
    for f in (0, 1, 4, 5, T // L - 1):
        for off in (0, 1, 127, 128, L - 1):
            if 0 <= f * L + off < T:
                r.add(f * L + off)
    r.update(np.random.default_rng(seed).integers(0, T, 20).tolist())
    return np.array(sorted(r))


@pytest.mark.slow
def test_rope_layer_full_size_sampled():
    """B1 H24 21 x 1560 bf16 layer with RoPE (dilation 4, causal), sampled rows."""
    w = WORKLOADS[2]
    inp = make_inputs(2)
    d = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L,
                             w.window, w.dilation, rope_base=BASE)
    torch.cuda.synchronize()
    hs = [0, 23]
    rows = _rows(w.T, w.L, 3)
    sub = {k: inp[k][:1][:, :, hs] for k in ("q", "k", "v", "alpha", "beta")}
    y_ref, S_ref = oracle.hlta_rows(sub["q"], sub["k"], sub["v"], sub["alpha"], sub["beta"],
                                    inp["gates"][:, hs], w.L, w.window, w.dilation, rows,
                                    rope_base=BASE)
    _assert_close(host(y[:, torch.as_tensor(rows, device=y.device)][:, :, hs]), y_ref,
                  f"rope layer y ({len(rows)} rows x {len(hs)} heads)")
    _assert_close(host(S[:, hs]), S_ref, "rope layer S")


@pytest.mark.slow
def test_rope_fp8_branch_full_size_sampled():
    """B4 H24 16 x 3600: RoPE fused with the E4M3 quantiser for the DSWA
    branch (dilation 4), then the branch, sampled rows against the oracle
    (RoPE in fp64, then the same quantiser)."""
    w = WORKLOADS[4]
    print("rope fp8 branch full size", flush=True)
    inp = make_inputs(4)
    d = inputs_to_dev(inp)
    q8, qs = K.kairos_rope(d["q"], w.L, w.dilation, BASE, fp8=True)
    k8, ks = K.kairos_rope(d["k"], w.L, w.dilation, BASE, fp8=True)
    out = K.kairos_window_fwd(q8, k8, d["v"], w.L, w.window, w.dilation, q_scales=qs, k_scales=ks)
    torch.cuda.synchronize()
    bs, hs = [0, 3], [0, 23]
    rows = _rows(w.T, w.L, 4)
    sel = lambda x: x[bs][:, :, hs]
    pos = oracle.branch_positions(w.T, w.L, w.dilation, 0)
    _, _, qh = oracle.fp8_quantize_blocks(oracle.rope(sel(inp["q"]), pos, BASE))
    _, _, kh = oracle.fp8_quantize_blocks(oracle.rope(sel(inp["k"]), pos, BASE))
    ref = oracle.windowed_attention_rows(qh, kh, sel(inp["v"]), rows, w.L, w.window, w.dilation)
    got = host(out[bs][:, torch.as_tensor(rows, device=out.device)][:, :, hs])
    _assert_close(got, ref, f"rope fp8 DSWA ({len(rows)} rows x {len(bs)}x{len(hs)} heads)")
