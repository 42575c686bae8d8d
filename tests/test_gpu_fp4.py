"""GPU parity of the 4-bit (FP4 E2M1) windowed Q/K path: the block quantiser
bit for bit against the oracle (codes packed two per byte, scales), and the
windowed branches and the layer on 4-bit Q/K against the oracle with the
same quantisation (rel_max <= 2e-2, rel_mean <= 5e-3).
"""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import dev_bf16, host, inputs_to_dev
from workloads import WORKLOADS, make_custom, make_inputs, to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3


def _assert_close(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= TOL_MAX and rmean <= TOL_MEAN, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


def _check_quantiser(xb):
    codes, scales = K.kairos_fp4_quantize(dev_bf16(xb))
    torch.cuda.synchronize()
    c_ref, s_ref, _ = oracle.fp4_quantize_blocks(bf16_bits_to_f32(xb))
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), oracle.fp4_pack(c_ref))
    return s_ref


@pytest.mark.parametrize("d", [32, 64, 128])
@pytest.mark.parametrize("T", [1, 150])
def test_fp4_quantize_random(d, T):
    rng = np.random.default_rng(d + T)
    x = rng.standard_normal((2, T, 3, d)).astype(np.float32) * 3
    xb = to_bf16_bits(x)
    xb[0, :min(T, 64), 1] = 0                       # an all-zero block
    _check_quantiser(xb)


def test_fp4_quantize_wide_range():
    rng = np.random.default_rng(7)
    T = 64 * 4 + 9
    x = rng.standard_normal((2, T, 5, 128)) * np.exp2(rng.uniform(-20, 10, size=(2, T, 5, 128)))
    _check_quantiser(to_bf16_bits(x.astype(np.float32)))


def test_fp4_quantize_every_bf16_value():
    """Every finite bf16 value of magnitude <= 6, both signs, in blocks whose
    maximum is 6 (s = 1, the quotient is the value): every rounding tie, the
    subnormal code and the saturation edge."""
    top = 0x40C0                                    # bf16 pattern of 6.0
    mags = np.arange(0, top + 1, dtype=np.uint16)
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    per_block = 64 * 128 - 1
    nblk = -(-len(vals) // per_block)
    blocks = np.zeros((nblk, 64 * 128), dtype=np.uint16)
    blocks[:, 0] = top
    flat = blocks[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(nblk, per_block)
    s_ref = _check_quantiser(blocks.reshape(1, nblk * 64, 1, 128))
    assert np.all(s_ref == 1.0)


CASES = [
    # B, F, L, H, w, dil, frame_offset, centred
    (1, 7, 100, 2, 150, 3, 0, False),
    (2, 6, 64, 1, 64, 4, 0, False),
    (1, 9, 130, 1, 300, 4, 3, False),
    (1, 12, 100, 2, 300, 6, 0, True),
    (1, 40, 24, 2, 50, 6, 0, False),           # frames shorter than a key block
]


@pytest.mark.parametrize("B,F,L,H,w,dil,fo,centered", CASES)
def test_fp4_window_branch(B, F, L, H, w, dil, fo, centered):
    T = F * L
    print(f"fp4 window B={B} F={F} L={L} w={w} dil={dil} fo={fo} centred={centered}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=F * L + w + 4)
    dv = inputs_to_dev(inp)
    q4, qs = K.kairos_fp4_quantize(dv["q"])
    k4, ks = K.kairos_fp4_quantize(dv["k"])
    _, _, qh = oracle.fp4_quantize_blocks(inp["q"])
    _, _, kh = oracle.fp4_quantize_blocks(inp["k"])
    for dl in sorted({1, dil}):
        out = K.kairos_window_fwd(q4, k4, dv["v"], L, w, dl, frame_offset=fo, q_scales=qs,
                                  k_scales=ks, centered=centered)
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(qh, kh, inp["v"], L, w, dl, fo, centered)
        _assert_close(host(out), ref, f"fp4 window dil={dl}")


@pytest.mark.parametrize("centered,rope", [(False, False), (True, False), (False, True)])
def test_fp4_layer(centered, rope):
    B, F, L, H, w, dil = 2, 8, 150, 2, 200, 4
    T = F * L
    print(f"fp4 layer centred={centered} rope={rope}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=404 + centered + 2 * rope)
    dv = inputs_to_dev(inp)
    base = 1e4 if rope else 0.0
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w,
                             dil, window_qk=K.FP4_E2M1, centered=centered, rope_base=base)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk="fp4", centered=centered,
                               rope_base=base if rope else None)
    _assert_close(host(y), y_ref, "fp4 layer y")
    _assert_close(host(S), S_ref, "fp4 layer S")


@pytest.mark.slow
def test_fp4_layer_full_size_sampled():
    """B4 H24 16 x 3600 (the FP8 layer workload's shape) with 4-bit windowed
    Q/K, sampled rows against the oracle with the same quantisation."""
    w = WORKLOADS[4]
    print("fp4 layer full size", flush=True)
    inp = make_inputs(4)
    d = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L,
                             w.window, w.dilation, window_qk=K.FP4_E2M1)
    torch.cuda.synchronize()
    bs, hs = [0, 3], [0, 23]
    sel = lambda x: x[bs][:, :, hs]
    rows = np.array(sorted({0, 1, 63, 64, 127, 128, w.L - 1, w.L, 2 * w.L + 5, w.T - 1, w.T - 2}
                           | set(np.random.default_rng(9).integers(0, w.T, 20).tolist())))
    o_ref, S_ref = oracle.gdn_recurrent(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]),
                                        inp["alpha"][bs][:, :, hs], inp["beta"][bs][:, :, hs])
    y_ref, _ = oracle.hlta_rows(sel(inp["q"]), sel(inp["k"]), sel(inp["v"]), inp["alpha"][bs][:, :, hs],
                                inp["beta"][bs][:, :, hs], inp["gates"][:, hs], w.L, w.window,
                                w.dilation, rows, window_qk="fp4", o_gdn=o_ref)
    y_got = host(y[bs][:, torch.as_tensor(rows, device=y.device)][:, :, hs])
    _assert_close(y_got, y_ref, f"fp4 layer y ({len(rows)} rows x {len(bs)}x{len(hs)} heads)")
    _assert_close(host(S[bs][:, hs]), S_ref, "fp4 layer S")
