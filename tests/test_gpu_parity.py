"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs, at sizes the oracle finishes in seconds that still span
several tiles, chunks and ragged tails.

Tolerances (relative to the reference tensor's magnitude, see conftest):
fp32 path rel_max <= 1e-4; bf16 / fp8 paths rel_max <= 2e-2 and
rel_mean <= 5e-3, on outputs and on the final state.  FP8 results are
compared with the oracle that applies the same quantisation; quantiser codes
and scales are compared bit for bit.
"""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import dev_bf16, dev_f32, host, inputs_to_dev
from workloads import make_custom, make_inputs

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3


def _assert_close(got, ref, what, tmax=TOL_MAX, tmean=TOL_MEAN):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= tmax and rmean <= tmean, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


# ------------------------------------------------------------------ gated delta rule

def test_gdn_f32_workload0():
    inp = make_inputs(0)
    d = inputs_to_dev(inp, "f32")
    out, S = K.kairos_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"])
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    _assert_close(host(out), o_ref, "o", 1e-4, 1e-4)
    _assert_close(host(S), S_ref, "S", 1e-4, 1e-4)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_gdn_f32_with_state(d):
    inp = make_custom(2, 77, 3, d, "f32", seed=11, alpha_kind="uniform", beta_kind="uniform")
    S0 = np.random.default_rng(3).standard_normal((2, 3, d, d)).astype(np.float32)
    dv = inputs_to_dev(inp, "f32")
    out, S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dev_f32(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0)
    _assert_close(host(out), o_ref, "o", 1e-4, 1e-4)
    _assert_close(host(S), S_ref, "S", 1e-4, 1e-4)


@pytest.mark.parametrize("B,T,H,d", [(1, 200, 2, 128), (2, 130, 3, 64), (1, 64, 1, 128),
                                     (1, 1, 2, 128), (1, 65, 16, 128), (3, 300, 8, 128)])
def test_gdn_bf16_chunked(B, T, H, d):
    inp = make_custom(B, T, H, d, "bf16", seed=100 + T + H)
    S0 = (np.random.default_rng(T).standard_normal((B, H, d, d)) * 0.5).astype(np.float32)
    dv = inputs_to_dev(inp)
    out, S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dev_f32(S0))
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0)
    _assert_close(host(out), o_ref, f"o B{B} T{T} H{H} d{d}")
    _assert_close(host(S), S_ref, f"S B{B} T{T} H{H} d{d}")


def test_gdn_bf16_zero_length_copies_state():
    S0 = np.random.default_rng(5).standard_normal((1, 2, 128, 128)).astype(np.float32)
    e = torch.empty((1, 0, 2, 128), dtype=torch.bfloat16, device="cuda:0")
    g = torch.empty((1, 0, 2), dtype=torch.float32, device="cuda:0")
    out, S = K.kairos_gdn_fwd(e, e, e, g, g, dev_f32(S0))
    torch.cuda.synchronize()
    np.testing.assert_array_equal(host(S), S0)


def test_gdn_bf16_retrieval_pin():
    """alpha = beta = 1 with orthonormal keys and q = k: o_t = v_t (bf16 path)."""
    rng = np.random.default_rng(9)
    d, T = 128, 128
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    kk = Qm.T.astype(np.float32)[None, :, None, :]
    from workloads import to_bf16_bits, bf16_bits_to_f32
    kb = to_bf16_bits(kk)
    vb = to_bf16_bits(rng.standard_normal((1, T, 1, d)).astype(np.float32))
    ones = dev_f32(np.ones((1, T, 1), np.float32))
    out, S = K.kairos_gdn_fwd(dev_bf16(kb), dev_bf16(kb), dev_bf16(vb), ones, ones)
    torch.cuda.synchronize()
    o_ref, _ = oracle.gdn_recurrent(bf16_bits_to_f32(kb), bf16_bits_to_f32(kb), bf16_bits_to_f32(vb),
                                    np.ones((1, T, 1)), np.ones((1, T, 1)))
    _assert_close(host(out), o_ref, "retrieval o")


# ------------------------------------------------------------------ fp8 quantiser

@pytest.mark.parametrize("T", [1, 64, 150, 1000])
def test_fp8_quantize_bit_exact(T):
    inp = make_custom(2, T, 3, 128, "bf16", seed=T)
    x = inp["q"] * np.float32(7.0)
    from workloads import to_bf16_bits, bf16_bits_to_f32
    xb = to_bf16_bits(x)
    xb[0, :min(T, 64), 1] = 0                       # an all-zero block
    codes, scales = K.kairos_fp8_quantize(dev_bf16(xb))
    torch.cuda.synchronize()
    c_ref, s_ref, _ = oracle.fp8_quantize_blocks(bf16_bits_to_f32(xb))
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


@pytest.mark.parametrize("d", [32, 64, 128])
def test_fp8_quantize_wide_range(d):
    """Values spread over 2^-20 .. 2^10 (non-power-of-two scales, many
    quotients in the E4M3 subnormal range and below), every head size, a
    ragged last block: bit-exact against the oracle."""
    from workloads import to_bf16_bits, bf16_bits_to_f32
    rng = np.random.default_rng(d)
    T = 64 * 5 + 23
    x = rng.standard_normal((2, T, 5, d)) * np.exp2(rng.uniform(-20, 10, size=(2, T, 5, d)))
    xb = to_bf16_bits(x.astype(np.float32))
    codes, scales = K.kairos_fp8_quantize(dev_bf16(xb))
    torch.cuda.synchronize()
    c_ref, s_ref, _ = oracle.fp8_quantize_blocks(bf16_bits_to_f32(xb))
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


def test_fp8_quantize_every_bf16_value():
    """Every finite bf16 value of magnitude <= 448 (both signs, both zeros,
    subnormals), placed in blocks whose maximum is 448 so that s = 1 and the
    quotient is the value itself: the codes match the oracle bit for bit.
    This covers every E4M3 rounding tie, the subnormal range and the
    saturation edge of the encoding."""
    from workloads import bf16_bits_to_f32
    top = 0x43E0                                   # bf16 pattern of 448
    mags = np.arange(0, top + 1, dtype=np.uint16)
    vals = np.concatenate([mags, mags | np.uint16(0x8000)])
    per_block = 64 * 128 - 1
    nblk = -(-len(vals) // per_block)
    blocks = np.zeros((nblk, 64 * 128), dtype=np.uint16)
    blocks[:, 0] = top
    flat = blocks[:, 1:].reshape(-1)
    flat[:len(vals)] = vals
    blocks[:, 1:] = flat.reshape(nblk, per_block)
    xb = blocks.reshape(1, nblk * 64, 1, 128)     # [B, T, H, d]: block = 64 tokens x 128
    codes, scales = K.kairos_fp8_quantize(dev_bf16(xb))
    torch.cuda.synchronize()
    c_ref, s_ref, _ = oracle.fp8_quantize_blocks(bf16_bits_to_f32(xb))
    assert np.all(s_ref == 1.0)
    np.testing.assert_array_equal(scales.cpu().numpy(), s_ref)
    np.testing.assert_array_equal(codes.cpu().numpy(), c_ref)


# ------------------------------------------------------------------ windowed branches

WIN_CASES = [
    # B, F, L, H, w, dil, frame_offset  (T = F*L, last frame full)
    (1, 7, 100, 2, 150, 3, 0),
    (1, 5, 200, 2, 200, 2, 1),
    (2, 6, 64, 1, 64, 4, 0),
    (1, 9, 130, 1, 300, 4, 3),
    (1, 3, 300, 1, 1000, 1, 0),
]


@pytest.mark.parametrize("B,F,L,H,w,dil,fo", WIN_CASES)
def test_window_single_branch(B, F, L, H, w, dil, fo):
    T = F * L
    inp = make_custom(B, T, H, 128, "bf16", seed=F * L + w)
    dv = inputs_to_dev(inp)
    for dl in (1, dil):
        out = K.kairos_window_fwd(dv["q"], dv["k"], dv["v"], L, w, dl, frame_offset=fo)
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(inp["q"], inp["k"], inp["v"], L, w, dl, fo)
        _assert_close(host(out), ref, f"window dil={dl}")


def test_window_partial_last_frame():
    B, H, L, w, dil = 1, 2, 100, 120, 2
    T = 4 * L + 37
    inp = make_custom(B, T, H, 128, "bf16", seed=77)
    dv = inputs_to_dev(inp)
    for dl in (1, dil):
        out = K.kairos_window_fwd(dv["q"], dv["k"], dv["v"], L, w, dl)
        torch.cuda.synchronize()
        _assert_close(host(out), oracle.windowed_attention(inp["q"], inp["k"], inp["v"], L, w, dl),
                      f"partial frame dil={dl}")


# E4M3 Q/K: key blocks follow frame ends and the call's 64-token blocks
# (frames of at least 64 tokens), or 64 group positions with per-key scales
# (shorter frames); frame offsets, frame lengths that 64 does not divide, a
# partial last frame and short frames move those boundaries around
FP8_WIN_CASES = WIN_CASES + [(1, 40, 24, 2, 50, 6, 0), (1, 12, 70, 2, 130, 4, 5)]


def _fp8_branch_check(B, T, L, H, w, dil, fo, seed):
    inp = make_custom(B, T, H, 128, "bf16", seed=seed)
    dv = inputs_to_dev(inp)
    q8, qs = K.kairos_fp8_quantize(dv["q"])
    k8, ks = K.kairos_fp8_quantize(dv["k"])
    _, _, qh = oracle.fp8_quantize_blocks(inp["q"])
    _, _, kh = oracle.fp8_quantize_blocks(inp["k"])
    for dl in sorted({1, dil}):
        out = K.kairos_window_fwd(q8, k8, dv["v"], L, w, dl, frame_offset=fo, q_scales=qs, k_scales=ks)
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(qh, kh, inp["v"], L, w, dl, fo)
        _assert_close(host(out), ref, f"fp8 window T={T} L={L} dil={dl} fo={fo}")


@pytest.mark.parametrize("B,F,L,H,w,dil,fo", FP8_WIN_CASES)
def test_window_single_branch_fp8(B, F, L, H, w, dil, fo):
    _fp8_branch_check(B, F * L, L, H, w, dil, fo, F * L + w + 1)


def test_window_partial_last_frame_fp8():
    _fp8_branch_check(1, 4 * 100 + 37, 100, 2, 120, 2, 0, 78)


@pytest.mark.parametrize("qf", ["bf16", "fp8", "fp4"])
@pytest.mark.parametrize("gain", [64.0, 1024.0])
def test_window_wide_scores(qf, gain):
    """Queries scaled by a power of two so that scores spread over tens to
    hundreds of log2 units: the running maximum keeps rising from block to
    block, which sends blocks formed against the running maximum alone back
    to the maximum and rescale path (and, past a few such blocks, stops
    those attempts for the wave)."""
    B, F, L, H, w, dil = 1, 6, 200, 2, 500, 2
    T = F * L
    print(f"wide scores {qf} gain={gain}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=int(gain) + 11)
    from workloads import to_bf16_bits
    inp["q"] = inp["q"] * np.float32(gain)                 # exact: gain is a power of two
    inp["q_bits"] = to_bf16_bits(inp["q"])
    dv = inputs_to_dev(inp)
    for dl in (1, dil):
        if qf == "bf16":
            out = K.kairos_window_fwd(dv["q"], dv["k"], dv["v"], L, w, dl)
            qh, kh = inp["q"], inp["k"]
        elif qf == "fp8":
            q8, qs = K.kairos_fp8_quantize(dv["q"])
            k8, ks = K.kairos_fp8_quantize(dv["k"])
            out = K.kairos_window_fwd(q8, k8, dv["v"], L, w, dl, q_scales=qs, k_scales=ks)
            qh, kh = oracle.fp8_quantize_blocks(inp["q"])[2], oracle.fp8_quantize_blocks(inp["k"])[2]
        else:
            q4, qs = K.kairos_fp4_quantize(dv["q"])
            k4, ks = K.kairos_fp4_quantize(dv["k"])
            out = K.kairos_window_fwd(q4, k4, dv["v"], L, w, dl, q_scales=qs, k_scales=ks)
            qh, kh = oracle.fp4_quantize_blocks(inp["q"])[2], oracle.fp4_quantize_blocks(inp["k"])[2]
        torch.cuda.synchronize()
        ref = oracle.windowed_attention(qh, kh, inp["v"], L, w, dl)
        _assert_close(host(out), ref, f"wide scores {qf} gain={gain} dil={dl}")


@pytest.mark.parametrize("B,F,L,H,w,dil,fo", WIN_CASES[:3])
def test_hlta_small(B, F, L, H, w, dil, fo):
    T = F * L
    inp = make_custom(B, T, H, 128, "bf16", seed=7 + F * L)
    dv = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"],
                             L, w, dil, frame_offset=fo)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, frame_offset=fo)
    _assert_close(host(y), y_ref, "y")
    _assert_close(host(S), S_ref, "S")


def test_hlta_fp8_small():
    B, F, L, H, w, dil = 2, 6, 150, 2, 200, 4
    T = F * L
    inp = make_custom(B, T, H, 128, "bf16", seed=321)
    dv = inputs_to_dev(inp)
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"],
                             L, w, dil, window_qk=K.FP8_E4M3)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk="fp8")
    _assert_close(host(y), y_ref, "y fp8")
    _assert_close(host(S), S_ref, "S fp8")


@pytest.mark.parametrize("qf", ["bf16", "fp8"])
def test_hlta_window_stage_wide_scores(qf):
    """The two-branch window stage (both windowed branches, gates, and a given
    GDN output, here zero) with queries scaled by 1024: scores spread over
    hundreds of log2 units in both branches of one kernel."""
    from workloads import to_bf16_bits
    B, F, L, H, w, dil = 1, 6, 150, 2, 200, 4
    T = F * L
    print(f"wide-score window stage {qf}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=907)
    inp["q"] = inp["q"] * np.float32(1024.0)               # exact: a power of two
    inp["q_bits"] = to_bf16_bits(inp["q"])
    dv = inputs_to_dev(inp)
    o_gdn = torch.zeros_like(dv["v"])
    ws = torch.empty(4 * B * T * H * 129, dtype=torch.uint8, device="cuda:0")
    if qf == "bf16":
        y = K.kairos_hlta_window_fwd(dv["q"], dv["k"], dv["v"], o_gdn, dv["gates"], L, w, dil, workspace=ws)
    else:
        q8, qs = K.kairos_fp8_quantize(dv["q"])
        k8, ks = K.kairos_fp8_quantize(dv["k"])
        y = K.kairos_hlta_window_fwd(q8, k8, dv["v"], o_gdn, dv["gates"], L, w, dil, q_scales=qs,
                                     k_scales=ks, workspace=ws)
    torch.cuda.synchronize()
    y_ref, _ = oracle.hlta_rows(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"], L, w,
                                dil, np.arange(T), window_qk=qf, o_gdn=np.zeros_like(inp["v"]))
    _assert_close(host(y), y_ref, f"wide-score window stage {qf}")


@pytest.mark.parametrize("rope_base,dil", [(0.0, 2), (1e4, 2), (1e4, 1), (500.0, 3)])
def test_streaming_equals_full_run(rope_base, dil):
    """Recurrent state passing: frames fed one call at a time with the GDN state
    carried and a key/value ring equal one full-length oracle run; with RoPE
    the ring keeps each branch's rotated keys (absolute positions)."""
    B, F, L, H, w = 1, 9, 96, 2, 150
    T = F * L
    print(f"stream rope_base={rope_base} dil={dil}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=55 + dil)
    dv = inputs_to_dev(inp)
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))
    k_ring = torch.zeros(K.ring_key_shape(B, R, L, H, 128, dil, rope_base), dtype=torch.bfloat16,
                         device="cuda:0")
    v_ring = torch.zeros((B, R, L, H, 128), dtype=torch.bfloat16, device="cuda:0")
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ys = []
    for f in range(F):
        sl = slice(f * L, (f + 1) * L)
        y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                 dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                 dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                 frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                 k_ring=k_ring, v_ring=v_ring, rope_base=rope_base)
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, rope_base=rope_base or None)
    _assert_close(np.concatenate([host(y) for y in ys], axis=1), y_ref, "stream y")
    _assert_close(host(state), S_ref, "stream S")


# ------------------------------------------------------------------ quantised windows per frame

@pytest.mark.parametrize("fmt,L,F,w,dil,rope", [("fp8", 100, 6, 150, 2, 0.0), ("fp4", 100, 6, 150, 2, 0.0),
                                                ("fp8", 40, 7, 90, 3, 0.0), ("fp8", 128, 4, 200, 2, 1e4)])
def test_layer_frame_blocks_matches_oracle(fmt, L, F, w, dil, rope):
    """Quantisation blocks that restart at every frame (64 does not divide L
    here, or L < 64), in one call, against the oracle's "frames" reading."""
    B, H = 1, 2
    T = F * L
    print(f"frame blocks {fmt} L{L} F{F} rope={rope}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=70 + L + F)
    dv = inputs_to_dev(inp)
    wq = K.FP8_E4M3 if fmt == "fp8" else K.FP4_E2M1
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                             window_qk=wq, qk_blocks=K.QK_BLOCKS_FRAMES, rope_base=rope)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=fmt, qk_blocks="frames", rope_base=rope or None)
    _assert_close(host(y), y_ref, "y")
    _assert_close(host(S), S_ref, "S")


@pytest.mark.parametrize("fmt,rope,dil,L", [("fp8", 0.0, 2, 96), ("fp4", 0.0, 2, 96), ("fp8", 1e4, 2, 96),
                                            ("fp4", 1e4, 3, 50), ("fp8", 0.0, 1, 40)])
def test_streaming_quantised_equals_full_run(fmt, rope, dil, L):
    """A rollout with quantised Q/K fed one frame per call (the ring keeps the
    keys' codes and block scales, rotated first with RoPE) equals one
    full-length oracle run with per-frame quantisation blocks."""
    B, F, H, w = 1, 9, 2, int(1.6 * L)
    T = F * L
    print(f"stream {fmt} rope={rope} dil={dil} L{L}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=80 + dil + L)
    dv = inputs_to_dev(inp)
    wq = K.FP8_E4M3 if fmt == "fp8" else K.FP4_E2M1
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))
    k_ring, v_ring = K.alloc_rings(B, L, H, 128, w, dil, R, wq, rope, K.QK_BLOCKS_FRAMES)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ys = []
    for f in range(F):
        sl = slice(f * L, (f + 1) * L)
        y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                 dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                 dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                 frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                 k_ring=k_ring, v_ring=v_ring, rope_base=rope, window_qk=wq,
                                 qk_blocks=K.QK_BLOCKS_FRAMES)
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=fmt, qk_blocks="frames", rope_base=rope or None)
    _assert_close(np.concatenate([host(y) for y in ys], axis=1), y_ref, "stream y")
    _assert_close(host(state), S_ref, "stream S")


# ------------------------------------------------------------------ more streaming and frame-block cases

@pytest.mark.parametrize("fmt,rope,dil", [("bf16", 1e4, 2), ("fp8", 1e4, 2), ("fp4", 0.0, 3)])
def test_streaming_batched_equals_full_run(fmt, rope, dil):
    """Two batch rows through the ring (the ring's and the scales' batch
    strides), fed one frame per call, against one full-length oracle run."""
    B, F, L, H = 2, 7, 96, 2
    w = int(1.6 * L)
    T = F * L
    print(f"stream batched {fmt} rope={rope} dil={dil}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=91 + dil)
    dv = inputs_to_dev(inp)
    wq = {"bf16": K.BF16, "fp8": K.FP8_E4M3, "fp4": K.FP4_E2M1}[fmt]
    qb = K.QK_BLOCKS_FRAMES if fmt != "bf16" else K.QK_BLOCKS_TOKENS
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))
    k_ring, v_ring = K.alloc_rings(B, L, H, 128, w, dil, R, wq, rope, qb)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ys = []
    for f in range(F):
        sl = slice(f * L, (f + 1) * L)
        y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                 dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                 dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                 frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                 k_ring=k_ring, v_ring=v_ring, rope_base=rope, window_qk=wq, qk_blocks=qb)
        ys.append(y)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=fmt, qk_blocks="frames" if fmt != "bf16" else "tokens",
                               rope_base=rope or None)
    _assert_close(np.concatenate([host(y) for y in ys], axis=1), y_ref, "stream y")
    _assert_close(host(state), S_ref, "stream S")


@pytest.mark.parametrize("fmt,L,F,extra,w,dil,centered", [
    ("fp8", 100, 5, 37, 150, 2, False),     # partial last frame: its blocks end with it
    ("fp4", 40, 6, 23, 90, 3, False),       # frames shorter than a block, partial last frame
    ("fp8", 128, 4, 0, 200, 3, True),       # centred windows on frame-aligned blocks
    ("fp8", 100, 5, 61, 160, 2, True),
])
def test_layer_frame_blocks_partial_and_centred(fmt, L, F, extra, w, dil, centered):
    B, H = 1, 2
    T = F * L + extra
    print(f"frame blocks {fmt} L{L} T{T} centred={centered}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=130 + L + extra)
    dv = inputs_to_dev(inp)
    wq = K.FP8_E4M3 if fmt == "fp8" else K.FP4_E2M1
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                             window_qk=wq, qk_blocks=K.QK_BLOCKS_FRAMES, centered=centered)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=fmt, qk_blocks="frames", centered=centered)
    _assert_close(host(y), y_ref, "y")
    _assert_close(host(S), S_ref, "S")


@pytest.mark.parametrize("fmt,blocks,L,F,w,dil,fo,centered", [
    ("bf16", "tokens", 100, 5, 40, 2, 0, False),   # window shorter than a frame
    ("fp8", "tokens", 150, 6, 30, 4, 1, False),
    ("fp8", "frames", 128, 4, 50, 3, 0, True),
    ("fp4", "frames", 96, 5, 20, 2, 2, True),
    ("fp8", "frames", 100, 4, 1, 2, 0, False),     # each query sees only itself
])
def test_hlta_window_shorter_than_frame(fmt, blocks, L, F, w, dil, fo, centered):
    """Both windowed branches with a window shorter than a frame: deep in a
    frame neither branch reaches another frame, so only the frame's own keys
    are scored, and the two branches' key sets within the frame coincide."""
    B, H = 1, 2
    T = F * L
    print(f"short window {fmt}/{blocks} L{L} F{F} w{w} dil{dil} fo{fo} centred={centered}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=900 + L + w)
    dv = inputs_to_dev(inp)
    wq = {"bf16": K.BF16, "fp8": K.FP8_E4M3, "fp4": K.FP4_E2M1}[fmt]
    qb = K.QK_BLOCKS_FRAMES if blocks == "frames" else K.QK_BLOCKS_TOKENS
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                             frame_offset=fo, window_qk=wq, qk_blocks=qb, centered=centered)
    torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, frame_offset=fo, window_qk=fmt, qk_blocks=blocks,
                               centered=centered)
    _assert_close(host(y), y_ref, "y")
    _assert_close(host(S), S_ref, "S")


@pytest.mark.parametrize("fmt,rope", [("fp8", 1e4), ("bf16", 0.0)])
def test_streaming_with_context_equals_full_run(fmt, rope):
    """A rollout whose frame calls take the overlapped schedule of a context
    (the GDN branch on the side stream beside the window kernel, the
    pre-passes and the combine on the caller's stream), with the ring, against
    one full-length oracle run."""
    B, F, L, H, w, dil = 1, 7, 96, 2, 150, 2
    T = F * L
    print(f"stream ctx {fmt} rope={rope}", flush=True)
    inp = make_custom(B, T, H, 128, "bf16", seed=97)
    dv = inputs_to_dev(inp)
    wq = K.FP8_E4M3 if fmt == "fp8" else K.BF16
    qb = K.QK_BLOCKS_FRAMES if fmt == "fp8" else K.QK_BLOCKS_TOKENS
    R = K.kairos_hlta_ring_frames_required(K.hlta_desc(B, L, H, 128, L, w, dil))
    k_ring, v_ring = K.alloc_rings(B, L, H, 128, w, dil, R, wq, rope, qb)
    state = torch.zeros((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    ys = []
    with K.Context() as ctx:
        for f in range(F):
            sl = slice(f * L, (f + 1) * L)
            y, _ = K.kairos_hlta_fwd(dv["q"][:, sl].contiguous(), dv["k"][:, sl].contiguous(),
                                     dv["v"][:, sl].contiguous(), dv["alpha"][:, sl].contiguous(),
                                     dv["beta"][:, sl].contiguous(), dv["gates"], L, w, dil,
                                     frame_offset=f, state_in=state, state_out=state, ring_frames=R,
                                     k_ring=k_ring, v_ring=v_ring, rope_base=rope, window_qk=wq,
                                     qk_blocks=qb, ctx=ctx)
            ys.append(y)
        torch.cuda.synchronize()
    y_ref, S_ref = oracle.hlta(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], inp["gates"],
                               L, w, dil, window_qk=fmt, qk_blocks="frames" if fmt == "fp8" else "tokens",
                               rope_base=rope or None)
    _assert_close(np.concatenate([host(y) for y in ys], axis=1), y_ref, "stream y")
    _assert_close(host(state), S_ref, "stream S")


@pytest.mark.parametrize("fmt,B,F,extra,L,H,w,dil,centered,use_ctx", [
    ("fp8", 1, 5, 37, 100, 2, 150, 2, False, False),
    ("fp8", 2, 4, 0, 128, 3, 200, 3, False, False),
    ("fp4", 1, 6, 23, 96, 2, 130, 2, True, False),
    ("fp8", 1, 3, 0, 64, 1, 64, 1, False, False),
    ("fp8", 1, 8, 0, 1024, 8, 1000, 4, False, True),    # operand pre-passes beside the scan
    ("fp4", 1, 8, 0, 1024, 8, 1000, 4, False, True),
])
def test_layer_equals_its_parts_bitwise(fmt, B, F, extra, L, H, w, dil, centered, use_ctx):
    """A quantised layer call equals, bit for bit, the chain of its public
    parts: the gated delta rule, the standalone quantisers of q and k (64-token
    blocks) and the windowed stage fed with their outputs."""
    T = F * L + extra
    print(f"layer vs parts {fmt} B{B} T{T} L{L} H{H} w{w} dil{dil} centred={centered} ctx={use_ctx}", flush=True)
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=700 + T + H))
    wq = K.FP8_E4M3 if fmt == "fp8" else K.FP4_E2M1
    ctx = K.Context() if use_ctx else None
    y, S = K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                             window_qk=wq, centered=centered, ctx=ctx)
    o_gdn, S2 = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"])
    quant = K.kairos_fp8_quantize if fmt == "fp8" else K.kairos_fp4_quantize
    cq, sq = quant(dv["q"])
    ck, sk = quant(dv["k"])
    y2 = K.kairos_hlta_window_fwd(cq, ck, dv["v"], o_gdn, dv["gates"], L, w, dil, q_scales=sq, k_scales=sk,
                                  centered=centered, window_qk=wq)
    torch.cuda.synchronize()
    if ctx is not None:
        ctx.close()
    assert torch.equal(S, S2), "final state differs from the gated delta rule alone"
    same = (y.view(torch.int16) == y2.view(torch.int16))
    assert bool(same.all()), f"{int((~same).sum())} of {same.numel()} outputs differ from the chained parts"
