"""Pins of the CPU oracle against facts fixed by the paper and by mathematics.

None of these checks re-types the oracle's own formula: each compares it with
a closed form, an invariant, a brute force, a second formulation or a
library routine (torch autograd, torch scaled-dot-product attention, torch's
float8_e4m3fn cast).  Source of the facts: Kairos paper (arXiv 2606.16533,
HTML v3), Sec. 2.2.1 (Eq. 1-6, step 4), Sec. 2.2.2 (Eq. 7-8), Sec. 2.3.2
(Remark 2, Eq. 18) and the long-horizon "recurrent state passing" paragraph.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from oracle import (gdn_recurrent, gdn_literal_eq6, gdn_chunked, windowed_attention,
                    windowed_attention_rows, window_bruteforce, dswa_reshape,
                    e4m3_round, e4m3_encode, e4m3_decode, fp8_quantize_blocks, hlta, hlta_rows)
from workloads import make_custom, WORKLOADS, make_inputs, round_bf16, to_bf16_bits, bf16_bits_to_f32

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _rand_inputs(rng, B, T, H, d, alpha=(0.8, 0.999), beta=(0.05, 1.0)):
    q = rng.standard_normal((B, T, H, d))
    k = rng.standard_normal((B, T, H, d))
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((B, T, H, d))
    a = rng.uniform(*alpha, size=(B, T, H))
    b = rng.uniform(*beta, size=(B, T, H))
    return q, k, v, a, b


# ----------------------------------------------------------------- gated delta rule

def test_gdn_retrieval_orthonormal_keys():
    """alpha = beta = 1 and orthonormal keys: every written value is retrieved
    exactly, and querying with the current key returns the current value
    (read-out after the update, step 4)."""
    rng = np.random.default_rng(1)
    d, T = 16, 16
    Qm, _ = np.linalg.qr(rng.standard_normal((d, d)))
    k = Qm.T[None, :, None, :]                 # T orthonormal keys
    v = rng.standard_normal((1, T, 1, d))
    o, S = gdn_recurrent(k, k, v, np.ones((1, T, 1)), np.ones((1, T, 1)))
    np.testing.assert_allclose(o[0, :, 0], v[0, :, 0], atol=1e-12)
    for i in range(T):
        np.testing.assert_allclose(S[0, 0] @ k[0, i, 0], v[0, i, 0], atol=1e-12)


def test_gdn_beta_one_overwrites_for_any_alpha():
    """With beta_t = 1 the update stores v_t exactly at key k_t whatever the
    decay and the history: S_t k_t = v_t.  This separates the canonical
    decay placement from the printed Eq. 6 (which gives v_t - (1-a_t) S_{t-1} k_t)."""
    rng = np.random.default_rng(2)
    q, k, v, a, _ = _rand_inputs(rng, 2, 20, 3, 8, alpha=(0.3, 0.9))
    S0 = rng.standard_normal((2, 3, 8, 8))
    o, _ = gdn_recurrent(k, k, v, a, np.ones_like(a), S0)
    np.testing.assert_allclose(o, v, atol=1e-12)
    o_lit, _ = gdn_literal_eq6(k, k, v, a, np.ones_like(a), S0)
    assert np.max(np.abs(o_lit - v)) > 1e-3


def test_gdn_key_collision():
    """Writing (k, v1) then (k, v2) with alpha = beta = 1 leaves S k = v2."""
    rng = np.random.default_rng(3)
    d = 8
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    k = np.stack([kk, kk])[None, :, None, :]
    v = rng.standard_normal((1, 2, 1, d))
    _, S = gdn_recurrent(k, k, v, np.ones((1, 2, 1)), np.ones((1, 2, 1)))
    np.testing.assert_allclose(S[0, 0] @ kk, v[0, 1, 0], atol=1e-12)


def test_gdn_beta_zero_is_pure_decay():
    """beta = 0: S_T = (prod a) S0 and o_t = (prod_{s<=t} a_s) S0 q_t."""
    rng = np.random.default_rng(4)
    q, k, v, a, _ = _rand_inputs(rng, 2, 30, 2, 8)
    S0 = rng.standard_normal((2, 2, 8, 8))
    o, S = gdn_recurrent(q, k, v, a, np.zeros_like(a), S0)
    cp = np.cumprod(a, axis=1)                                     # [B, T, H]
    np.testing.assert_allclose(S, cp[:, -1][..., None, None] * S0, rtol=1e-12)
    exp_o = cp[..., None] * np.einsum("bhvk,bthk->bthv", S0, q)
    np.testing.assert_allclose(o, exp_o, rtol=1e-11, atol=1e-12)


def test_gdn_contraction_eq18():
    """Two runs that differ only in S0: ||dS_t||_F <= prod_{s<=t} a_s ||dS0||_F
    (each step multiplies the difference by a_t (I - b_t k k^T), whose norm is
    <= a_t for unit k and b in [0, 1]); and the state stays bounded by
    rho^t ||S0|| + max b ||v|| / (1 - rho), rho = max a (Eq. 18 with e_0 the
    initial state and xi the written value)."""
    rng = np.random.default_rng(5)
    q, k, v, a, b = _rand_inputs(rng, 1, 200, 2, 8, alpha=(0.85, 0.99), beta=(0.0, 1.0))
    S0a = rng.standard_normal((1, 2, 8, 8)) * 10
    S0b = rng.standard_normal((1, 2, 8, 8)) * 10
    d0 = np.linalg.norm(S0a - S0b, axis=(-2, -1))
    for T in (1, 7, 50, 200):
        _, Sa = gdn_recurrent(q[:, :T], k[:, :T], v[:, :T], a[:, :T], b[:, :T], S0a)
        _, Sb = gdn_recurrent(q[:, :T], k[:, :T], v[:, :T], a[:, :T], b[:, :T], S0b)
        dT = np.linalg.norm(Sa - Sb, axis=(-2, -1))
        bound = np.prod(a[:, :T], axis=1) * d0
        assert np.all(dT <= bound * (1 + 1e-12))
        rho = a[:, :T].max()
        vmax = np.linalg.norm(v[:, :T], axis=-1).max() * b[:, :T].max()
        assert np.all(np.linalg.norm(Sa, axis=(-2, -1))
                      <= rho ** T * np.linalg.norm(S0a, axis=(-2, -1)) + vmax / (1 - rho) + 1e-9)


def test_gdn_step_is_sgd_on_decayed_state():
    """Eq. 3's reading as one gradient step: the canonical update equals one SGD
    step with learning rate beta on 0.5 ||v - S k||^2 taken at the decayed
    state a S_{t-1}; the printed Eq. 6 takes the step at S_{t-1} and decays
    the old state alone.  Gradients come from torch autograd."""
    rng = np.random.default_rng(6)
    d = 6
    S_prev = rng.standard_normal((d, d))
    kk = rng.standard_normal(d)
    kk /= np.linalg.norm(kk)
    vv = rng.standard_normal(d)
    a, b = 0.83, 0.41

    def grad_at(S):
        St = torch.tensor(S, dtype=torch.float64, requires_grad=True)
        loss = 0.5 * torch.sum((torch.tensor(vv) - St @ torch.tensor(kk)) ** 2)
        loss.backward()
        return St.grad.numpy()

    canonical_expected = a * S_prev - b * grad_at(a * S_prev)
    literal_expected = a * S_prev - b * grad_at(S_prev)
    x = lambda arr: arr[None, None, None, :]
    _, S_can = gdn_recurrent(x(kk), x(kk), x(vv), np.full((1, 1, 1), a), np.full((1, 1, 1), b),
                             S_prev[None, None])
    _, S_lit = gdn_literal_eq6(x(kk), x(kk), x(vv), np.full((1, 1, 1), a), np.full((1, 1, 1), b),
                               S_prev[None, None])
    np.testing.assert_allclose(S_can[0, 0], canonical_expected, atol=1e-13)
    np.testing.assert_allclose(S_lit[0, 0], literal_expected, atol=1e-13)


def test_literal_eq6_is_canonical_with_rescaled_inputs():
    """literal(a, b, v) == canonical(a, b / a, a v): the two readings are the
    same kernel with rescaled inputs."""
    rng = np.random.default_rng(7)
    q, k, v, a, b = _rand_inputs(rng, 1, 40, 2, 8, alpha=(0.7, 0.99), beta=(0.05, 0.6))
    S0 = rng.standard_normal((1, 2, 8, 8))
    o1, S1 = gdn_literal_eq6(q, k, v, a, b, S0)
    o2, S2 = gdn_recurrent(q, k, a[..., None] * v, a, b / a, S0)
    np.testing.assert_allclose(o1, o2, rtol=1e-10, atol=1e-12)
    np.testing.assert_allclose(S1, S2, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("d", [4, 8, 16, 32])
@pytest.mark.parametrize("C", [1, 2, 4, 16, 64])
def test_gdn_chunked_equals_recurrence(d, C):
    """Chunkwise evaluation equals token-by-token evaluation (brute force over
    lengths that leave ragged last chunks).  C = 1 is the recurrence itself."""
    rng = np.random.default_rng(100 + d + C)
    for T in (1, 2, 5, 63, 64, 65, 130):
        q, k, v, a, b = _rand_inputs(rng, 1, T, 2, d)
        S0 = rng.standard_normal((1, 2, d, d))
        o1, S1 = gdn_recurrent(q, k, v, a, b, S0)
        o2, S2 = gdn_chunked(q, k, v, a, b, S0, chunk=C)
        np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-11)
        np.testing.assert_allclose(S2, S1, rtol=1e-9, atol=1e-11)


def test_gdn_state_passing_equals_single_run():
    """Recurrent state passing (long-horizon generation): running the sequence
    in pieces and carrying S equals one run."""
    rng = np.random.default_rng(8)
    q, k, v, a, b = _rand_inputs(rng, 2, 90, 2, 8)
    o, S = gdn_recurrent(q, k, v, a, b)
    S_c = None
    outs = []
    for s, e in ((0, 17), (17, 64), (64, 90)):
        oo, S_c = gdn_recurrent(q[:, s:e], k[:, s:e], v[:, s:e], a[:, s:e], b[:, s:e], S_c)
        outs.append(oo)
    np.testing.assert_allclose(np.concatenate(outs, 1), o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(S_c, S, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------- windowed attention

def _sdpa(q, k, v, mask=None, causal=False):
    """torch's scaled-dot-product attention on [B, T, H, d] fp64 inputs."""
    tq, tk, tv = (torch.tensor(np.moveaxis(x, 2, 1)) for x in (q, k, v))
    out = torch.nn.functional.scaled_dot_product_attention(
        tq, tk, tv, attn_mask=None if mask is None else torch.tensor(mask), is_causal=causal)
    return np.moveaxis(out.numpy(), 1, 2)


def test_swa_wide_window_is_causal_attention():
    rng = np.random.default_rng(10)
    q, k, v, _, _ = _rand_inputs(rng, 2, 70, 3, 16)
    for w in (70, 71, 500):
        np.testing.assert_allclose(windowed_attention(q, k, v, 10, w, 1), _sdpa(q, k, v, causal=True),
                                   rtol=1e-10, atol=1e-12)


def test_swa_band_matches_masked_library_attention():
    rng = np.random.default_rng(11)
    q, k, v, _, _ = _rand_inputs(rng, 1, 90, 2, 8)
    i = np.arange(90)[:, None]
    j = np.arange(90)[None, :]
    for w in (2, 5, 33):
        band = (j > i - w) & (j <= i)
        np.testing.assert_allclose(windowed_attention(q, k, v, 9, w, 1), _sdpa(q, k, v, mask=band),
                                   rtol=1e-10, atol=1e-12)


def test_swa_window_one_returns_values():
    rng = np.random.default_rng(12)
    q, k, v, _, _ = _rand_inputs(rng, 1, 40, 2, 8)
    np.testing.assert_allclose(windowed_attention(q, k, v, 8, 1, 1), v, atol=1e-13)
    np.testing.assert_allclose(windowed_attention(q, k, v, 8, 1, 3), v, atol=1e-13)


@pytest.mark.parametrize("T,L,w,dil,fo", [(24, 4, 5, 1, 0), (28, 4, 4, 4, 0), (30, 4, 6, 3, 2),
                                          (23, 5, 7, 2, 1), (20, 4, 1, 2, 0)])
def test_window_blocked_equals_bruteforce(T, L, w, dil, fo):
    rng = np.random.default_rng(13 + T + w)
    q, k, v, _, _ = _rand_inputs(rng, 1, T, 2, 4)
    np.testing.assert_allclose(windowed_attention(q, k, v, L, w, dil, fo),
                               window_bruteforce(q, k, v, L, w, dil, fo), rtol=1e-11, atol=1e-12)


@pytest.mark.parametrize("F,L,w,dil,fo", [(7, 6, 6, 4, 0), (8, 5, 9, 2, 0), (9, 4, 4, 3, 5),
                                          (12, 3, 5, 4, 2), (5, 7, 20, 6, 0)])
def test_dswa_mask_equals_literal_rearrange(F, L, w, dil, fo):
    """Eq. 8: DSWA = SWA on the frame-residue rearrangement; the mask form used
    by the kernels equals gather -> SWA -> scatter, also when F mod d != 0
    and with an absolute frame offset."""
    rng = np.random.default_rng(20 + F * L)
    q, k, v, _, _ = _rand_inputs(rng, 1, F * L, 2, 8)
    np.testing.assert_allclose(windowed_attention(q, k, v, L, w, dil, fo),
                               dswa_reshape(q, k, v, L, w, dil, fo), rtol=1e-11, atol=1e-12)


def test_dswa_wide_window_is_causal_attention_per_group():
    """A window covering whole residue groups reduces each group to full causal
    attention (library routine applied to the gathered group)."""
    rng = np.random.default_rng(21)
    F, L, dil = 9, 5, 4
    q, k, v, _, _ = _rand_inputs(rng, 1, F * L, 2, 8)
    o = windowed_attention(q, k, v, L, 10 ** 6, dil)
    for r in range(dil):
        idx = np.concatenate([np.arange(f * L, (f + 1) * L) for f in range(F) if f % dil == r])
        np.testing.assert_allclose(o[:, idx], _sdpa(q[:, idx], k[:, idx], v[:, idx], causal=True),
                                   rtol=1e-10, atol=1e-12)


def test_dswa_dilation_one_is_swa():
    rng = np.random.default_rng(22)
    q, k, v, _, _ = _rand_inputs(rng, 1, 60, 2, 8)
    np.testing.assert_allclose(dswa_reshape(q, k, v, 6, 13, 1),
                               _sdpa(q, k, v, mask=(np.arange(60)[None, :] > np.arange(60)[:, None] - 13)
                                     & (np.arange(60)[None, :] <= np.arange(60)[:, None])),
                               rtol=1e-10, atol=1e-12)


def test_window_rows_subset_and_convex_hull():
    rng = np.random.default_rng(23)
    q, k, v, _, _ = _rand_inputs(rng, 1, 50, 2, 8)
    full = windowed_attention(q, k, v, 7, 9, 2, 1)
    rows = np.array([49, 0, 13, 14, 30, 7])
    np.testing.assert_allclose(windowed_attention_rows(q, k, v, rows, 7, 9, 2, 1), full[:, rows],
                               rtol=1e-13, atol=1e-14)
    # every output is a convex combination of values: within their range
    assert np.all(full <= v.max(axis=1, keepdims=True) + 1e-12)
    assert np.all(full >= v.min(axis=1, keepdims=True) - 1e-12)


# ----------------------------------------------------------------- fp8

def test_e4m3_matches_torch_cast():
    rng = np.random.default_rng(30)
    x = np.concatenate([rng.standard_normal(100000) * 30, rng.standard_normal(20000) * 1e-2,
                        rng.uniform(-448, 448, 20000)]).astype(np.float32)
    grid = e4m3_decode(np.arange(256))
    grid = np.sort(grid[np.isfinite(grid)])
    mids = ((grid[1:] + grid[:-1]) / 2).astype(np.float32)          # exact ties
    x = np.concatenate([x, mids, grid.astype(np.float32)])
    x = np.clip(x, -448, 448)
    t = torch.from_numpy(x).to(torch.float8_e4m3fn)
    np.testing.assert_array_equal(e4m3_round(x), t.to(torch.float64).numpy())
    np.testing.assert_array_equal(e4m3_encode(e4m3_round(x)), t.view(torch.uint8).numpy())


def test_e4m3_saturates_and_roundtrips():
    assert np.all(e4m3_round(np.array([449.0, 1e6, -5000.0])) == np.array([448.0, 448.0, -448.0]))
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    np.testing.assert_array_equal(e4m3_encode(e4m3_decode(codes)), codes)
    assert e4m3_decode(np.array([0x7E]))[0] == 448.0 and e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9


def test_fp8_block_quantiser_properties():
    rng = np.random.default_rng(31)
    x = round_bf16(rng.standard_normal((2, 150, 3, 16)).astype(np.float32))
    x[1, 64:128, 2] = 0.0                                  # an all-zero block
    codes, scales, xh = fp8_quantize_blocks(x)
    assert scales.shape == (2, 3, 3)
    assert scales[1, 2, 1] == 1.0 and np.all(codes[1, 64:128, 2] == 0)
    dec = e4m3_decode(codes)
    for b in range(2):
        for h in range(3):
            for blk in range(3):
                sl = dec[b, blk * 64:(blk + 1) * 64, h]
                if scales[b, h, blk] != 1.0 or np.any(sl):
                    assert np.max(np.abs(sl)) == 448.0
    # half an e4m3 ulp: 2^-4 relative in the normal range, 2^-10 * s below it
    s_tok = np.repeat(scales, 64, axis=2)[:, :, :150].transpose(0, 2, 1)[..., None].astype(np.float64)
    bound = np.maximum(2.0 ** -4 * np.abs(x), 2.0 ** -10 * s_tok) * (1 + 1e-6)
    assert np.all(np.abs(xh - x) <= bound)


def test_fp8_lossless_on_grid_values():
    """Inputs already on the e4m3 grid with block amax 448 have scale exactly 1
    and quantise losslessly."""
    rng = np.random.default_rng(32)
    grid = e4m3_decode(np.arange(0, 0x7F))
    x = rng.choice(np.concatenate([grid, -grid]), size=(1, 128, 2, 8)).astype(np.float32)
    x[0, 0, :, 0] = 448.0
    x[0, 64, :, 0] = -448.0
    codes, scales, xh = fp8_quantize_blocks(x)
    assert np.all(scales == 1.0)
    np.testing.assert_array_equal(xh, x.astype(np.float64))


# ----------------------------------------------------------------- hybrid layer

def test_hlta_gate_isolation_and_half_sum():
    rng = np.random.default_rng(40)
    q, k, v, a, b = _rand_inputs(rng, 1, 48, 2, 8)
    L, w, dil = 6, 6, 2
    o_swa = windowed_attention(q, k, v, L, w, 1)
    o_dswa = windowed_attention(q, k, v, L, w, dil)
    o_gdn, S = gdn_recurrent(q, k, v, a, b)
    for z, want in (((40, -40, -40), o_swa), ((-40, 40, -40), o_dswa), ((-40, -40, 40), o_gdn)):
        y, S2 = hlta(q, k, v, a, b, np.array(z, float)[:, None] * np.ones((3, 2)), L, w, dil)
        np.testing.assert_allclose(y, want, rtol=1e-12, atol=1e-12)
        np.testing.assert_allclose(S2, S, rtol=1e-14)
    y, _ = hlta(q, k, v, a, b, np.zeros((3, 2)), L, w, dil)
    np.testing.assert_allclose(y, 0.5 * (o_swa + o_dswa + o_gdn), rtol=1e-13, atol=1e-14)


def test_hlta_fp8_mode_equals_bf16_mode_on_grid_inputs():
    rng = np.random.default_rng(41)
    grid = e4m3_decode(np.arange(0x30, 0x48))                 # 0.5 .. 3.0 range
    B, T, H, d = 1, 128, 2, 8
    q = rng.choice(np.concatenate([grid, -grid]), size=(B, T, H, d)).astype(np.float32)
    k = rng.choice(np.concatenate([grid, -grid]), size=(B, T, H, d)).astype(np.float32)
    q[:, ::64, :, 0] = 448.0
    k[:, ::64, :, 0] = -448.0
    _, _, v, a, b = _rand_inputs(rng, B, T, H, d)
    z = rng.standard_normal((3, H))
    y8, _ = hlta(q, k, v, a, b, z, 16, 20, 2, window_qk="fp8")
    y16, _ = hlta(q, k, v, a, b, z, 16, 20, 2, window_qk="bf16")
    np.testing.assert_array_equal(y8, y16)


def test_hlta_rows_subset():
    rng = np.random.default_rng(42)
    q, k, v, a, b = _rand_inputs(rng, 2, 40, 2, 8)
    z = rng.standard_normal((3, 2))
    y, S = hlta(q, k, v, a, b, z, 5, 7, 3, frame_offset=2)
    rows = np.array([3, 39, 20, 21])
    yr, Sr = hlta_rows(q, k, v, a, b, z, 5, 7, 3, rows, frame_offset=2)
    np.testing.assert_allclose(yr, y[:, rows], rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(Sr, S)


# ----------------------------------------------------------------- input generator

def test_generator_is_deterministic_and_shaped():
    a = make_custom(1, 70, 3, 32, "bf16", seed=5)
    b = make_custom(1, 70, 3, 32, "bf16", seed=5)
    for key in ("q", "k", "v", "alpha", "beta", "gates"):
        np.testing.assert_array_equal(a[key], b[key])
    assert a["q"].shape == (1, 70, 3, 32) and a["alpha"].shape == (1, 70, 3) and a["gates"].shape == (3, 3)
    np.testing.assert_array_equal(round_bf16(a["q"]), a["q"])
    np.testing.assert_allclose(np.linalg.norm(a["k"].astype(np.float64), axis=-1), 1.0, atol=2 ** -7)
    assert np.all((a["alpha"] > 0) & (a["alpha"] < 1)) and np.all((a["beta"] > 0) & (a["beta"] < 1))
    f = make_inputs(0)
    assert f["q"].dtype == np.float32 and "q_bits" not in f
    np.testing.assert_allclose(np.linalg.norm(f["k"].astype(np.float64), axis=-1), 1.0, atol=1e-6)
    assert np.all((f["alpha"] >= 0.9) & (f["alpha"] <= 0.999))


def test_bf16_rounding_is_nearest_even():
    x = np.array([1.0 + 2 ** -8, 1.0 + 3 * 2 ** -8, -1.0 - 2 ** -8, 1.0 + 2 ** -8 + 2 ** -20], np.float32)
    got = bf16_bits_to_f32(to_bf16_bits(x))
    want = torch.from_numpy(x).to(torch.bfloat16).to(torch.float32).numpy()
    np.testing.assert_array_equal(got, want)


from hypothesis import given, settings, strategies as st


@settings(max_examples=60, deadline=None, derandomize=True)
@given(T=st.integers(1, 36), L=st.integers(1, 12), w=st.integers(1, 30), dil=st.integers(1, 4),
       fo=st.integers(0, 5), centered=st.booleans(), seed=st.integers(0, 2 ** 31 - 1))
def test_window_blocked_equals_bruteforce_property(T, L, w, dil, fo, centered, seed):
    """The blocked window oracle against the scalar key-set definition on
    arbitrary tiny shapes: partial last frames, windows shorter or longer than
    a frame, dilations, frame offsets, causal and centred."""
    rng = np.random.default_rng(seed)
    q, k, v, _, _ = _rand_inputs(rng, 1, T, 2, 4)
    np.testing.assert_allclose(windowed_attention(q, k, v, L, w, dil, fo, centered=centered),
                               window_bruteforce(q, k, v, L, w, dil, fo, centered=centered),
                               rtol=1e-11, atol=1e-12)


@settings(max_examples=40, deadline=None, derandomize=True)
@given(T=st.integers(0, 100), d=st.sampled_from([2, 4, 8]), C=st.integers(1, 70), split=st.floats(0, 1),
       seed=st.integers(0, 2 ** 31 - 1))
def test_gdn_chunked_and_state_passing_property(T, d, C, split, seed):
    """On arbitrary tiny shapes: the chunkwise form with any chunk length
    equals the token recurrence, and running the sequence in two pieces with
    the state carried across equals one run."""
    rng = np.random.default_rng(seed)
    q, k, v, a, b = _rand_inputs(rng, 1, T, 2, d)
    S0 = rng.standard_normal((1, 2, d, d))
    o1, S1 = gdn_recurrent(q, k, v, a, b, S0)
    o2, S2 = gdn_chunked(q, k, v, a, b, S0, chunk=C)
    np.testing.assert_allclose(o2, o1, rtol=1e-9, atol=1e-11)
    np.testing.assert_allclose(S2, S1, rtol=1e-9, atol=1e-11)
    s = int(round(split * T))
    oa, Sa = gdn_recurrent(q[:, :s], k[:, :s], v[:, :s], a[:, :s], b[:, :s], S0)
    ob, Sb = gdn_recurrent(q[:, s:], k[:, s:], v[:, s:], a[:, s:], b[:, s:], Sa)
    np.testing.assert_allclose(np.concatenate([oa, ob], axis=1), o1, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(Sb, S1, rtol=1e-12, atol=1e-13)
