"""GPU parity of the gated delta rule when the scan is split over time (few
(b, h), long sequences): a first pass runs segments from a zero state and
their transitions from the identity, a combine applies the segment maps, and
a second pass reruns every segment from its true start.  Compared with the
oracle's token-by-token recurrence (oracle.gdn_recurrent) on every output
token (so every segment boundary) and on the final state, with ragged last
chunks, non-zero initial states, the in-place state carry and d = 64.

The number of segments P is read back from the workspace size, which holds
two D x D fp32 slots per (b, h) and segment when P > 1, so every case below
asserts that it runs the split scan it is meant to test."""
import numpy as np
import pytest
import torch

import oracle
import video_world_model_chunkwise_amd as K
from tests.conftest import rel_errors
from tests.gpu_util import dev_f32, host, inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu

TOL_MAX, TOL_MEAN = 2e-2, 5e-3


def _segments(B, T, H, d):
    up = lambda x: (x + 255) // 256 * 256
    n = -(-T // 64)
    base = up(B * H * n * 64 * 64 * 2) + up(B * H * n * 64 * 4)
    extra = K.kairos_gdn_workspace_size(K.gdn_desc(B, T, H, d)) - base
    per = 2 * B * H * d * d * 4
    assert extra % per == 0
    return max(1, extra // per)


def _check(got, ref, what):
    assert np.all(np.isfinite(got)), f"{what}: non-finite values"
    rmax, rmean = rel_errors(got, ref)
    print(f"{what}: rel_max={rmax:.3e} rel_mean={rmean:.3e}", flush=True)
    assert rmax <= TOL_MAX and rmean <= TOL_MEAN, f"{what}: rel_max {rmax:.3e} rel_mean {rmean:.3e}"


@pytest.mark.parametrize("B,T,H,d,with_state,in_place", [
    (1, 4100, 2, 128, False, False),      # 65 chunks, last one 4 tokens
    (1, 4100, 2, 128, True, False),
    (1, 6000, 3, 128, True, True),        # state_out is state_in
    (2, 5000, 1, 64, True, False),        # d = 64
    (1, 8192, 4, 128, True, False),       # whole chunks only
])
def test_split_scan_matches_recurrence(B, T, H, d, with_state, in_place):
    P = _segments(B, T, H, d)
    print(f"split scan B{B} T{T} H{H} d{d} P={P} state={with_state} in_place={in_place}", flush=True)
    assert P > 1
    inp = make_custom(B, T, H, d, "bf16", seed=900 + T + H + d)
    dv = inputs_to_dev(inp)
    S0 = None
    if with_state:
        S0 = (0.1 * np.random.default_rng(T).standard_normal((B, H, d, d))).astype(np.float32)
    s_in = dev_f32(S0) if S0 is not None else None
    s_out = s_in if in_place else None
    out, S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], state_in=s_in,
                              state_out=s_out)
    torch.cuda.synchronize()
    o_ref, S_ref = oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"], S0)
    got = host(out)
    _check(got, o_ref, "o")
    _check(host(S), S_ref, "S")
    # each segment on its own (the first chunks after a boundary start from a
    # combined state): no segment may be far worse than the whole
    L = -(-(-(-T // 64)) // P) * 64
    for j in range(P):
        sl = slice(j * L, min(T, (j + 1) * L))
        _check(got[:, sl], o_ref[:, sl], f"o segment {j}")


def test_split_scan_poisoned_workspace_and_determinism():
    """NaN-filled outputs, state and workspace give the same bits as zeroed
    ones, and repeated runs are bit-identical: every slot the split scan reads
    is written first in the same call."""
    B, T, H, d = 1, 4100, 2, 128
    assert _segments(B, T, H, d) > 1
    dv = inputs_to_dev(make_custom(B, T, H, d, "bf16", seed=931))
    S0 = dev_f32((0.1 * np.random.default_rng(5).standard_normal((B, H, d, d))).astype(np.float32))
    nws = K.kairos_gdn_workspace_size(K.gdn_desc(B, T, H, d))
    ws = torch.empty(nws, dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, T, H, d), dtype=torch.bfloat16, device="cuda:0")
    S = torch.empty((B, H, d, d), dtype=torch.float32, device="cuda:0")
    res = []
    for fill in (0xFF, 0x00, 0xFF):
        for t in (ws, out.view(torch.uint8), S.view(torch.uint8)):
            t.fill_(fill)
        K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], state_in=S0, out=out,
                         state_out=S, workspace=ws)
        torch.cuda.synchronize()
        res.append((out.clone(), S.clone()))
    for r in res[1:]:
        assert torch.equal(r[0], res[0][0]) and torch.equal(r[1], res[0][1])
    assert torch.isfinite(res[0][0].float()).all() and torch.isfinite(res[0][1]).all()
