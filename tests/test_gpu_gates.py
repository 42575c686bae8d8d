"""GPU: the debug check of the gated delta rule's gates (kairos_gdn_check_gates)
counts exactly the (b, t, h) with alpha outside (0, 1] or beta outside
[0, beta_max], NaN included, against numpy's count of the same predicate, on
random gates with planted values on both sides of every bound; with
KAIROS_DEBUG set the GDN and layer calls refuse out-of-range gates
(KAIROS_ERR_RANGE) and run in-range ones."""
import numpy as np
import pytest
import torch

import video_world_model_chunkwise_amd as K
from tests.gpu_util import inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _expected(a, b, bmax):
    return int(np.count_nonzero(~((a > 0) & (a <= 1)) | ~((b >= 0) & (b <= bmax))))


@pytest.mark.parametrize("B,T,H", [(1, 0, 1), (1, 1, 1), (2, 1000, 3), (4, 57600, 24)])
def test_gate_check_counts(B, T, H):
    print(f"gate check B{B} T{T} H{H}", flush=True)
    rng = np.random.default_rng(B * 7919 + T + H)
    a = rng.uniform(0.5, 1.0, (B, T, H)).astype(np.float32)
    b = rng.uniform(0.0, 1.0, (B, T, H)).astype(np.float32)
    fa, fb = a.reshape(-1), b.reshape(-1)
    n = fa.size
    if n >= 24:
        idx = rng.permutation(n)[:24]
        inside_a = [1.0, 1e-30, np.nextafter(np.float32(0), np.float32(1)) * 2 ** 24]
        inside_b = [0.0, -0.0, 1.0]
        outside_a = [0.0, -0.0, -0.5, np.nextafter(np.float32(1), np.float32(2)), np.nan, np.inf, -np.inf]
        outside_b = [-1e-30, np.nextafter(np.float32(1), np.float32(2)), 1.5, 2.5, np.nan, np.inf, -np.inf]
        vals = [("a", x) for x in inside_a + outside_a] + [("b", x) for x in inside_b + outside_b]
        for i, (which, x) in zip(idx, vals):
            (fa if which == "a" else fb)[i] = np.float32(x)
    da, db = torch.from_numpy(a).to("cuda:0"), torch.from_numpy(b).to("cuda:0")
    for bmax in (1.0, 2.0):
        got = K.kairos_gdn_check_gates(da, db, beta_max=bmax)
        assert got == _expected(a, b, bmax), (bmax, got, _expected(a, b, bmax))
    if n >= 24:
        assert _expected(a, b, 1.0) >= 12


def test_debug_env_refuses_out_of_range_gates(monkeypatch):
    B, F, L, H, w, dil = 1, 3, 100, 2, 150, 2
    T = F * L
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=5))
    monkeypatch.setenv("KAIROS_DEBUG", "1")
    K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"])      # in range: runs
    K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil)
    torch.cuda.synchronize()
    alpha = dv["alpha"].clone()
    alpha[0, 17, 1] = 1.5
    with pytest.raises(K.KairosError) as e:
        K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], alpha, dv["beta"])
    assert e.value.status == K.KAIROS_ERR_RANGE
    beta = dv["beta"].clone()
    beta[0, 3, 0] = float("nan")
    with pytest.raises(K.KairosError) as e:
        K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], beta, dv["gates"], L, w, dil)
    assert e.value.status == K.KAIROS_ERR_RANGE
