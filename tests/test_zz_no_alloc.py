"""GPU: kairos_gdn_fwd_noalloc (workspace = the library's per-device scratch
array) against kairos_gdn_fwd with a caller workspace, on two calls in a
row, the second smaller and starting from a non-zero state: the same kernels
on the same inputs, so outputs and states must be bit-identical (stricter
than the 2e-2 / 5e-3 parity bar)."""
import pytest
import torch

import video_world_model_chunkwise_amd as K
from tests.gpu_util import inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _pair(B, T, H, seed, with_state):
    print(f"no-alloc GDN B{B} T{T} H{H} state_in={with_state}", flush=True)
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=seed))
    s_in = None
    if with_state:
        g = torch.Generator(device="cuda:0")
        g.manual_seed(seed)
        s_in = 0.1 * torch.randn((B, H, 128, 128), generator=g, device="cuda:0")
    ref_o, ref_S = K.kairos_gdn_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], state_in=s_in)
    out = torch.full_like(ref_o, float("nan"))
    S = torch.full_like(ref_S, float("nan"))
    K.kairos_gdn_fwd_noalloc(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], state_in=s_in,
                             out=out, state_out=S)
    torch.cuda.synchronize()
    assert torch.equal(out, ref_o), "output differs from kairos_gdn_fwd"
    assert torch.equal(S, ref_S), "state differs from kairos_gdn_fwd"


def test_noalloc_matches_workspace_call_twice():
    _pair(2, 4096, 16, 811, False)        # 29.9 MB of the 64 MiB array, scan split in 3 segments
    _pair(1, 1000, 4, 812, True)          # smaller, ragged last chunk, state carried in


def test_noalloc_refuses_oversized_problem():
    B, T, H = 1, 40000, 32                # workspace above 64 MiB
    assert K.kairos_gdn_workspace_size(K.gdn_desc(B, T, H, 128)) > 64 << 20
    x = torch.zeros((B, T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    a = torch.full((B, T, H), 0.9, device="cuda:0")
    with pytest.raises(K.KairosError) as e:
        K.kairos_gdn_fwd_noalloc(x, x, x, a, a, out=torch.empty_like(x))
    assert e.value.status == -7
