"""GPU: the layer call runs the windowed branches' operand pre-passes on the
library's per-device side stream, joined back by events.  Callers on two
streams at once, and a layer call captured into a graph and replayed with
eager work in between, must give results bit-identical to plain sequential
calls (same kernels, same inputs: any race or missing join shows as a
difference)."""
import pytest
import torch

import video_world_model_chunkwise_amd as K
from tests.gpu_util import inputs_to_dev
from workloads import make_custom

pytestmark = pytest.mark.gpu


def _bufs(B, T, H, L, w, dil):
    desc = K.hlta_desc(B, T, H, 128, L, w, dil, window_qk=K.FP8_E4M3)
    ws = torch.empty(K.kairos_hlta_workspace_size(desc), dtype=torch.uint8, device="cuda:0")
    out = torch.empty((B, T, H, 128), dtype=torch.bfloat16, device="cuda:0")
    state = torch.empty((B, H, 128, 128), dtype=torch.float32, device="cuda:0")
    return out, state, ws


def _layer(dv, L, w, dil, out, state, ws, stream=None):
    K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                      window_qk=K.FP8_E4M3, out=out, state_out=state, workspace=ws, stream=stream)


def test_layer_on_two_streams_at_once():
    B, F, L, H, w, dil = 1, 8, 200, 4, 300, 4
    T = F * L
    print("two streams", flush=True)
    dvs = [inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=s)) for s in (501, 502)]
    bufs = [_bufs(B, T, H, L, w, dil) for _ in dvs]
    refs = []
    for dv, (o, S, ws) in zip(dvs, bufs):
        _layer(dv, L, w, dil, o, S, ws)
        torch.cuda.synchronize()
        refs.append((o.clone(), S.clone()))
    streams = (torch.cuda.Stream(), torch.cuda.Stream())
    for it in range(3):
        for o, S, _ in bufs:
            o.zero_()
            S.zero_()
        torch.cuda.synchronize()
        for i, st in enumerate(streams):
            with torch.cuda.stream(st):
                o, S, ws = bufs[i]
                _layer(dvs[i], L, w, dil, o, S, ws, stream=st)
        torch.cuda.synchronize()
        for (o, S, _), (ro, rS) in zip(bufs, refs):
            assert torch.equal(o, ro), f"iteration {it}: output differs"
            assert torch.equal(S, rS), f"iteration {it}: state differs"


def test_layer_graph_replays_match_eager():
    B, F, L, H, w, dil = 1, 6, 200, 2, 300, 4
    T = F * L
    print("graph capture", flush=True)
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=503))
    o, S, ws = _bufs(B, T, H, L, w, dil)
    _layer(dv, L, w, dil, o, S, ws)          # eager; the first call also creates the side stream
    torch.cuda.synchronize()
    ref_o, ref_S = o.clone(), S.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer(dv, L, w, dil, o, S, ws)      # warm-up on a non-default stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(dv, L, w, dil, o, S, ws)
    for it in range(3):
        o.zero_()
        S.zero_()
        junk = (dv["q"].float() * 2).sum()   # eager work between the replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(junk)
        assert torch.equal(o, ref_o), f"replay {it}: output differs"
        assert torch.equal(S, ref_S), f"replay {it}: state differs"
