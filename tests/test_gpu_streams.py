"""GPU: with a kairos_context the layer call runs part of its work on the
context's side stream, joined back by events.  Callers on two streams at
once, a layer call captured into a graph and replayed with eager work in
between, and eager calls on a second host thread while the first thread
holds a capture open on the same context must all give results
bit-identical to sequential calls of the same schedule (same kernels, same
inputs: any race or missing join shows as a difference)."""
import threading

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


def _layer(dv, L, w, dil, out, state, ws, stream=None, ctx=None):
    K.kairos_hlta_fwd(dv["q"], dv["k"], dv["v"], dv["alpha"], dv["beta"], dv["gates"], L, w, dil,
                      window_qk=K.FP8_E4M3, out=out, state_out=state, workspace=ws, stream=stream,
                      ctx=ctx)


def test_context_matches_single_stream():
    """Both schedules a context enables against the single-stream call.  For a
    larger call the pre-passes run beside the scan: same kernels, bit-identical
    results.  For a small call the GDN branch runs beside the window kernel and
    a combine kernel adds it: (o_swa + o_dswa) + o_gdn instead of the
    epilogue's o_dswa + (o_swa + o_gdn) in fp32, so y may differ by the bf16
    rounding of that reordering (at most one bf16 step); the state is the same
    GDN computation and must be bit-identical."""
    for (B, F, L, H, w, dil, seed, exact) in ((1, 6, 200, 2, 300, 4, 504, False),
                                              (1, 8, 1024, 8, 1000, 4, 505, True)):
        T = F * L
        print(f"context vs single stream F{F} L{L} H{H}", flush=True)
        dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=seed))
        o, S, ws = _bufs(B, T, H, L, w, dil)
        _layer(dv, L, w, dil, o, S, ws)
        torch.cuda.synchronize()
        ref_o, ref_S = o.clone(), S.clone()
        with K.Context() as ctx:
            for _ in range(2):
                o.zero_()
                S.zero_()
                _layer(dv, L, w, dil, o, S, ws, ctx=ctx)
                torch.cuda.synchronize()
                assert torch.equal(S, ref_S)
                if exact:
                    assert torch.equal(o, ref_o)
                else:
                    r = ref_o.float()
                    step = r.abs() * 2.0 ** -7 + 1e-5 * r.abs().max()
                    assert bool(((o.float() - r).abs() <= step).all())


def test_layer_on_two_streams_at_once():
    B, F, L, H, w, dil = 1, 8, 200, 4, 300, 4
    T = F * L
    print("two streams", flush=True)
    dvs = [inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=s)) for s in (501, 502)]
    bufs = [_bufs(B, T, H, L, w, dil) for _ in dvs]
    ctx = K.Context()
    refs = []
    for dv, (o, S, ws) in zip(dvs, bufs):
        _layer(dv, L, w, dil, o, S, ws, ctx=ctx)
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
                _layer(dvs[i], L, w, dil, o, S, ws, stream=st, ctx=ctx)
        torch.cuda.synchronize()
        for (o, S, _), (ro, rS) in zip(bufs, refs):
            assert torch.equal(o, ro), f"iteration {it}: output differs"
            assert torch.equal(S, rS), f"iteration {it}: state differs"
    ctx.close()


def test_layer_graph_replays_match_eager():
    B, F, L, H, w, dil = 1, 6, 200, 2, 300, 4
    T = F * L
    print("graph capture", flush=True)
    dv = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=503))
    o, S, ws = _bufs(B, T, H, L, w, dil)
    ctx = K.Context()
    _layer(dv, L, w, dil, o, S, ws, ctx=ctx)
    torch.cuda.synchronize()
    ref_o, ref_S = o.clone(), S.clone()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _layer(dv, L, w, dil, o, S, ws, ctx=ctx)   # warm-up on a non-default stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _layer(dv, L, w, dil, o, S, ws, ctx=ctx)
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
    ctx.close()


def test_capture_on_one_thread_eager_calls_on_another():
    """Thread A captures layer calls into a graph on a shared context while
    thread B makes eager layer calls with the same context on its own stream.
    B's calls must not land in A's graph (they run on B's stream alone while
    the side stream belongs to A's capture), and both results must equal the
    sequential references."""
    B, F, L, H, w, dil = 1, 6, 200, 2, 300, 4
    T = F * L
    print("capture + eager threads", flush=True)
    dva = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=506))
    dvb = inputs_to_dev(make_custom(B, T, H, 128, "bf16", seed=507))
    ba, bb = _bufs(B, T, H, L, w, dil), _bufs(B, T, H, L, w, dil)
    # references of both schedules: with the context's side stream, and on
    # one stream (what a call does while another capture holds the side stream)
    ctx = K.Context()
    refs, refs1 = [], []
    for dv, (o, S, ws) in ((dva, ba), (dvb, bb)):
        _layer(dv, L, w, dil, o, S, ws, ctx=ctx)
        torch.cuda.synchronize()
        refs.append((o.clone(), S.clone()))
        _layer(dv, L, w, dil, o, S, ws)
        torch.cuda.synchronize()
        refs1.append((o.clone(), S.clone()))
    sb = torch.cuda.Stream()
    g = torch.cuda.CUDAGraph()
    errors = []
    start = threading.Barrier(2)

    def eager_b():
        try:
            with torch.cuda.stream(sb):
                start.wait()
                for _ in range(20):
                    _layer(dvb, L, w, dil, *bb, stream=sb, ctx=ctx)
                sb.synchronize()
        except Exception as e:          # reported by the main thread
            errors.append(e)

    tb = threading.Thread(target=eager_b)
    tb.start()
    try:
        with torch.cuda.graph(g, capture_error_mode="thread_local"):
            start.wait()
            for _ in range(4):
                _layer(dva, L, w, dil, *ba, ctx=ctx)
    finally:
        tb.join()
    assert not errors, errors
    torch.cuda.synchronize()
    assert torch.equal(bb[1], refs[1][1]), "eager thread: state differs"
    assert torch.equal(bb[0], refs[1][0]) or torch.equal(bb[0], refs1[1][0]), "eager thread differs"
    for it in range(2):
        ba[0].zero_()
        ba[1].zero_()
        bb[0].zero_()
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(ba[0], refs[0][0]), f"replay {it}: output differs"
        assert torch.equal(ba[1], refs[0][1]), f"replay {it}: state differs"
        assert not bb[0].any(), "the graph wrote the eager thread's output"
    ctx.close()
