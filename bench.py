#!/usr/bin/env python3
"""Benchmark of the hybrid linear temporal attention forward on one MI355X.

One step = one kairos_hlta_fwd call of the whole layer (FP8 E4M3 quantisation
of the windowed Q/K, the chunkwise gated delta rule with its fp32 state, SWA +
DSWA banded attention, gated combination) on the B=4, H=24, d=128,
16 frames x 3600 tokens workload with inputs resident in HBM.  Prints ONE
JSON line (metric, value = tokens/s of the whole job, roofline of the
dominant kernel measured live with HIP events on the launch stream, the CPU
oracle timed on a bounded sample, and a per-stage / per-workload breakdown).

    python bench.py [--gpus 1] [--steps 10] [--warmup 3] [--quick] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "GDN / hybrid temporal-attention fwd tokens/s + % roofline, H=24 d=128, 1 GPU"

# MI355X published peaks
PEAK_HBM_GBS = 8000.0
# SIMD time of one wave64 VALU instruction: 2 clocks for fp32 arithmetic (the
# published 157.3 TFLOP/s fp32 vector peak is 32 FMA lanes per clock per SIMD);
# 8 clocks for a transcendental (v_exp_f32), measured on gfx950 with two or
# more waves per SIMD issuing independent instructions
VALU_ISSUE_CLK = 2
TRANS_ISSUE_CLK = 8
# exponentials per second: 256 CU x 4 SIMD x 64 lanes / 8 clocks x 2.4 GHz
PEAK_EXP_PER_S = 256 * 4 * (64 / TRANS_ISSUE_CLK) * 2.4e9
SIMDS, CLOCK_HZ = 1024, 2.4e9
PEAK_BF16_TFLOPS = 2500.0
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
# QK^T at the 4-bit peak, P V at the bf16 peak (equal flops): time-weighted peak
PEAK_FP4_BLEND_TFLOPS = 2.0 / (1.0 / PEAK_FP4_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)

# algorithmic work per unit: the bytes one token of one head must move through
# HBM at least once (q, k, v read and o written in bf16, alpha and beta in
# fp32), and the flops of the chunkwise form per token (one chunk-head: the
# five C x C x d products of the Gram, output and solve operands, the three
# C x d x d state products, and the C^3 / 3 of the triangular inverse)
GDN_BYTES_PER_TOKEN_HEAD = 3 * 128 * 2 + 128 * 2 + 2 * 4      # q, k, v, o bf16 + alpha, beta fp32
CHUNK = 64


def gdn_flops_per_token_head(d=128, C=CHUNK):
    return (2 * (5 * C * C * d + 3 * C * d * d) + C ** 3 / 3) / C


def window_pairs(T, L, w, dil, frame_offset=0, centered=False):
    """Exact (query, key) pair count of one windowed branch (all groups):
    causal (i - w, i], or centred |j - i| <= floor(w / 2)."""
    F = -(-T // L)
    total = 0
    for r in range(dil):
        n = 0
        for f in range(F):
            if (f + frame_offset) % dil == r:
                n += min(L, T - f * L)
        if centered:
            rad = w // 2
            side = n * (n - 1) // 2 if n <= rad + 1 else rad * (rad + 1) // 2 + (n - rad - 1) * rad
            total += n + 2 * side
        else:
            m = min(n, w)
            total += m * (m + 1) // 2 + (n - m) * w
    return total


def shared_frame_pairs(T, L, w, centered=False):
    """(query, key) pairs of a query's own frame inside its window: within a
    frame the SWA and DSWA positions differ by a constant, so both branches
    hold exactly these pairs, with the same scores when they score the same
    q and k; they are computed once.  Every pair the two windows share when
    w <= (dil - 1) L + 1 (causal) or floor(w / 2) < L (centred)."""
    total = 0
    for f in range(-(-T // L)):
        n = min(L, T - f * L)
        total += window_pairs(n, n, w, 1, 0, centered)
    return total


def hybrid_pairs(T, L, w, dil, centered=False, shared=True):
    """Distinct (query, key) pairs of the two windowed branches of the hybrid
    layer (SWA + DSWA, less the own-frame pairs they share when both score the
    same q and k, i.e. without RoPE)."""
    pairs = window_pairs(T, L, w, 1, 0, centered) + window_pairs(T, L, w, dil, 0, centered)
    return pairs - (shared_frame_pairs(T, L, w, centered) if shared and dil > 1 else 0)


def read_counter_summary(name):
    """key: value lines of a committed counter summary under profiles/."""
    out = {}
    path = os.path.join(ROOT, "profiles", name)
    if os.path.exists(path):
        for line in open(path):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                out[key.strip()] = val.strip()
    return out


def src_sha(*names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "video_world_model_chunkwise_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


# ------------------------------------------------------------------ CPU baseline

def _oracle_costs(w, Tg, rows_n, Hs, seed_off):
    """Oracle seconds per token of a layer workload's three parts (a token of
    one batch row, all heads: the workload takes B T times that), from a
    bounded sample: the gated delta rule over Tg tokens x all heads, the
    block quantiser (FP8 workloads) and both windowed branches for rows_n
    query rows of the last frame of a 2 dil + 1 frame prefix x Hs heads."""
    import numpy as np
    import oracle
    from workloads import make_custom
    inp = make_custom(1, Tg, w.H, w.d, "bf16", seed=w.seed + seed_off)
    t0 = time.perf_counter()
    oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    c_gdn = (time.perf_counter() - t0) / Tg                       # per token (one batch row, all heads)
    if not w.L:
        return {"gdn": c_gdn}
    F = 2 * w.dilation + 1
    inp = make_custom(1, F * w.L, Hs, w.d, "bf16", seed=w.seed + seed_off + 1)
    rows = np.arange((F - 1) * w.L, (F - 1) * w.L + rows_n)
    q, k = inp["q"], inp["k"]
    c_quant = 0.0
    if w.window_qk == "fp8":
        t0 = time.perf_counter()
        _, _, q = oracle.fp8_quantize_blocks(q)
        _, _, k = oracle.fp8_quantize_blocks(k)
        c_quant = (time.perf_counter() - t0) / (F * w.L) * (w.H / Hs)
    t0 = time.perf_counter()
    oracle.windowed_attention_rows(q, k, inp["v"], rows, w.L, w.window, 1)
    oracle.windowed_attention_rows(q, k, inp["v"], rows, w.L, w.window, w.dilation)
    c_win = (time.perf_counter() - t0) / len(rows) * (w.H / Hs)
    return {"gdn": c_gdn, "fp8_quant": c_quant, "windows": c_win}


def cpu_baseline(w, WORKLOADS):
    """The oracle (untuned) on bounded samples; tokens/s of the benchmark
    workload's whole layer extrapolated from per-token costs of its three
    parts, and the same figure for every workload."""
    import oracle
    from workloads import make_inputs
    try:
        from threadpoolctl import threadpool_info
        blas_threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    except Exception:
        blas_threads = 1
    t_all = time.perf_counter()
    Tg, rows_n, Hs = 8192, 1536, 4
    c = _oracle_costs(w, Tg, rows_n, Hs, 7)
    per_token = sum(c.values())
    # the same loop on one BLAS thread, over a quarter of the tokens
    c_gdn_1 = None
    try:
        from threadpoolctl import threadpool_limits
        from workloads import make_custom
        T1 = Tg // 4
        inp = make_custom(1, T1, w.H, w.d, "bf16", seed=w.seed + 9)
        with threadpool_limits(limits=1):
            t0 = time.perf_counter()
            oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
            c_gdn_1 = (time.perf_counter() - t0) / T1
    except Exception:
        pass
    # every workload: workload 0 whole; the others by the sampled per-token costs
    per_workload = {}
    w0 = WORKLOADS[0]
    inp = make_inputs(0)
    t0 = time.perf_counter()
    oracle.gdn_recurrent(inp["q"], inp["k"], inp["v"], inp["alpha"], inp["beta"])
    dt = time.perf_counter() - t0
    per_workload[w0.name] = {"seconds": round(dt, 4), "tokens_per_s": round(w0.B * w0.T / dt, 1),
                             "sample": "whole workload"}
    for wi in (1, 2, 3):
        ww = WORKLOADS[wi]
        cw = _oracle_costs(ww, 512, 128, 2, 11 + wi)
        pt = sum(cw.values())
        per_workload[ww.name] = {"tokens_per_s": round(1.0 / pt, 1), "est_seconds": round(pt * ww.B * ww.T, 1),
                                 "per_token_s": cw,
                                 "sample": "GDN 512 tokens x all heads" + ("" if not ww.L else
                                           "; windows 128 rows x 2 heads, scaled")}
    per_workload[w.name] = {"tokens_per_s": round(1.0 / per_token, 1), "est_seconds": round(per_token * w.B * w.T, 1),
                            "per_token_s": c, "sample": "the headline sample"}
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {
        "value": 1.0 / per_token, "unit": "tokens/s", "cores": int(blas_threads), "kind": "oracle",
        "threads": {"blas_threads": int(blas_threads), "logical_cpus": os.cpu_count(),
                    "affinity_cpus": affinity},
        "sample": (f"numpy fp64 oracle: gated delta rule over {Tg} tokens x {w.H} heads; "
                   f"E4M3 block quantiser over {(2 * w.dilation + 1) * w.L} tokens x {Hs} heads; SWA+DSWA for "
                   f"{rows_n} query rows (window {w.window}, dilation {w.dilation}) x {Hs} heads; "
                   f"per-token costs summed and scaled to {w.B} x {w.H} heads"),
        "seconds": round(time.perf_counter() - t_all, 2),
        "per_token_s": c,
        "gdn_tokens_per_s_1_thread": (round(1.0 / c_gdn_1, 1) if c_gdn_1 else None),
        "per_workload": per_workload,
        "host": host_description(),
    }


def host_description():
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "logical_cpus": os.cpu_count()}


# ------------------------------------------------------------------ GPU timing helpers

def time_stats(ms):
    """avg / min / median / p10 / p90 of a list of times (nearest-rank
    percentiles)."""
    ms = sorted(ms)
    n = len(ms)
    pick = lambda p: ms[min(n - 1, max(0, int(math.ceil(p * n)) - 1))]
    return {"avg_ms": sum(ms) / n, "min_ms": ms[0], "median_ms": pick(0.5), "p10_ms": pick(0.1),
            "p90_ms": pick(0.9), "n": n}


def versions(torch):
    """Software and device the numbers were taken with."""
    v = {"torch": torch.__version__, "hip_runtime": getattr(torch.version, "hip", None)}
    try:
        with open("/opt/rocm/.info/version") as f:
            v["rocm"] = f.read().strip()
    except OSError:
        v["rocm"] = None
    try:
        with open("/sys/module/amdgpu/version") as f:
            v["amdgpu_driver"] = f.read().strip()
    except OSError:
        v["amdgpu_driver"] = None
    try:
        p = torch.cuda.get_device_properties(0)
        v["device"] = {"name": p.name, "arch": getattr(p, "gcnArchName", None),
                       "compute_units": p.multi_processor_count, "memory_GB": round(p.total_memory / 1e9, 1)}
    except Exception:
        v["device"] = None
    return v


class StageTimer:
    """HIP events recorded on the current (launch) stream around each call."""

    def __init__(self, torch):
        self.torch = torch
        self.acc = {}

    def run(self, name, fn, reps, before=None):
        torch = self.torch
        fn()                                        # untimed: first launch loads the kernel
        torch.cuda.synchronize()
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
              for _ in range(reps)]
        for a, b in ev:
            if before is not None:
                before()                            # untimed (e.g. a cache flush)
            a.record()
            fn()
            b.record()
        torch.cuda.synchronize()
        self.acc[name] = time_stats([a.elapsed_time(b) for a, b in ev])
        return self.acc[name]["avg_ms"]


def gdn_segments_of(K, w):
    """Segments of the time-split scan for a shape, read back from the GDN
    workspace size (two D x D fp32 slots per (b, h) and segment when split)."""
    up = lambda x: (x + 255) // 256 * 256
    n = -(-w.T // 64)
    base = up(w.B * w.H * n * 64 * 64 * 2) + up(w.B * w.H * n * 64 * 4)
    extra = K.kairos_gdn_workspace_size(K.gdn_desc(w.B, w.T, w.H, w.d)) - base
    return max(1, extra // (2 * w.B * w.H * w.d * w.d * 4))


def layer_step_fn(K, d, w, bufs, fp8, ctx=None):
    def step():
        K.kairos_hlta_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L, w.window,
                          w.dilation, window_qk=K.FP8_E4M3 if fp8 else K.BF16, out=bufs["out"],
                          state_out=bufs["state"], workspace=bufs["ws"], ctx=ctx)
    return step


def alloc_layer(K, torch, w, d, fp8):
    desc = K.hlta_desc(w.B, w.T, w.H, w.d, w.L, w.window, w.dilation,
                       window_qk=K.FP8_E4M3 if fp8 else K.BF16)
    nws = K.kairos_hlta_workspace_size(desc)
    return {
        "out": torch.empty_like(d["v"]),
        "state": torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device="cuda:0"),
        "ws": torch.empty(max(nws, 1), dtype=torch.uint8, device="cuda:0"),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--quick", action="store_true", help="skip the per-workload breakdown")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="also run one plain 1 GiB device copy (reference for memory counters)")
    ap.add_argument("--gdn-workload", type=int, default=None,
                    help="only time kairos_gdn_fwd on this workload index (prints its own JSON line)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the benchmark runs on one GPU; sharding the path across GPUs is not "
              "implemented (use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch
    import video_world_model_chunkwise_amd as K
    from workloads import WORKLOADS, make_device_inputs

    K.lib()                                         # fail loudly if the library is missing
    torch.cuda.init()
    dev = torch.device("cuda:0")
    if args.gdn_workload is not None:
        gdn_only(K, torch, WORKLOADS[args.gdn_workload], make_device_inputs, args)
        return
    w = WORKLOADS[4]                                # B4 H24 d128, 16 x 3600 tokens, FP8 windows
    fp8 = w.window_qk == "fp8"
    d = make_device_inputs(w, dev)
    bufs = alloc_layer(K, torch, w, d, fp8)
    ctx = K.Context()                               # side stream of the layer calls
    step = layer_step_fn(K, d, w, bufs, fp8, ctx)
    print(f"[bench] workload {w.name}: inputs ready", file=sys.stderr, flush=True)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for a_ev, b_ev in evs:
        a_ev.record()
        step()
        b_ev.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_per_step = wall * 1e3 / max(args.steps, 1)
    step_stats = time_stats([a_ev.elapsed_time(b_ev) for a_ev, b_ev in evs]) if evs else None
    tokens = w.B * w.T
    value = tokens / (ms_per_step / 1e3)
    print(f"[bench] layer: {ms_per_step:.3f} ms/step", file=sys.stderr, flush=True)

    # ---- stages, each one kernel launch, timed with events on the launch stream
    st = StageTimer(torch)
    reps = max(args.steps, 3)
    codes_q = torch.empty(d["q"].shape, dtype=torch.uint8, device=dev)
    codes_k = torch.empty_like(codes_q)
    nb = (w.T + 63) // 64
    sq = torch.empty((w.B, w.H, nb), dtype=torch.float32, device=dev)
    sk = torch.empty_like(sq)
    o_gdn = torch.empty_like(d["v"])
    yws = torch.empty(4 * (d["v"].numel() + d["v"].numel() // w.d), dtype=torch.uint8, device=dev)
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device=dev)
    t_quant = st.run("fp8_quant_q", lambda: K.kairos_fp8_quantize(d["q"], codes_q, sq), reps)
    st.run("fp8_quant_k", lambda: K.kairos_fp8_quantize(d["k"], codes_k, sk), reps)
    t_gdn = st.run("gdn_chunk", lambda: K.kairos_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"],
                                                         out=o_gdn, state_out=S), reps)
    t_win = st.run("window_hybrid", lambda: K.kairos_hlta_window_fwd(
        codes_q, codes_k, d["v"], o_gdn, d["gates"], w.L, w.window, w.dilation, q_scales=sq,
        k_scales=sk, out=bufs["out"], workspace=yws), reps)
    # cold launches: the 256 MB Infinity Cache overwritten (a 512 MB fill) before each
    flush_buf = torch.empty(512 << 20, dtype=torch.uint8, device=dev)
    flush = lambda: flush_buf.fill_(1)
    t_layer_warm = st.run("layer_warm", step, reps)
    t_layer_cold = st.run("layer_cold", step, 3, before=flush)
    t_gdn_cold = st.run("gdn_chunk_cold", lambda: K.kairos_gdn_fwd(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o_gdn, state_out=S), 3, before=flush)
    del flush_buf
    # the same stage on 4-bit (E2M1) Q/K, and the whole layer with 4-bit windows
    c4q = torch.empty((w.B, w.T, w.H, w.d // 2), dtype=torch.uint8, device=dev)
    c4k = torch.empty_like(c4q)
    # scales of their own: the centred stage below reads the E4M3 scales
    sq4, sk4 = torch.empty_like(sq), torch.empty_like(sk)
    t_q4 = st.run("fp4_quant_q", lambda: K.kairos_fp4_quantize(d["q"], c4q, sq4), reps)
    K.kairos_fp4_quantize(d["k"], c4k, sk4)
    t_win4 = st.run("window_hybrid_fp4", lambda: K.kairos_hlta_window_fwd(
        c4q, c4k, d["v"], o_gdn, d["gates"], w.L, w.window, w.dilation, q_scales=sq4,
        k_scales=sk4, out=bufs["out"], workspace=yws), reps)
    desc4 = K.hlta_desc(w.B, w.T, w.H, w.d, w.L, w.window, w.dilation, window_qk=K.FP4_E2M1)
    ws4 = torch.empty(K.kairos_hlta_workspace_size(desc4), dtype=torch.uint8, device=dev)
    t_layer4 = st.run("layer_fp4", lambda: K.kairos_hlta_fwd(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L, w.window, w.dilation,
        window_qk=K.FP4_E2M1, out=bufs["out"], state_out=bufs["state"], workspace=ws4, ctx=ctx), reps)
    del ws4, c4q, c4k, sq4, sk4
    # the same stage with centred windows (Eq. 7 as printed) and the pages' DSWA dilation 6
    t_win_c = st.run("window_hybrid_centered_dil6", lambda: K.kairos_hlta_window_fwd(
        codes_q, codes_k, d["v"], o_gdn, d["gates"], w.L, w.window, 6, q_scales=sq,
        k_scales=sk, out=bufs["out"], workspace=yws, centered=True), reps)

    # input prologue of the gated delta rule on the same shape: raw keys and
    # gate logits -> unit keys and gates ("k": the canonical inputs), and with
    # query normalisation and the printed-Eq.-6 rescaling ("qk_literal": every
    # stream the kernel can move)
    gen = torch.Generator(device=dev)
    gen.manual_seed(w.seed + 7)
    za = 4.0 - torch.randn((w.B, w.T, w.H), generator=gen, device=dev)
    zb = torch.randn((w.B, w.T, w.H), generator=gen, device=dev)
    p_k, p_q, p_v = (torch.empty_like(d["v"]) for _ in range(3))
    p_a, p_b = torch.empty_like(za), torch.empty_like(zb)
    t_pro_k = st.run("gdn_prologue_k", lambda: K.kairos_gdn_prologue(
        d["q"], za, zb, k_out=p_k, alpha_out=p_a, beta_out=p_b), reps)
    t_pro_all = st.run("gdn_prologue_qk_literal", lambda: K.kairos_gdn_prologue(
        d["q"], za, zb, q=d["k"], v=d["v"], literal=True, k_out=p_k, alpha_out=p_a, beta_out=p_b,
        q_out=p_q, v_out=p_v), reps)
    # RoPE fused with the E4M3 quantiser (one tensor, DSWA positions), and the
    # whole layer with RoPE on both windowed branches
    t_rope = st.run("rope_fp8_q", lambda: K.kairos_rope(d["q"], w.L, w.dilation, 1e4, fp8=True,
                                                        out=codes_q, scales=sq), reps)
    rope_bytes = d["q"].numel() * 3 + sq.numel() * 4          # bf16 in, codes + scales out
    desc_r = K.hlta_desc(w.B, w.T, w.H, w.d, w.L, w.window, w.dilation,
                         window_qk=K.FP8_E4M3 if fp8 else K.BF16, rope_base=1e4)
    ws_r = torch.empty(K.kairos_hlta_workspace_size(desc_r), dtype=torch.uint8, device=dev)
    t_layer_rope = st.run("layer_rope", lambda: K.kairos_hlta_fwd(
        d["q"], d["k"], d["v"], d["alpha"], d["beta"], d["gates"], w.L, w.window, w.dilation,
        window_qk=K.FP8_E4M3 if fp8 else K.BF16, out=bufs["out"], state_out=bufs["state"],
        workspace=ws_r, rope_base=1e4, ctx=ctx), reps)
    del ws_r
    rows = w.B * w.T * w.H
    pro_bytes = {"gdn_prologue_k": rows * (2 * w.d * 2 + 16),
                 "gdn_prologue_qk_literal": rows * (6 * w.d * 2 + 16)}
    del p_k, p_q, p_v, p_a, p_b, za, zb

    # distinct pairs: the own-frame pairs that SWA and DSWA share count once
    pairs = hybrid_pairs(w.T, w.L, w.window, w.dilation)
    pairs_branches = window_pairs(w.T, w.L, w.window, 1) + window_pairs(w.T, w.L, w.window, w.dilation)
    win_flops = pairs * 4 * w.d * w.B * w.H          # QK^T 2d + PV 2d per (query, key) pair
    pairs_c = hybrid_pairs(w.T, w.L, w.window, 6, centered=True)
    win_flops_c = pairs_c * 4 * w.d * w.B * w.H
    if fp8:
        # QK^T at the fp8 peak, PV at the bf16 peak: time-weighted (blended) peak
        peak = 2.0 / (1.0 / PEAK_FP8_TFLOPS + 1.0 / PEAK_BF16_TFLOPS)
    else:
        peak = PEAK_BF16_TFLOPS
    achieved = win_flops / (t_win / 1e3) / 1e12
    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": round(peak, 1),
                "unit": "TFLOP/s", "frac": round(achieved / peak, 4), "traffic": None,
                "kernel": "win_attn_kernel<1 (E4M3), hybrid>",
                "algorithmic_flops_per_launch": win_flops,
                "avg_launch_ms": round(t_win, 4)}
    # HBM traffic of the kernel from the committed counter summary, valid only
    # while the kernel's sources are the ones the counters were taken on
    cpath = os.path.join(ROOT, "profiles", "hlta_fp8_B4H24F16L3600_hbm_counters.txt")
    cnt = {}
    if fp8 and os.path.exists(cpath):
        for line in open(cpath):
            if ":" in line and not line.startswith("#"):
                key, val = line.split(":", 1)
                cnt[key.strip()] = val.strip()
    win_fresh = cnt.get("win_attn_kernel.source_sha") == src_sha("window_attn.hip", "common.hpp", "launch.hpp")
    if win_fresh:
        roofline["traffic"] = float(cnt["win_attn_kernel.traffic_bytes_per_launch"])
    # the second ceiling of the window kernel: one exponential per (query, key)
    # pair at the transcendental rate, and (from the committed SQ counters,
    # while they match the kernel's source) the VALU and MFMA issue times
    exps = pairs * w.B * w.H
    roofline["exp_ceiling"] = {"exps_per_launch": exps, "peak_per_s": PEAK_EXP_PER_S,
                               "bound_ms": round(exps / PEAK_EXP_PER_S * 1e3, 4),
                               "frac": round(exps / PEAK_EXP_PER_S * 1e3 / t_win, 4)}
    sq = read_counter_summary("hlta_fp8_B4H24F16L3600_sq_counters.txt")
    if sq.get("win_attn_kernel.source_sha") == src_sha("window_attn.hip", "common.hpp", "launch.hpp"):
        v = float(sq["win_attn_kernel.SQ_INSTS_VALU"])
        tr = float(sq["win_attn_kernel.SQ_INSTS_VALU_TRANS_F32"])
        m = float(sq["win_attn_kernel.SQ_VALU_MFMA_BUSY_CYCLES"])
        # the shader clock the kernel actually ran at (GPU busy cycles over the
        # dispatch's duration in the counter pass): busy cycles become time at
        # that clock, and the published peak assumes the 2.4 GHz maximum
        clk = float(sq.get("win_attn_kernel.shader_clock_hz", CLOCK_HZ))
        roofline["counters"] = {
            "valu_insts_per_launch": v, "trans_insts_per_launch": tr,
            "mfma_insts_per_launch": float(sq["win_attn_kernel.SQ_INSTS_MFMA"]),
            "shader_clock_ghz": round(clk / 1e9, 3),
            "valu_issue_ms": round(((v - tr) * VALU_ISSUE_CLK + tr * TRANS_ISSUE_CLK) / SIMDS / clk * 1e3, 4),
            "mfma_busy_ms": round(m / SIMDS / clk * 1e3, 4),
            "frac_of_peak_at_shader_clock": round(roofline["frac"] * CLOCK_HZ / clk, 4),
            "source": "profiles/hlta_fp8_B4H24F16L3600_sq_counters.txt"}
    pro_fresh = cnt.get("gdn_prologue_kernel.source_sha") == src_sha("prologue.hip", "common.hpp",
                                                                    "launch.hpp")

    gdn_tok_heads = w.B * w.T * w.H
    gdn_bytes = gdn_tok_heads * GDN_BYTES_PER_TOKEN_HEAD + 2 * w.B * w.H * w.d * w.d * 4
    gdn_flops = gdn_tok_heads * gdn_flops_per_token_head(w.d)
    # the gated delta rule's own roofline (HBM-bound): its launch sequence
    # (prep + scan) timed as one stage, algorithmic bytes over that time
    gdn_ach = gdn_bytes / (t_gdn / 1e3) / 1e9
    roofline_gdn = {"bound": "hbm", "achieved": round(gdn_ach, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                    "frac": round(gdn_ach / PEAK_HBM_GBS, 4), "traffic": None,
                    "kernel": "gdn_prep_kernel + gdn_scan_kernel (one kairos_gdn_fwd)",
                    "algorithmic_bytes_per_launch": gdn_bytes, "avg_launch_ms": round(t_gdn, 4),
                    "median_ms": round(st.acc["gdn_chunk"]["median_ms"], 4)}
    if cnt.get("gdn_scan_kernel.source_sha") == src_sha("gdn.hip", "common.hpp", "launch.hpp") \
            and "gdn.traffic_bytes_per_launch" in cnt:
        roofline_gdn["traffic"] = float(cnt["gdn.traffic_bytes_per_launch"])
    breakdown = {
        "stages_ms": {k: round(v["avg_ms"], 4) for k, v in st.acc.items()},
        "stages_stats_ms": {k: {q: round(x, 4) for q, x in v.items() if q != "avg_ms"}
                            for k, v in st.acc.items()},
        "gdn_branch": {
            "ms": round(t_gdn, 4), "tokens_per_s": round(tokens / (t_gdn / 1e3)),
            "alg_GB_per_s": round(gdn_bytes / (t_gdn / 1e3) / 1e9, 1),
            "hbm_frac": round(gdn_bytes / (t_gdn / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
            "alg_TFLOP_per_s": round(gdn_flops / (t_gdn / 1e3) / 1e12, 1),
            "bf16_mfma_frac": round(gdn_flops / (t_gdn / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4),
        },
        "window_stage": {"ms": round(t_win, 4), "alg_TFLOP_per_s": round(achieved, 1),
                         "pairs_per_bh": pairs, "pairs_per_bh_both_branches": pairs_branches},
        "cold_vs_warm": {"layer_warm_ms": round(t_layer_warm, 4), "layer_cold_ms": round(t_layer_cold, 4),
                         "gdn_branch_warm_ms": round(t_gdn, 4), "gdn_branch_cold_ms": round(t_gdn_cold, 4),
                         "flush": "512 MB fill before each timed launch (Infinity Cache 256 MB)"},
        "fp4": {
            "quant_q_ms": round(t_q4, 4),
            "quant_alg_GB_per_s": round(d["q"].numel() * 2.5 / (t_q4 / 1e3) / 1e9, 1),
            "window_stage_ms": round(t_win4, 4),
            "window_alg_TFLOP_per_s": round(win_flops / (t_win4 / 1e3) / 1e12, 1),
            "window_mfma_frac": round(win_flops / (t_win4 / 1e3) / 1e12 / PEAK_FP4_BLEND_TFLOPS, 4),
            "layer_ms": round(t_layer4, 4), "layer_tokens_per_s": round(tokens / (t_layer4 / 1e3)),
        },
        "window_stage_centered_dil6": {
            "ms": round(t_win_c, 4), "pairs_per_bh": pairs_c,
            "alg_TFLOP_per_s": round(win_flops_c / (t_win_c / 1e3) / 1e12, 1),
            "mfma_frac": round(win_flops_c / (t_win_c / 1e3) / 1e12 / peak, 4)},
        "rope": {
            "rope_fp8_q": {"ms": round(t_rope, 4), "alg_bytes": rope_bytes,
                           "alg_GB_per_s": round(rope_bytes / (t_rope / 1e3) / 1e9, 1),
                           "hbm_frac": round(rope_bytes / (t_rope / 1e3) / 1e9 / PEAK_HBM_GBS, 4)},
            "layer_rope": {"ms": round(t_layer_rope, 4),
                           "tokens_per_s": round(tokens / (t_layer_rope / 1e3))},
        },
        "gdn_prologue": {
            name: {"ms": round(t, 4), "alg_bytes": pro_bytes[name],
                   "alg_GB_per_s": round(pro_bytes[name] / (t / 1e3) / 1e9, 1),
                   "hbm_frac": round(pro_bytes[name] / (t / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                   "traffic": (float(cnt[name + ".traffic_bytes_per_launch"])
                               if pro_fresh and name + ".traffic_bytes_per_launch" in cnt else None)}
            for name, t in (("gdn_prologue_k", t_pro_k), ("gdn_prologue_qk_literal", t_pro_all))},
    }
    del codes_q, codes_k, o_gdn, d, bufs
    torch.cuda.empty_cache()

    if not args.quick:
        breakdown.update(workload_breakdown(K, torch, WORKLOADS, make_device_inputs, reps, ctx))
    if args.calibrate_copy:
        src = torch.empty(1 << 29, dtype=torch.bfloat16, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    cpu = None
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline ...", file=sys.stderr, flush=True)
        cpu = cpu_baseline(w, WORKLOADS)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3+bf16" if fp8 else "bf16", "data": "synthetic",
        "config": {"workload": w.name, "B": w.B, "T": w.T, "H": w.H, "d": w.d, "L": w.L,
                   "frames": w.T // w.L, "window": w.window, "dilation": w.dilation,
                   "window_qk": "fp8_e4m3" if fp8 else "bf16", "chunk": CHUNK},
        "roofline": roofline, "roofline_gdn": roofline_gdn, "cpu_baseline": cpu,
        "step_ms": ({k: round(v, 4) for k, v in step_stats.items() if k != "n"} if step_stats else None),
        "versions": versions(torch), "breakdown": breakdown,
    }
    print(json.dumps(line), flush=True)


def gdn_only(K, torch, w, make_device_inputs, args):
    """kairos_gdn_fwd alone on one workload: W untimed calls, then K calls
    timed with events on the launch stream; one JSON line."""
    d = make_device_inputs(w, torch.device("cuda:0"))
    o = torch.empty_like(d["v"])
    S = torch.empty((w.B, w.H, w.d, w.d), dtype=torch.float32, device="cuda:0")
    ws = torch.empty(max(1, K.kairos_gdn_workspace_size(K.gdn_desc(w.B, w.T, w.H, w.d))), dtype=torch.uint8,
                     device="cuda:0")
    fn = lambda: K.kairos_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o, state_out=S, workspace=ws)
    for _ in range(args.warmup):
        fn()
    st = StageTimer(torch)
    st.run("gdn", fn, max(args.steps, 1))
    r = st.acc["gdn"]
    gb = w.B * w.T * w.H * GDN_BYTES_PER_TOKEN_HEAD + 2 * w.B * w.H * w.d * w.d * 4
    print(json.dumps({"gdn_workload": w.name, "steps": args.steps, **{k: round(v, 4) for k, v in r.items()},
                      "alg_bytes": gb, "alg_GB_per_s": round(gb / (r["avg_ms"] / 1e3) / 1e9, 1),
                      "hbm_frac": round(gb / (r["avg_ms"] / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                      "scan_segments": gdn_segments_of(K, w)}), flush=True)


def workload_breakdown(K, torch, WORKLOADS, make_device_inputs, reps, ctx):
    out = {}
    dev = torch.device("cuda:0")
    st = StageTimer(torch)
    # gated delta rule alone, B2 H16 T4096
    w1 = WORKLOADS[1]
    d = make_device_inputs(w1, dev)
    o = torch.empty_like(d["v"])
    S = torch.empty((w1.B, w1.H, w1.d, w1.d), dtype=torch.float32, device=dev)
    fn = lambda: K.kairos_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o, state_out=S)
    fn()
    t = st.run("gdn_B2H16T4096", fn, reps)
    th = w1.B * w1.T * w1.H
    out["gdn_B2H16T4096"] = {"ms": round(t, 4), "tokens_per_s": round(w1.B * w1.T / (t / 1e3)),
                             "alg_GB_per_s": round(th * GDN_BYTES_PER_TOKEN_HEAD / (t / 1e3) / 1e9, 1)}
    del d, o, S
    # bf16 hybrid layer, B1 H24 21 x 1560, and its gated delta rule branch alone
    w2 = WORKLOADS[2]
    d = make_device_inputs(w2, dev)
    o = torch.empty_like(d["v"])
    S = torch.empty((w2.B, w2.H, w2.d, w2.d), dtype=torch.float32, device=dev)
    fn = lambda: K.kairos_gdn_fwd(d["q"], d["k"], d["v"], d["alpha"], d["beta"], out=o, state_out=S)
    t = st.run("gdn_B1H24T32760", fn, reps)
    th = w2.B * w2.T * w2.H
    gb = th * GDN_BYTES_PER_TOKEN_HEAD + 2 * w2.B * w2.H * w2.d * w2.d * 4
    out["gdn_B1H24T32760"] = {"ms": round(t, 4), "median_ms": round(st.acc["gdn_B1H24T32760"]["median_ms"], 4),
                              "tokens_per_s": round(w2.B * w2.T / (t / 1e3)),
                              "alg_GB_per_s": round(gb / (t / 1e3) / 1e9, 1),
                              "hbm_frac": round(gb / (t / 1e3) / 1e9 / PEAK_HBM_GBS, 4),
                              "scan_segments": gdn_segments_of(K, w2)}
    del o, S
    bufs = alloc_layer(K, torch, w2, d, False)
    fn = layer_step_fn(K, d, w2, bufs, False, ctx)
    fn()
    t = st.run("layer_bf16_B1H24F21L1560", fn, reps)
    pairs = hybrid_pairs(w2.T, w2.L, w2.window, w2.dilation)
    fl = pairs * 4 * w2.d * w2.B * w2.H + w2.B * w2.T * w2.H * gdn_flops_per_token_head(w2.d)
    out["layer_bf16_B1H24F21L1560"] = {"ms": round(t, 4), "tokens_per_s": round(w2.B * w2.T / (t / 1e3)),
                                       "alg_TFLOP_per_s": round(fl / (t / 1e3) / 1e12, 1),
                                       "bf16_mfma_frac": round(fl / (t / 1e3) / 1e12 / PEAK_BF16_TFLOPS, 4)}
    del d, bufs
    # streamed rollout, 61 frames x 1560, one call per frame with state carry and ring
    w3 = WORKLOADS[3]
    d = make_device_inputs(w3, dev)
    R = w3.ring_frames
    kr = torch.zeros((w3.B, R, w3.L, w3.H, w3.d), dtype=torch.bfloat16, device=dev)
    vr = torch.zeros_like(kr)
    state = torch.zeros((w3.B, w3.H, w3.d, w3.d), dtype=torch.float32, device=dev)
    L = w3.L
    frames = [{key: d[key][:, f * L:(f + 1) * L].contiguous() for key in ("q", "k", "v", "alpha", "beta")}
              for f in range(w3.T // L)]
    y = torch.empty_like(frames[0]["v"])
    desc = K.hlta_desc(w3.B, L, w3.H, w3.d, L, w3.window, w3.dilation, ring_frames=R)
    ws = torch.empty(max(K.kairos_hlta_workspace_size(desc), 1), dtype=torch.uint8, device=dev)

    def rollout():
        for f, fr in enumerate(frames):
            K.kairos_hlta_fwd(fr["q"], fr["k"], fr["v"], fr["alpha"], fr["beta"], d["gates"], L,
                              w3.window, w3.dilation, frame_offset=f, state_in=state, state_out=state,
                              ring_frames=R, k_ring=kr, v_ring=vr, out=y, workspace=ws, ctx=ctx)
    rollout()
    t = st.run("stream_B1H24F61L1560", rollout, 3)
    out["stream_B1H24F61L1560"] = {"ms_total": round(t, 3), "ms_per_frame": round(t / len(frames), 4),
                                   "tokens_per_s": round(w3.T / (t / 1e3))}
    del d, frames, kr, vr
    torch.cuda.empty_cache()
    return out


if __name__ == "__main__":
    main()
