#!/usr/bin/env python3
"""Benchmark of the MI355X W4 MoE expert layer.

One step = one pass of the whole hot path over one batch of T tokens:
moe_route -> moe_w4_gate_up -> moe_w4_down -> moe_combine, on the
prefill workload of 512 tokens (hidden 2048, 256 routed experts top-8 plus one
shared expert, expert intermediate 512, 4-bit weights in groups of 64).
Inputs are resident in HBM before timing starts; R copies of the weights (and
router) are rotated so that no call finds the previous call's weights in the
256 MB Infinity Cache.

Prints one JSON line.  Also measured (reported under "extra"): the
2048-token Zipf-skewed prefill (MFMA fraction of the two GEMMs) and batch-1
decode (HBM fraction of the two GEMMs; its launch-bound steps are timed from
HIP graph replays), and the CPU oracle on the host cores.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0          # MI355X HBM3E
PEAK_BF16_TFLOPS = 2500.0      # MI355X dense bf16 MFMA
PEAK_FP32_TFLOPS = 157.3       # MI355X fp32 vector, published (packed fp32 instructions)
# 256 CUs x 4 SIMDs x 16 lanes x 2 flops (one fused multiply-add) x 2.4 GHz:
# the fp32 vector rate without packed instructions, which this build never emits
PEAK_FP32_UNPACKED_TFLOPS = 256 * 4 * 16 * 2 * 2.4e9 / 1e12
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_gate_up_prefill512.txt")
DOMINANT = "w4_gemm_small_kernel<4, 2, true, 0>"   # the gate/up GEMM of the 512-token workload
# Tile height bound per workload: uniform routing at 512 tokens gives every
# expert 7-27 rows, so 32-row tiles cover them and the shared expert's 512
# rows in 16 blocks; the skewed 2048-token batch has groups of up to ~2000
# rows that want tall tiles; batch-1 decode has one row per group.
TILE_M_MAX = {"prefill512": 32, "prefill2048_zipf": 128, "chunked16384": 128, "decode1": 32}


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=200)
    p.add_argument("--warmup", type=int, default=50)
    p.add_argument("--copies", type=int, default=4, help="weight copies rotated between steps")
    p.add_argument("--tile-m-max", type=int, default=None,
                   help="largest GEMM tile height (default: per workload)")
    p.add_argument("--no-extra", action="store_true", help="skip the 2048-token, decode and chunked-prompt legs")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    p.add_argument("--overlap", action="store_true",
                   help="run the shared expert's FFN on a second stream, concurrent with routing")
    p.add_argument("--calib-copy-mb", type=int, default=0,
                   help="also run one plain device copy of this size (counter calibration)")
    p.add_argument("--only", choices=["prefill512", "prefill2048_zipf", "decode1", "chunked16384",
                                      "small_batches", "ablations", "tile_sweep", "gdn_prefill2048"],
                   default=None,
                   help="time a single workload (profiling runs)")
    p.add_argument("--traffic-from", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"), default=None,
                   help="turn two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE) of "
                        "'--only prefill512 --calib-copy-mb N' into the stored traffic record")
    return p.parse_args()


def kernel_source_hash() -> str:
    """Hash of the GEMM kernels' sources with comments and whitespace removed,
    so the stored traffic record survives edits that leave the code alone."""
    import re
    h = hashlib.sha256()
    for f in ("moe_common.h", "route.h", "ffn.hip"):
        with open(os.path.join(ROOT, "w4_dequant_expert_amd", "csrc", f)) as fh:
            text = fh.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()[:16]


class Workload:
    """Device-resident inputs of one configuration and R rotated weight copies."""

    def __init__(self, name, copies, tile_m_max=None, T=None):
        import numpy as np
        import torch

        import w4_dequant_expert_amd as moe
        from synth import build_config

        c = build_config(name, T=T)
        sh = c["shape"]
        tile_m_max = tile_m_max or TILE_M_MAX[name]
        self.tile_m_max = tile_m_max
        self.name, self.c, self.sh = name, c, sh
        self.T = c["T"]
        base_r = moe.DeviceBank(c["routed"])
        base_s = moe.DeviceBank(c["shared"])
        wr = torch.from_numpy(c["wr"]).to("cuda")
        bias = None if c["bias"] is None else torch.from_numpy(c["bias"]).to("cuda")
        self.copies = [(base_r, base_s, wr)]
        for _ in range(copies - 1):
            self.copies.append((base_r.clone(), base_s.clone(), wr.clone()))
        self.layer = moe.MoeLayer(sh.H, sh.I, sh.E, sh.k, sh.n_shared, base_r, base_s, wr, bias,
                                  T_max=max(self.T, 1), tile_m_max=tile_m_max, export_logits=False)
        self.x = torch.from_numpy(c["x"].view(np.int16)).to("cuda")
        self.y = torch.empty((self.T, sh.H), dtype=torch.int16, device="cuda")
        # second stream (default priority) for the shared expert, and its events
        self.side = torch.cuda.Stream()
        self.ready = torch.cuda.Event()
        self.done = torch.cuda.Event()

    def step(self, i, ev=None, x=None, overlap=False):
        """One layer call.  Without events: route, then the FFN and the combine
        in one library call (down and combine fused for one token), on one
        stream; with overlap, the shared expert's FFN on a
        second stream, concurrent with routing (it needs no routing tables),
        the routed experts' FFN after routing, and the combine once both are
        done.  With events (the stage breakdown): route, gate/up, down and
        combine in sequence on one stream, each stage between its own events."""
        import torch
        r, s, wr = self.copies[i % len(self.copies)]
        L = self.layer
        L.w_router = wr
        x = self.x if x is None else x
        if ev is None and not overlap:  # one stream: route, then FFN and combine in one call
            d = L.route(x)
            L.ffn_combine(d, x, self.y, r, s)
            return
        if ev is None:
            main = torch.cuda.current_stream()
            if self.sh.n_shared:
                # after the previous call's combine has read y_slots
                self.ready.record(main)
                self.side.wait_event(self.ready)
                L.shared_ffn(L.dims(x.shape[0]), x, s, stream=self.side)
            d = L.route(x)
            L.routed_ffn(d, x, r)
            if self.sh.n_shared:
                self.done.record(self.side)
                main.wait_event(self.done)
            L.combine(d, self.y)
            return
        ev[0].record()
        d = L.route(x)
        ev[1].record()
        L.gate_up(d, x, r, s)
        ev[2].record()
        L.down(d, r, s)
        ev[3].record()
        L.combine(d, self.y)
        ev[4].record()

    def work(self):
        """Algorithmic flops and bytes of one call, from the real routing counts."""
        import torch
        torch.cuda.synchronize()
        counts = self.layer.rt.counts.cpu().numpy()
        sh, T = self.sh, self.T
        H, I, E, k = sh.H, sh.I, sh.E, sh.k
        rows = T * k + (T if sh.n_shared else 0)
        touched = int((counts > 0).sum()) + sh.n_shared
        gu_w = 2 * I * H * 9 // 16           # 4.5 bits per weight
        dn_w = H * I * 9 // 16
        # algorithmic bytes (what the method must move): the touched experts'
        # 4.5-bit weights, x, the router and y; h and y_slots are the
        # implementation's intermediates, reported apart
        return dict(
            rows=rows, touched=touched,
            flops_gate_up=rows * 4 * H * I, flops_down=rows * 2 * H * I,
            bytes_gate_up=touched * gu_w + T * H * 2,
            bytes_down=touched * dn_w,
            bytes_layer=touched * (gu_w + dn_w) + H * E * 4 + 2 * T * H * 2,
            bytes_h=2 * rows * I, bytes_y_slots=2 * rows * H,
        )


TIMING_NOTE = ("tokens_per_s and ms_per_step: wall clock of whole layer calls (route, grouped "
               "FFN, combine) with no events in between, after an untimed pass of the stage "
               "launches and the warm-up calls; stage times: per-launch averages of back-to-back "
               "launches of each stage alone between two HIP events, after the timed calls")


def time_workload(wl, steps, warmup, fresh_tokens=None, overlap=False, fixed_copy=None, stages=True):
    """`warmup` untimed and `steps` timed whole layer calls with no events in
    between (overlap: the shared expert on a second stream), wall clock; then
    the average duration (ms) of each stage's launches -- moe_route,
    moe_w4_gate_up, moe_w4_down, moe_combine -- from max(steps, 50)
    back-to-back launches of that stage alone between two HIP events on the
    stream they run on (rotating weight copies; the tables of one routing
    call).  One untimed pass of the stage launches comes first, so that the
    timed calls run at the clocks the same work settles to, whatever the
    warm-up count.  fixed_copy: every call uses that weight copy (the warm,
    R = 1 measurement); stages=False skips the stage launches."""
    import torch
    tok = (lambda i: None) if fresh_tokens is None else (lambda i: fresh_tokens[i % len(fresh_tokens)])
    cp = (lambda i: i) if fixed_copy is None else (lambda i: fixed_copy)
    wl.step(cp(0), x=tok(0), overlap=overlap)  # routing tables for the stage launches
    if stages:
        stage_times(wl, max(steps, 50))
    for i in range(warmup):
        wl.step(cp(i), x=tok(i), overlap=overlap)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        wl.step(cp(warmup + i), x=tok(warmup + i), overlap=overlap)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    return wall, (stage_times(wl, max(steps, 50)) if stages else {})


def stage_times(wl, n):
    """Average per-launch duration of each stage, n back-to-back launches each."""
    import torch
    L = wl.layer
    x = wl.x
    cp = wl.copies

    def route(i):
        L.w_router = cp[i % len(cp)][2]
        L.route(x)
    d = L.dims(x.shape[0])
    out = {}
    for name, fn in (("route_ms", route),
                     ("gate_up_ms", lambda i: L.gate_up(d, x, cp[i % len(cp)][0], cp[i % len(cp)][1])),
                     ("down_ms", lambda i: L.down(d, cp[i % len(cp)][0], cp[i % len(cp)][1])),
                     ("combine_ms", lambda i: L.combine(d, wl.y))):
        fn(0)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(n):
            fn(i)
        e1.record()
        torch.cuda.synchronize()
        out[name] = e0.elapsed_time(e1) / n
    L.w_router = cp[0][2]
    return out


def graph_ms(fn, n_inner, replays=5):
    """Device time per call of fn(i), i = 0..n_inner-1, captured once in a HIP
    graph and replayed: launch-bound calls then run back to back."""
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(n_inner):
            fn(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(n_inner):
            fn(i)
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(replays):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (replays * n_inner)


def stream_ceiling(nbytes, copies=40, workgroups=(256, 512, 1024, 2048, 4096), graph=True):
    """The streaming-read ceiling B' for nbytes per launch: moe_read_probe over
    `copies` distinct buffers (more than the Infinity Cache holds), the best
    launch shape counting.  graph=True replays the launches from a HIP graph,
    like the decode steps; graph=False times back-to-back launches with HIP
    events on the stream they run on (large single launches, like the
    prefill GEMMs).  Also the per-launch time of a one-workgroup probe of 16
    bytes (a kernel that does nothing measurable), the graph's fixed cost per
    kernel node."""
    import torch

    import w4_dequant_expert_amd as moe
    n = (nbytes + 15) // 16 * 16
    bufs = [torch.ones(n, dtype=torch.uint8, device="cuda") for _ in range(copies)]
    sink = torch.zeros(max(workgroups), dtype=torch.int32, device="cuda")
    stream = torch.cuda.current_stream()  # the events' stream (events mode)

    def events_ms(fn, reps=3):
        for i in range(copies):
            fn(i)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for r in range(reps):
            for i in range(copies):
                fn(i)
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / (reps * copies)

    timer = (lambda fn: graph_ms(fn, copies)) if graph else events_ms
    best = None
    per_wg = {}
    for wg in workgroups:
        # the stream current at each call: under graph capture, the capturing one
        ms = timer(lambda i: moe.moe_read_probe(bufs[i], n, sink, wg, torch.cuda.current_stream()))
        per_wg[wg] = round(ms * 1e3, 3)
        if best is None or ms < best[0]:
            best = (ms, wg)
    empty_ms = timer(lambda i: moe.moe_read_probe(bufs[i], 16, sink, 1, torch.cuda.current_stream()))
    del bufs
    return dict(bytes=n, best_us=round(best[0] * 1e3, 3), workgroups=best[1],
                gbs=n / (best[0] * 1e-3) / 1e9, us_by_workgroups=per_wg,
                empty_kernel_us=round(empty_ms * 1e3, 3),
                timing="hip graph replay" if graph else "hip events, back-to-back launches")


def mfma_ceiling(workgroups=512, iters=4000, reps=3):
    """The achievable bf16 matrix-core rate P': moe_mfma_probe with the tall
    GEMM's launch shape (four-wave workgroups, two per CU), timed with HIP
    events on the stream it runs on; the best of `reps` launches."""
    import torch

    import w4_dequant_expert_amd as moe
    sink = torch.zeros(workgroups * 4, dtype=torch.float32, device="cuda")
    stream = torch.cuda.current_stream()
    moe.moe_mfma_probe(workgroups, 10, sink, stream)
    best = None
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        moe.moe_mfma_probe(workgroups, iters, sink, stream)
        e1.record(stream)
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1)
        best = ms if best is None else min(best, ms)
    flops = workgroups * 4 * iters * 8 * 32 * 32 * 16 * 2
    return dict(tflops=flops / (best * 1e-3) / 1e12, ms=best, workgroups=workgroups, iters=iters)


def decode_leg(copies=40):
    """Batch-1 decode: whole steps and each stage timed from HIP graph replays
    (40 steps per graph, each with its own weight copy and fresh token)."""
    import numpy as np
    import torch

    from synth import make_tokens
    wl = Workload("decode1", copies)
    fresh = [torch.from_numpy(make_tokens(1, 2048, 4, t0=i).view(np.int16)).to("cuda")
             for i in range(copies)]
    for i in range(5):
        wl.step(i, x=fresh[i], overlap=False)
    # eager steps (host launch overhead included) for reference; one stream,
    # as in the captured graph
    w_eager, _ = time_workload(wl, 200, 20, fresh, overlap=False)
    step_ms = graph_ms(lambda i: wl.step(i, x=fresh[i], overlap=False), copies)
    # warm (R = 1): every step of the graph reads weight copy 0
    warm_ms = graph_ms(lambda i: wl.step(0, x=fresh[i], overlap=False), copies)
    # the shared expert's FFN on a second stream (a parallel branch of the
    # graph), concurrent with routing; then the routed experts and the combine
    overlap_ms = graph_ms(lambda i: wl.step(i, x=fresh[i], overlap=True), copies)
    L = wl.layer
    d = L.dims(1)
    x0 = fresh[0]
    L.route(x0)

    def route(i):
        L.w_router = wl.copies[i][2]
        L.route(fresh[i])
    route_ms = graph_ms(route, copies)
    L.w_router = wl.copies[0][2]
    L.route(x0)
    gu_ms = graph_ms(lambda i: L.gate_up(d, x0, wl.copies[i][0], wl.copies[i][1]), copies)
    dn_ms = graph_ms(lambda i: L.down(d, wl.copies[i][0], wl.copies[i][1]), copies)
    ffn_ms = graph_ms(lambda i: L.ffn(d, x0, wl.copies[i][0], wl.copies[i][1]), copies)
    cb_ms = graph_ms(lambda i: L.combine(d, wl.y), copies)
    wk = wl.work()
    g_s = (gu_ms + dn_ms) * 1e-3  # the two GEMM launches
    ceiling = stream_ceiling(wk["bytes_gate_up"] + wk["bytes_down"], copies)
    gemm_gbs = (wk["bytes_gate_up"] + wk["bytes_down"]) / g_s / 1e9
    out = dict(
        tokens_per_s=1.0 / (step_ms * 1e-3), ms_per_step=step_ms, timing="hip graph replay",
        shared_overlap_ms_per_step=round(overlap_ms, 5),
        warm_r1=dict(tokens_per_s=1.0 / (warm_ms * 1e-3), ms_per_step=round(warm_ms, 5), weight_copies=1,
                     note="warm: one weight copy reused by every step (served from the Infinity Cache)"),
        eager_tokens_per_s=200 / w_eager,
        route_ms=round(route_ms, 5), ffn_ms=round(ffn_ms, 5), combine_ms=round(cb_ms, 5),
        gate_up_ms=round(gu_ms, 5), down_ms=round(dn_ms, 5),
        gate_up_hbm_gbs=wk["bytes_gate_up"] / (gu_ms * 1e-3) / 1e9,
        down_hbm_gbs=wk["bytes_down"] / (dn_ms * 1e-3) / 1e9,
        gemm_hbm_gbs=gemm_gbs, gemm_frac_hbm=gemm_gbs / PEAK_HBM_GBS,
        stream_ceiling=ceiling, gemm_frac_of_stream_ceiling=gemm_gbs / ceiling["gbs"],
        gemm_bytes=wk["bytes_gate_up"] + wk["bytes_down"],
        bytes_per_token=wk["bytes_layer"], weight_copies=copies)
    del wl
    return out


def gdn_leg(reps=20, warmup=5):
    """The Gated DeltaNet scan over the 2048-token sequence (16 key heads, 32
    value heads of width 128), token by token (gdn_scan) and chunked
    (gdn_scan_chunked, both of its kernels): back-to-back calls timed with HIP
    events on the stream they run on; the faster form is reported.  Algorithmic work per token, value head and state
    element: the two dot products (2 fused multiply-adds) and the update (a
    multiply and a fused multiply-add), 7 flops."""
    import numpy as np
    import torch

    import w4_dequant_expert_amd as moe
    from synth import build_gdn_config

    c = build_gdn_config("gdn_prefill2048")
    sh = c["shape"]

    def dev(a):
        a = np.ascontiguousarray(a)
        return torch.from_numpy(a.view(np.int16) if a.dtype == np.uint16 else a).to("cuda")

    q, k, v, g, b = (dev(c[n]) for n in ("q", "k", "v", "g", "beta"))
    o = torch.empty((sh.T, sh.n_v_heads, sh.dv), dtype=torch.int16, device="cuda")
    s_out = torch.empty((sh.n_v_heads, sh.dv, sh.dk), dtype=torch.float32, device="cuda")
    d = moe.GdnDims(sh.T, sh.n_k_heads, sh.n_v_heads, sh.dk, sh.dv)
    ws_bytes = moe.gdn_scan_chunked_ws_bytes(d)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    stream = torch.cuda.current_stream()

    def timed(call):
        for _ in range(warmup):
            call()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            call()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps

    ms_direct = timed(lambda: moe.gdn_scan(d, q, k, v, g, b, None, s_out, o, stream))
    ms_chunk = timed(lambda: moe.gdn_scan_chunked(d, q, k, v, g, b, None, s_out, o, ws, ws_bytes,
                                                  stream))
    flops = 7.0 * sh.T * sh.n_v_heads * sh.dv * sh.dk
    ms = min(ms_direct, ms_chunk)
    tflops = flops / (ms * 1e-3) / 1e12
    return dict(tokens_per_s=sh.T / (ms * 1e-3), ms_per_scan=ms,
                method="chunked" if ms_chunk <= ms_direct else "direct",
                direct_ms=ms_direct, chunked_ms=ms_chunk, chunked_ws_bytes=ws_bytes,
                tokens=sh.T, key_heads=sh.n_k_heads, value_heads=sh.n_v_heads, head_dim=sh.dk,
                algorithmic_flops=flops, tflops=tflops,
                direct_tflops=flops / (ms_direct * 1e-3) / 1e12,
                chunked_tflops=flops / (ms_chunk * 1e-3) / 1e12,
                frac_fp32_vector=tflops / PEAK_FP32_TFLOPS,
                frac_fp32_vector_unpacked=tflops / PEAK_FP32_UNPACKED_TFLOPS,
                state_bytes_kept_on_chip=sh.n_v_heads * sh.dv * sh.dk * 4)


def small_batch_leg(Ts=(2, 4, 8), copies=40):
    """Batches of 2..8 tokens (speculative-verification sized): whole layer
    calls replayed from a HIP graph, a fresh batch and weight copy per call;
    distinct experts touched and the weight bytes they pull in."""
    import numpy as np
    import torch

    from synth import make_tokens
    out = {}
    for T in Ts:
        wl = Workload("decode1", copies, T=T)
        fresh = [torch.from_numpy(make_tokens(T, 2048, 4, t0=T * i).view(np.int16)).to("cuda")
                 for i in range(copies)]
        for i in range(3):
            wl.step(i, x=fresh[i], overlap=False)
        step_ms = graph_ms(lambda i: wl.step(i, x=fresh[i], overlap=False), copies)
        wl.step(0, x=fresh[0], overlap=False)
        wk = wl.work()
        gemm_bytes = wk["bytes_gate_up"] + wk["bytes_down"]
        out[f"T{T}"] = dict(tokens_per_s=T / (step_ms * 1e-3), ms_per_step=round(step_ms, 5),
                            touched_experts=wk["touched"], gemm_bytes=gemm_bytes,
                            layer_hbm_gbs=wk["bytes_layer"] / (step_ms * 1e-3) / 1e9)
        del wl, fresh
        torch.cuda.empty_cache()
    return out


def host_route_tables(topk_idx, E, k, n_shared, tile_m_max, tile_gran):
    """The routing steps after top-k (histogram, exclusive scan, stable scatter,
    block map) computed on the host with numpy, as an engine that brings the
    selections back to the CPU does: the host-synced side of the routing
    ablation.  Same rules as the device tables (checked against them)."""
    import numpy as np
    T = topk_idx.shape[0]
    flat = topk_idx.reshape(-1)
    counts = np.bincount(flat, minlength=E).astype(np.int32)
    offsets = np.zeros(E + 1, dtype=np.int32)
    np.cumsum(counts, out=offsets[1:])
    sorted_slot = np.argsort(flat, kind="stable").astype(np.int32)
    slot_pos = np.empty_like(sorted_slot)
    slot_pos[sorted_slot] = np.arange(T * k, dtype=np.int32)
    blocks = []
    for g, c, first in [(e, int(counts[e]), int(offsets[e])) for e in range(E)] + \
            ([(E, T, T * k)] if n_shared else []):
        if c == 0:
            continue
        nb = -(-c // tile_m_max)
        base, rem = divmod(c, nb)
        tm = -(-(base + (rem > 0)) // tile_gran) * tile_gran
        for i in range(nb):
            rows = base + (i < rem)
            blocks.append((g, first, rows, tm))
            first += rows
    return counts, offsets, sorted_slot, slot_pos, np.array(blocks, dtype=np.int32).reshape(-1, 4)


def ablation_leg(copies, steps=30):
    """The pages' two MoE ablations at 512 tokens, end to end, each against the
    library's own layer call (moe_route, moe_grouped_w4_ffn, moe_combine:
    routing on the GPU, reconstruction fused into the grouped GEMMs).
    - Host-synced routing: the selections (top-k) are copied to the host, the
      histogram, scan, scatter and block map are built there (numpy), copied
      back, and the same GEMM and combine kernels run on them.  (moe_route
      still builds its own tables on the GPU; the host ones replace them.)
    - Unfused reconstruction: every call expands the packed 4-bit weights of
      the 257 experts to bfloat16 in memory (moe_w4_dequant_packed, the same
      reconstruction as the tall GEMM), then runs batched bfloat16 GEMMs on
      them (torch.bmm over each expert's rows, padded to 32; the shared expert
      as plain GEMMs), SwiGLU and the weighted combine as tensor operations."""
    import numpy as np
    import torch

    import w4_dequant_expert_amd as moe
    wl = Workload("prefill512", copies)
    sh = wl.sh
    L = wl.layer
    T, E, k, H, I = wl.T, sh.E, sh.k, sh.H, sh.I
    rt = L.rt
    idx_host = torch.empty((T, k), dtype=torch.int32, pin_memory=True)
    tables_ok = []

    def host_synced(i):
        r, s_, wr = wl.copies[i % len(wl.copies)]
        L.w_router = wr
        d = L.route(wl.x)
        idx_host.copy_(rt.topk_idx, non_blocking=True)
        torch.cuda.current_stream().synchronize()
        counts, offsets, ss, sp, blocks = host_route_tables(idx_host.numpy(), E, k, sh.n_shared,
                                                            wl.tile_m_max, 16)
        if not tables_ok:  # the host tables are the device's, once checked
            tables_ok.append(np.array_equal(ss, rt.sorted_slot.cpu().numpy()) and
                             np.array_equal(blocks, rt.blocks[:len(blocks)].cpu().numpy()))
        rt.counts.copy_(torch.from_numpy(counts), non_blocking=True)
        rt.offsets.copy_(torch.from_numpy(offsets), non_blocking=True)
        rt.sorted_slot.copy_(torch.from_numpy(ss), non_blocking=True)
        rt.slot_pos.copy_(torch.from_numpy(sp), non_blocking=True)
        rt.blocks[:len(blocks)].copy_(torch.from_numpy(blocks), non_blocking=True)
        rt.n_blocks.fill_(len(blocks))
        L.ffn(d, wl.x, r, s_)
        L.combine(d, wl.y)

    # unfused: expanded bf16 weights, batched GEMMs over the rows in expert
    # order, each expert's rows padded to P (every expert has at most P rows at
    # 512 tokens); the shared expert as plain GEMMs over all tokens.  Every
    # batched product takes contiguous operands only.
    base_r, base_s = wl.copies[0][0], wl.copies[0][1]
    P = 32
    w_gu = torch.empty((E, 2 * I, H), dtype=torch.bfloat16, device="cuda")
    w_dn = torch.empty((E, H, I), dtype=torch.bfloat16, device="cuda")
    s_gu = torch.empty((1, 2 * I, H), dtype=torch.bfloat16, device="cuda")
    s_dn = torch.empty((1, H, I), dtype=torch.bfloat16, device="cuda")
    xb = wl.x.view(torch.bfloat16)
    F = torch.nn.functional

    def expand():
        moe.moe_w4_dequant_packed(E, 2 * I, H, True, base_r.t["gu"], w_gu)
        moe.moe_w4_dequant_packed(E, H, I, False, base_r.t["dn"], w_dn)
        moe.moe_w4_dequant_packed(1, 2 * I, H, True, base_s.t["gu"], s_gu)
        moe.moe_w4_dequant_packed(1, H, I, False, base_s.t["dn"], s_dn)

    def unfused_gemms():
        expert = torch.repeat_interleave(torch.arange(E, device="cuda"), rt.counts.long(),
                                         output_size=T * k)
        pos = torch.arange(T * k, device="cuda") - rt.offsets[:E].long()[expert]
        pad = expert * P + pos                                          # padded row of each slot row
        a = torch.zeros((E * P, H), dtype=torch.bfloat16, device="cuda")
        a[pad] = xb.index_select(0, rt.sorted_slot.long() // k)
        at = a.view(E, P, H).transpose(1, 2).contiguous()               # [E][H][P]
        gt = torch.bmm(w_gu, at)                                        # [E][2I][P]
        ht = (F.silu(gt[:, :I].float()) * gt[:, I:].float()).to(torch.bfloat16).contiguous()
        yt = torch.bmm(w_dn, ht)                                        # [E][H][P]
        ys = yt.transpose(1, 2).reshape(E * P, H)[pad]                  # rows in expert order
        g2 = F.linear(xb, s_gu[0])                                      # shared expert
        y_sh = F.linear((F.silu(g2[:, :I].float()) * g2[:, I:].float()).to(torch.bfloat16), s_dn[0])
        sel = ys.index_select(0, rt.slot_pos.long()).view(T, k, H).float()
        y = (sel * rt.topk_w.unsqueeze(-1)).sum(1) + y_sh.float()
        return y.to(torch.bfloat16)

    def unfused(i):
        L.route(wl.x)
        expand()
        return unfused_gemms()

    def timed(fn):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) / steps * 1e3
    # warm the clocks, then alternate the paths
    for i in range(100):
        wl.step(i)
    for i in range(10):
        host_synced(i)
    out = {}
    L.w_router = wl.copies[0][2]
    wl.step(0)  # the fused call on weight copy 0, then the unfused path on the same inputs
    torch.cuda.synchronize()
    assert int(rt.counts.max().item()) <= P
    yf = wl.y.view(torch.bfloat16).float()
    y_unf = unfused(0).float()
    out["unfused_vs_fused_max_rel"] = float(((y_unf - yf).abs().max(1).values /
                                             yf.abs().max(1).values).max())
    fused, syn, unf, exp_only = [], [], [], []
    for _ in range(3):
        fused.append(timed(wl.step))
        syn.append(timed(host_synced))
        unf.append(timed(unfused))
        exp_only.append(timed(lambda i: expand()))
    fused_ms, synced_ms = min(fused), min(syn)
    out.update(
        fused_layer_ms=round(fused_ms, 5),
        host_synced_routing_layer_ms=round(synced_ms, 5),
        gpu_resident_routing_speedup=synced_ms / fused_ms,
        host_tables_match_device=bool(tables_ok and tables_ok[0]),
        note="layer calls at 512 tokens, wall clock per call over 30 calls, best of 3 alternated "
             "passes")
    unf_ms, exp_ms = min(unf), min(exp_only)
    out.update(unfused_layer_ms=round(unf_ms, 5), unfused_expand_ms=round(exp_ms, 5),
               unfused_expanded_bytes=(w_gu.numel() + w_dn.numel() + s_gu.numel() + s_dn.numel()) * 2,
               fused_dequant_speedup=unf_ms / fused_ms)
    del wl, w_gu, w_dn, s_gu, s_dn
    torch.cuda.empty_cache()
    return out


def tile_sweep_leg(copies, steps=100, warmup=50):
    """The pages' tile-height ablation: whole layer calls at 512 and 2048
    (Zipf-skewed) tokens for each bound on the block map's tile height."""
    import torch
    out = {}
    for name in ("prefill512", "prefill2048_zipf"):
        for m in (16, 32, 64, 128):
            wl = Workload(name, copies, m)
            wall, _ = time_workload(wl, steps, warmup)
            out[f"{name}_M{m}"] = round(wl.T * steps / wall, 1)
            del wl
            torch.cuda.empty_cache()
    return out


def chunked_leg(copies, reps=3):
    """Long prompt: 16384 tokens as 8 independent layer calls of 2048 tokens
    (route, gate/up, down, combine each), timed per chunk with HIP events over
    `reps` passes; steady state is the median over chunks 2..8 of each chunk's
    fastest pass.  Temporary device memory per chunk is the layer's scratch
    (routing tables and workspace, h, y_slots), all allocated once up front;
    the allocator's peak during the timed passes is reported beside it."""
    import statistics

    import numpy as np
    import torch

    from synth import CONFIGS, make_tokens
    cfg = CONFIGS["chunked16384"]
    chunk, n = cfg["chunk"], cfg["T"] // cfg["chunk"]
    wl = Workload("chunked16384", copies, T=chunk)
    xs = [torch.from_numpy(make_tokens(chunk, wl.sh.H, cfg["x_seed"], t0=c * chunk).view(np.int16))
          .to("cuda") for c in range(n)]
    for c in range(n):                       # warm-up pass
        wl.step(c, x=xs[c])
    torch.cuda.synchronize()
    base = torch.cuda.memory_allocated()
    torch.cuda.reset_peak_memory_stats()
    ms = [[] for _ in range(n)]
    for r in range(reps):
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for c in range(n):
            evs[c][0].record()
            wl.step(n * (r + 1) + c, x=xs[c])
            evs[c][1].record()
        torch.cuda.synchronize()
        for c in range(n):
            ms[c].append(evs[c][0].elapsed_time(evs[c][1]))
    best = [min(v) for v in ms]
    steady = statistics.median(best[1:])
    L = wl.layer
    scratch = [t for t in vars(L.rt).values() if isinstance(t, torch.Tensor)] + [L.h, L.y_slots]
    temp = sum(t.numel() * t.element_size() for t in scratch)
    out = dict(tokens_per_s=chunk / (steady * 1e-3), chunk_tokens=chunk, chunks=n,
               chunk_ms=[round(v, 4) for v in best], steady_chunk_ms=round(steady, 4),
               temp_bytes_per_chunk=temp,
               alloc_peak_during_chunks=torch.cuda.max_memory_allocated() - base,
               weight_copies=copies)
    del wl, xs
    return out


def traffic_record():
    try:
        with open(TRAFFIC_FILE) as fh:
            rec = json.load(fh)
    except (OSError, ValueError):
        return None
    if rec.get("kernel_source_hash") != kernel_source_hash():
        return None       # the kernel changed since the counters were taken
    return rec.get("bytes_per_launch")


def _pmc_rows(d, counter):
    """Per-dispatch values of one counter from a rocprofv3 --pmc CSV directory."""
    import csv
    import glob
    out = []
    for f in glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True):
        for r in csv.DictReader(open(f)):
            if r["Counter_Name"] == counter:
                out.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    return out


def write_traffic(fetch_dir, write_dir, calib_bytes):
    """HBM bytes per launch of the dominant kernel, scaled by the same counters'
    reading for a plain device copy of calib_bytes (read once, written once)."""
    rec = {"kernel": DOMINANT, "kernel_source_hash": kernel_source_hash()}
    for key, d, counter in (("fetch", fetch_dir, "FETCH_SIZE"), ("write", write_dir, "WRITE_SIZE")):
        rows = _pmc_rows(d, counter)
        kern = [v for _, n, v in rows if DOMINANT in n]
        copy = [v for _, n, v in rows if "copyBuffer" in n or "copy" in n.lower()]
        kib = sorted(kern)[len(kern) // 2]           # median over launches, KiB
        calib_kib = max(copy)                        # the large calibration copy
        factor = (calib_bytes / 1024.0) / calib_kib
        rec[key + "_kib_raw"] = kib
        rec[key + "_calib_kib_raw"] = calib_kib
        rec[key + "_scale"] = factor
        rec[key + "_bytes"] = kib * 1024.0 * factor
    rec["bytes_per_launch"] = rec["fetch_bytes"] + rec["write_bytes"]
    with open(TRAFFIC_FILE, "w") as fh:
        json.dump(rec, fh, indent=1)
    return rec


def cpu_baseline(name, budget_tokens):
    """The oracle, untuned, on the host cores: route + layer for a sample of the batch."""
    import oracle
    from synth import build_config
    c = build_config(name, T=budget_tokens)
    sh = c["shape"]
    threads, host_cpus = cpu_share()
    t0 = time.perf_counter()
    r = oracle.route(c["x"], c["wr"], c["bias"], sh.k, sh.n_shared, 128, 16, nthreads=threads)
    oracle.moe_layer(c["x"], r["topk_idx"], r["topk_w"], c["routed"], c["shared"], nthreads=threads)
    dt = time.perf_counter() - t0
    return dict(value=budget_tokens / dt, unit="tokens/s", cores=threads, kind="oracle",
                host_logical_cpus=host_cpus,
                sample=f"first {budget_tokens} tokens of the {name} batch: router, top-k, tables and "
                       f"float64 layer output ({dt:.1f} s), one oracle thread per CPU this job may "
                       f"use ({threads} of the host's {host_cpus})")


def cpu_single_thread():
    """The oracle on one thread for the tiny 16-token layer and one decode
    token of the full-shape layer (its own seeded token), route + layer."""
    import oracle
    from synth import build_config
    out = {}
    for name, T in (("tiny16", None), ("decode1", 1)):
        c = build_config(name, T=T)
        sh = c["shape"]
        t0 = time.perf_counter()
        r = oracle.route(c["x"], c["wr"], c["bias"], sh.k, sh.n_shared, 128, 16, nthreads=1)
        oracle.moe_layer(c["x"], r["topk_idx"], r["topk_w"], c["routed"], c["shared"], nthreads=1)
        dt = time.perf_counter() - t0
        out[name] = dict(tokens_per_s=c["T"] / dt, tokens=c["T"], seconds=round(dt, 4), threads=1)
    return out


def gdn_cpu_baseline(tokens=256):
    """The scan's oracle (numpy float64, untuned) on a bounded sample: the first
    `tokens` tokens of the 2048-token sequence at all 32 value heads."""
    import oracle
    from synth import bf16_bits_to_f32, build_gdn_config
    c = build_gdn_config("gdn_prefill2048", T=tokens)
    f = [bf16_bits_to_f32(c[n]) for n in ("q", "k", "v")]
    threads, host_cpus = cpu_share()
    t0 = time.perf_counter()
    oracle.gated_delta_scan(*f, c["g"], c["beta"])
    dt = time.perf_counter() - t0
    return dict(value=tokens / dt, unit="tokens/s", cores=threads, kind="oracle",
                host_logical_cpus=host_cpus,
                sample=f"first {tokens} tokens of the 2048-token sequence, 32 value heads ({dt:.1f} s); "
                       "numpy's BLAS threads")


def cpu_share():
    """(CPUs this process may run on, the host's logical CPUs): the affinity mask,
    bounded by a cgroup CPU quota when one is set."""
    host = os.cpu_count() or 1
    try:
        n = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        n = host
    try:
        with open("/sys/fs/cgroup/cpu.max") as fh:
            quota, period = fh.read().split()[:2]
        if quota != "max":
            n = min(n, max(1, int(int(quota) / int(period))))
    except (OSError, ValueError):
        pass
    return max(1, n), host


def main():
    args = parse()
    if args.traffic_from:
        print(json.dumps(write_traffic(*args.traffic_from, calib_bytes=(args.calib_copy_mb or 256) << 20)))
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only: --gpus {args.gpus} is not supported "
              "(the layer shards by token with no exchange; see the design notes)", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch

    import w4_dequant_expert_amd  # noqa: F401  (fails loudly without the HIP library)

    if args.calib_copy_mb:
        n = args.calib_copy_mb * (1 << 20)
        a = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calib_copy_bytes": n}), file=sys.stderr)
        del a, b

    extra = {}
    main_name = args.only or "prefill512"
    if main_name == "decode1":  # profiling runs of the decode leg alone
        print(json.dumps({"decode1": decode_leg(40)}))
        return
    if main_name == "chunked16384":
        print(json.dumps({"chunked16384": chunked_leg(args.copies)}))
        return
    if main_name == "small_batches":
        print(json.dumps({"small_batches": small_batch_leg()}))
        return
    if main_name == "ablations":
        print(json.dumps({"ablations_prefill512": ablation_leg(args.copies)}))
        return
    if main_name == "gdn_prefill2048":
        print(json.dumps({"gdn_prefill2048": gdn_leg()}))
        return
    if main_name == "tile_sweep":  # tokens/s per tile-height bound (not in the default run)
        print(json.dumps({"tile_sweep": tile_sweep_leg(args.copies)}))
        return
    # The headline workload is built first (seconds of host work with the GPU
    # idle), then the other workloads run (when requested), then the headline:
    # its W warm-up and K timed calls follow GPU work directly, at the GPU's
    # working clocks.
    wl = Workload(main_name, args.copies, args.tile_m_max)
    sib = {}
    if not args.no_extra and args.only is None:
        extra["ablations_prefill512"] = ablation_leg(args.copies)
        torch.cuda.empty_cache()
        extra["small_batches"] = small_batch_leg()
        torch.cuda.empty_cache()
        extra["chunked16384"] = chunked_leg(args.copies)
        torch.cuda.empty_cache()
        dec = decode_leg(40)
        extra["decode1"] = dec
        sib["roofline_decode1"] = {
            "bound": "hbm", "kernels": "w4_gemv_kernel<4, true, true> + <1, false, false> (gate/up, down)",
            "achieved": dec["gemm_hbm_gbs"], "peak": PEAK_HBM_GBS, "unit": "GB/s",
            "frac": dec["gemm_frac_hbm"], "algorithmic_bytes": dec["gemm_bytes"],
            "avg_launch_ms": {"gate_up": dec["gate_up_ms"], "down": dec["down_ms"]},
            "stream_ceiling_gbs": dec["stream_ceiling"]["gbs"],
            "frac_of_stream_ceiling": dec["gemm_frac_of_stream_ceiling"]}
        torch.cuda.empty_cache()
        gd = gdn_leg()
        if not args.no_cpu:
            gd["cpu_baseline"] = gdn_cpu_baseline()
        extra["gdn_prefill2048"] = gd
        if gd["method"] == "chunked":
            # float32 matrix instructions; the same published 157.3 TFLOP/s
            sib["roofline_gdn_prefill2048"] = {
                "bound": "mfma", "kernels": "gdn_chunk_prep_kernel + gdn_chunk_scan_kernel (fp32 MFMA)",
                "achieved": gd["tflops"], "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s",
                "frac": gd["tflops"] / PEAK_FP32_TFLOPS,
                "algorithmic_flops": gd["algorithmic_flops"], "avg_ms": gd["ms_per_scan"],
                "token_by_token_kernel_ms": gd["direct_ms"]}
        else:
            sib["roofline_gdn_prefill2048"] = {
                "bound": "alu", "kernel": "gdn_scan_kernel", "achieved": gd["tflops"],
                "peak": PEAK_FP32_TFLOPS, "unit": "TFLOP/s", "frac": gd["frac_fp32_vector"],
                "peak_without_packed_fp32": PEAK_FP32_UNPACKED_TFLOPS,
                "frac_without_packed_fp32": gd["frac_fp32_vector_unpacked"],
                "algorithmic_flops": gd["algorithmic_flops"], "avg_launch_ms": gd["ms_per_scan"]}
        torch.cuda.empty_cache()
        # the 2048-token GEMM-heavy leg last, directly before the headline
        wl2 = Workload("prefill2048_zipf", args.copies, None)
        n2 = max(args.steps // 2, 50)
        w2, st2 = time_workload(wl2, n2, max(args.warmup // 2, 20), overlap=args.overlap)
        wk2 = wl2.work()
        g2 = (st2["gate_up_ms"] + st2["down_ms"]) * 1e-3
        tf2 = (wk2["flops_gate_up"] + wk2["flops_down"]) / g2 / 1e12
        extra["prefill2048_zipf"] = dict(
            tokens_per_s=wl2.T * n2 / w2, timing=TIMING_NOTE,
            sequential_ms_per_step=round(sum(st2.values()), 5),
            **{k: round(v, 5) for k, v in st2.items()},
            gemm_tflops=tf2, gemm_frac_mfma=tf2 / PEAK_BF16_TFLOPS,
            touched_experts=wk2["touched"], tile_m_max=wl2.tile_m_max)
        pc = mfma_ceiling()
        sib["roofline_prefill2048_zipf"] = {
            "bound": "mfma", "kernels": "w4_gemm_tall4_kernel<true> + <false> (gate/up, down)",
            "achieved": tf2, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": tf2 / PEAK_BF16_TFLOPS,
            "mfma_ceiling_tflops": pc["tflops"], "frac_of_mfma_ceiling": tf2 / pc["tflops"],
            "algorithmic_flops": wk2["flops_gate_up"] + wk2["flops_down"],
            "avg_launch_ms": {"gate_up": st2["gate_up_ms"], "down": st2["down_ms"]}}
        del wl2
        torch.cuda.empty_cache()

    ceil512 = None
    if not args.no_extra and args.only is None:
        # B' for the headline GEMM: a plain streaming read of its algorithmic
        # bytes, four buffers rotating (more than the Infinity Cache holds)
        wl.step(0)  # the routing of a call fixes the touched experts
        torch.cuda.synchronize()
        ceil512 = stream_ceiling(wl.work()["bytes_gate_up"], copies=4,
                                 workgroups=(1024, 2048, 4096, 8192), graph=False)
        torch.cuda.empty_cache()
    wall, stages = time_workload(wl, args.steps, args.warmup, overlap=args.overlap)
    work = wl.work()
    ms = wall / args.steps * 1e3
    tok_s = wl.T * args.steps / wall
    gu_s = stages["gate_up_ms"] * 1e-3
    dn_s = stages["down_ms"] * 1e-3
    achieved = work["bytes_gate_up"] / gu_s / 1e9
    gemm_tflops = (work["flops_gate_up"] + work["flops_down"]) / (gu_s + dn_s) / 1e12
    gemm_gbs = (work["bytes_gate_up"] + work["bytes_down"]) / (gu_s + dn_s) / 1e9
    warm = None
    if not args.no_extra and args.only is None:
        # the same calls with one weight copy reused (R = 1): the weights stay
        # partly in the 256 MB Infinity Cache; labelled warm, never the headline
        w_wall, _ = time_workload(wl, args.steps, args.warmup, fixed_copy=0, stages=False)
        warm = dict(tokens_per_s=wl.T * args.steps / w_wall, ms_per_step=w_wall / args.steps * 1e3,
                    weight_copies=1, note="warm: one weight copy reused by every call")
    extra[main_name] = dict(
        tokens_per_s=tok_s, ms_per_step=ms, timing=TIMING_NOTE, warm_r1=warm,
        sequential_ms_per_step=round(sum(stages.values()), 5),
        **{k: round(v, 5) for k, v in stages.items()},
        gemm_tflops=gemm_tflops, gemm_frac_mfma=gemm_tflops / PEAK_BF16_TFLOPS,
        gemm_hbm_gbs=gemm_gbs, gemm_frac_hbm=gemm_gbs / PEAK_HBM_GBS,
        layer_bytes=work["bytes_layer"], touched_experts=work["touched"],
        implementation_bytes={"h": work["bytes_h"], "y_slots": work["bytes_y_slots"]})
    del wl
    torch.cuda.empty_cache()

    out = {
        "metric": "MoE-layer tokens/s + %MFMA peak at T=512/2048; %HBM peak at T=1",
        "value": tok_s,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": main_name, "tokens": wl_T(main_name), "hidden": 2048,
                   "experts": 256, "top_k": 8, "shared_experts": 1, "expert_intermediate": 512,
                   "weights": "4-bit codes, bf16 scale+bias per 64", "weight_copies": args.copies,
                   "tile_m_max": args.tile_m_max or TILE_M_MAX[main_name]},
        "roofline": {"bound": "hbm", "kernel": DOMINANT,
                     "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                     "frac": achieved / PEAK_HBM_GBS, "traffic": traffic_record(),
                     "algorithmic_bytes": work["bytes_gate_up"],
                     "implementation_bytes": {"h_written": work["bytes_h"]},
                     "avg_launch_ms": stages["gate_up_ms"],
                     "stream_ceiling": ceil512,
                     "stream_ceiling_gbs": ceil512["gbs"] if ceil512 else None,
                     "frac_of_stream_ceiling": achieved / ceil512["gbs"] if ceil512 else None},
        **sib,
        "cpu_baseline": None,
        "extra": extra,
    }
    if not args.no_cpu and args.only is None:
        out["cpu_baseline"] = cpu_baseline("prefill512", 512)
        out["cpu_baseline"]["single_thread"] = cpu_single_thread()
    print(json.dumps(out))


def wl_T(name):
    from synth import CONFIGS
    return CONFIGS[name]["T"]


if __name__ == "__main__":
    main()
