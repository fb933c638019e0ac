#!/usr/bin/env python3
"""Benchmark of the ConvRot quantized linear on one MI355X.

One step = one ConvRot INT8 linear at the prefill workload (M=4096 tokens, K=5376, N=16128,
bf16 activations with outlier channels, prepared INT8 weights, fp32 bias, bf16 out):
rotate+quantize the activations, then the INT8 MFMA GEMM with the fused dequant epilogue.
Inputs and weights cycle through rings of distinct buffers (>= 1 GiB each), so every step
reads HBM rather than the last-level cache.  `value` is whole-step int8 TOP/s.

The same run also measures, each with its own timed loop:
  * decode (M=12) linears on the four Qwen3-VL-32B-like shapes: weight GB/s of the INT8 decode
    GEMV (x pre-quantized) and end to end (rotate+quantize + GEMV), replayed from HIP graphs
    so that host launch gaps are not counted (eager times are reported beside them), and the
    same for the W4A8 decode GEMV (INT4 group-scaled weights in the W4A8 block layout);
  * the W4A4 linear at M=4096, K=5376, N=10752 and the mixed profile with 20% W8A8 layers;
  * the 64-layer Qwen3-32B-shaped stack at M=2048 (all weights resident, 31 GB of INT8);
  * the CPU oracle on a bounded sample of the prefill workload (cpu_baseline).
Per-kernel durations come from HIP events recorded on the stream the kernels run on.

Counter runs (L2-miss traffic): `--only copy` runs a plain 256 MiB device copy for calibrating
FETCH_SIZE / WRITE_SIZE; `--pmc-summary` turns four rocprofv3 counter CSVs into
profiles/hbm_traffic.json, which this script reads back for the roofline's `traffic` (bytes the L2
requests from the memory side; the last-level cache serves part of them, so they bound the HBM
traffic from above); `--counter-table` prints per-kernel counter means from --pmc CSVs.
"""
from __future__ import annotations

import argparse
import csv
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s (published)
PEAK_FP6_TFLOPS = 10100.0    # MI355X dense FP6 MFMA, TFLOP/s (published)
RING_BYTES = 1 << 30
COPY_PROBE_BYTES = 256 << 20
TRAFFIC_JSON = os.path.join(ROOT, "profiles", "hbm_traffic.json")
# What `traffic` counts: the L2's requests to the memory side (FETCH_SIZE + WRITE_SIZE), calibrated
# on a plain copy.  The 256 MB last-level cache sits behind the L2 and serves part of them, so the
# figure bounds the kernel's HBM traffic from above rather than equalling it.
TRAFFIC_KIND = ("L2-miss bytes per launch (TCC FETCH_SIZE + WRITE_SIZE, scaled by a plain copy's counts); "
                "includes what the last-level cache serves: an upper bound on HBM bytes")
KERNEL_SOURCES = {"gemm_i8": "gemm_i8.hip", "rotate_quant": "rotate_quant.hip", "gemv_i8": "gemv_i8.hip",
                  "gemm_w4a4": "gemm_w4a4.hip"}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "w4a4", "stack", "split", "copy"], default="all",
                    help="restrict the measured workloads (profiling runs); 'copy' = the counter calibration copy")
    ap.add_argument("--stack-layers", type=int, default=64)
    ap.add_argument("--trace-table", metavar="KERNEL_TRACE_CSV",
                    help="print markdown tables of kernel durations (per kernel, and per kernel x launch "
                         "configuration) from a rocprofv3 --kernel-trace CSV and exit")
    ap.add_argument("--counter-table", nargs="+", metavar="CSV",
                    help="print a markdown table of per-dispatch mean counters per kernel from rocprofv3 --pmc "
                         "counter CSVs (one or more passes) and exit")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="write profiles/hbm_traffic.json from rocprofv3 --pmc counter CSVs and exit")
    return ap.parse_args()


def ring_count(bytes_each: int) -> int:
    return max(2, -(-RING_BYTES // max(bytes_each, 1)))


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int4_quantized_linear_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(key: str, current_hash: str):
    """L2-miss bytes per launch (FETCH_SIZE + WRITE_SIZE scaled by a plain copy's counts, an upper
    bound on HBM bytes) from the committed counter summary, if it was taken on the current kernel
    source; otherwise None."""
    try:
        d = json.load(open(TRAFFIC_JSON))["kernels"].get(key)
    except (OSError, ValueError, KeyError):
        return None
    if not d or d.get("source_hash") != current_hash:
        return None
    return d.get("bytes_per_launch")


# --------------------------------------------------------------------------------------------
# timing helpers


SETTLE_S = 0.3


def settle(fn, torch, seconds: float = SETTLE_S):
    """Repeat fn(i) untimed for `seconds` of wall time.  The host-side input generation before
    each section leaves the GPU idle for seconds, and its clocks need a few hundred milliseconds
    of load to reach their steady state (measured on the prefill step: 371 us per GEMM after
    5 warm-up steps, 317 us once settled)."""
    t0 = time.perf_counter()
    i = 0
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            fn(i)
            i += 1
        torch.cuda.synchronize()


def timed_loop(fn, steps: int, warmup: int, torch):
    """Settle, run fn(i) warmup times, then time exactly `steps` calls; returns (wall ms per
    step, [per-call event lists])."""
    settle(fn, torch)
    for i in range(warmup):
        fn(i)
    torch.cuda.synchronize()
    marks = []
    t0 = time.perf_counter()
    for i in range(steps):
        marks.append(fn(warmup + i))
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, marks


def graph_time_us(torch, launch, n_calls: int, reps: int) -> float:
    """Capture n_calls launches (launch(i) enqueues one on the current stream) into a HIP graph,
    replay it reps times, return microseconds per launch (median over replays)."""
    launch(0)                               # first call outside capture (device checks, lazy init)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            for i in range(n_calls):
                launch(i)
    torch.cuda.synchronize()
    per = []
    with torch.cuda.stream(s):
        settle(lambda i: g.replay(), torch)
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(s)
            g.replay()
            e1.record(s)
            e1.synchronize()
            per.append(e0.elapsed_time(e1) * 1e3 / n_calls)
    torch.cuda.synchronize()
    del g
    return statistics.median(per)


# --------------------------------------------------------------------------------------------
# workloads


def bench_prefill(cr, wl, torch, steps, warmup):
    M, K, N = wl.PREFILL["M"], wl.PREFILL["K"], wl.PREFILL["N"]
    dev = torch.device("cuda:0")
    log("prefill: generating inputs M=%d K=%d N=%d" % (M, K, N))
    x, w, b = wl.prefill_inputs()
    xd, wd, bd = x.to(dev), w.to(dev), b.to(dev)
    wq0, ws0 = cr.prepare_weight(wd, 256, 8)
    del wd
    nx = ring_count(M * K * 2)
    nw = ring_count(N * K)
    xs = [xd] + [xd.clone() for _ in range(nx - 1)]
    wqs = [wq0] + [wq0.clone() for _ in range(nw - 1)]
    xq = torch.empty((M, K), dtype=torch.int8, device=dev)
    xsc = torch.empty((M,), dtype=torch.float32, device=dev)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
    st = torch.cuda.current_stream(dev)
    log("prefill: rings of %d activations, %d weights" % (nx, nw))

    def step(i):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(3)]
        e[0].record(st)
        cr._call("convrot_quantize_act", xs[i % nx].data_ptr(), cr.CONVROT_DTYPE_BF16, M, K, 256, 8,
                 xq.data_ptr(), xsc.data_ptr(), st.cuda_stream)
        e[1].record(st)
        cr._call("convrot_linear", None, 0, xq.data_ptr(), xsc.data_ptr(), M, N, K, 256, wqs[i % nw].data_ptr(),
                 ws0.data_ptr(), bd.data_ptr(), y.data_ptr(), None, 0, st.cuda_stream)
        e[2].record(st)
        return e

    wall, marks = timed_loop(step, steps, warmup, torch)

    # rotate+quantize alone, replayed from a HIP graph of 20 launches over the activation ring: the
    # in-step event pair above also spans the dispatch of the kernel right after the previous GEMM
    def rq_launch(i):
        cr._call("convrot_quantize_act", xs[i % nx].data_ptr(), cr.CONVROT_DTYPE_BF16, M, K, 256, 8,
                 xq.data_ptr(), xsc.data_ptr(), torch.cuda.current_stream(dev).cuda_stream)

    t_rq_graph_us = graph_time_us(torch, rq_launch, 20, 20)
    t_rq = sum(m[0].elapsed_time(m[1]) for m in marks) / steps
    t_gemm = sum(m[1].elapsed_time(m[2]) for m in marks) / steps
    t_step = sum(m[0].elapsed_time(m[2]) for m in marks) / steps
    ops = 2.0 * M * N * K
    rq_bytes = M * K * 2 + M * K + 4 * M
    gemm_bytes = M * K + N * K + 4 * M + 4 * N + 4 * N + 2 * M * N
    return dict(M=M, K=K, N=N, ops=ops, wall_ms=wall, step_ms=t_step, rq_ms=t_rq, gemm_ms=t_gemm,
                rq_graph_us=t_rq_graph_us, rq_bytes=rq_bytes, gemm_bytes=gemm_bytes)


def bench_decode(cr, wl, torch, steps, warmup):
    dev = torch.device("cuda:0")
    out = {}
    for (K, N) in wl.DECODE_SHAPES:
        M = wl.DECODE_M
        x, w = wl.decode_inputs(K, N)
        xd = x.to(dev)
        wq0, ws0 = cr.prepare_weight(w.to(dev), 256, 8)
        nw = ring_count(N * K)
        wqs = [wq0] + [wq0.clone() for _ in range(nw - 1)]
        xq, xsc = cr.quantize_act(xd, 256, 8)
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsz = cr.workspace_bytes(M, N, K, 8)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)

        def gemv(i):
            cr._call("convrot_linear", None, 0, xq.data_ptr(), xsc.data_ptr(), M, N, K, 256,
                     wqs[i % nw].data_ptr(), ws0.data_ptr(), None, y.data_ptr(), ws.data_ptr(), wsz,
                     torch.cuda.current_stream(dev).cuda_stream)

        def e2e(i):
            cr._call("convrot_linear", xd.data_ptr(), cr.CONVROT_DTYPE_BF16, None, None, M, N, K, 256,
                     wqs[i % nw].data_ptr(), ws0.data_ptr(), None, y.data_ptr(), ws.data_ptr(), wsz,
                     torch.cuda.current_stream(dev).cuda_stream)

        def eager(fn):
            st = torch.cuda.current_stream(dev)

            def one(i):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(st)
                fn(i)
                e[1].record(st)
                return e
            _, m = timed_loop(one, steps, warmup, torch)
            return sum(a.elapsed_time(b) for a, b in m) / steps * 1e3

        n_calls = max(nw, 20)
        tg = graph_time_us(torch, gemv, n_calls, max(steps, 5))
        te = graph_time_us(torch, e2e, n_calls, max(steps, 5))
        tg_eager, te_eager = eager(gemv), eager(e2e)
        wbytes = N * K + 4 * N
        gbs = wbytes / (tg * 1e-6) / 1e9
        row = dict(weight_bytes=wbytes, gemv_us=tg, e2e_us=te, weight_GBps=gbs,
                   frac_hbm=gbs / PEAK_HBM_GBS, gemv_eager_us=tg_eager, e2e_eager_us=te_eager,
                   splits=None, timing="hip graph replay of %d launches" % n_calls)
        log("decode K=%d N=%d: GEMV %.2f us (%.0f GB/s, %.0f%% of HBM), e2e %.2f us; eager %.2f / %.2f us" % (
            K, N, tg, gbs, 100 * gbs / PEAK_HBM_GBS, te, tg_eager, te_eager))
        del wqs, wq0
        torch.cuda.empty_cache()

        # W4A8: the same tokens (INT8) against INT4 group-scaled weights in the W4A8 block layout
        wq40, ws40 = cr.prepare_weight(w.to(dev), 256, 4)
        wp40 = cr.pack_weight_w4a8(wq40, ws40)
        del wq40, ws40
        wb4 = N * K // 2 + 2 * N * (K // 256)
        nw4 = ring_count(wb4)
        w4s = [wp40] + [wp40.clone() for _ in range(nw4 - 1)]
        wsz4 = cr.workspace_bytes_w4a8(M, N, K)
        ws4 = torch.empty(max(wsz4, 256), dtype=torch.uint8, device=dev)

        def gemv4(i):
            cr._call("convrot_linear_w4a8", None, 0, xq.data_ptr(), xsc.data_ptr(), M, N, K, 256,
                     w4s[i % nw4].data_ptr(), wp40.numel(), None, y.data_ptr(), None, 0,
                     torch.cuda.current_stream(dev).cuda_stream)

        def e2e4(i):
            cr._call("convrot_linear_w4a8", xd.data_ptr(), cr.CONVROT_DTYPE_BF16, None, None, M, N, K, 256,
                     w4s[i % nw4].data_ptr(), wp40.numel(), None, y.data_ptr(), ws4.data_ptr(), wsz4,
                     torch.cuda.current_stream(dev).cuda_stream)

        n4 = max(nw4, 20)
        t4 = graph_time_us(torch, gemv4, n4, max(steps, 5))
        t4e = graph_time_us(torch, e2e4, n4, max(steps, 5))
        gbs4 = wb4 / (t4 * 1e-6) / 1e9
        row.update(w4a8_weight_bytes=wb4, w4a8_gemv_us=t4, w4a8_e2e_us=t4e, w4a8_weight_GBps=gbs4,
                   w4a8_frac_hbm=gbs4 / PEAK_HBM_GBS, w4a8_speedup_vs_w8a8=tg / t4)
        log("decode K=%d N=%d: W4A8 GEMV %.2f us (%.0f GB/s, %.0f%% of HBM), e2e %.2f us, %.2fx the INT8 GEMV" % (
            K, N, t4, gbs4, 100 * gbs4 / PEAK_HBM_GBS, t4e, tg / t4))
        out["K%d_N%d" % (K, N)] = row
        del w4s, wp40
        torch.cuda.empty_cache()
    return out


def bench_w4a4(cr, wl, torch, steps, warmup):
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    M, K, N = wl.W4A4_SHAPE["M"], wl.W4A4_SHAPE["K"], wl.W4A4_SHAPE["N"]
    x, w, b = wl.prefill_inputs(M, K, N, cfg=wl.CFG_W4A4)
    xd, wd, bd = x.to(dev), w.to(dev), b.to(dev)
    wq4, ws4 = cr.prepare_weight(wd, 256, 4)
    wq8, ws8 = cr.prepare_weight(wd, 256, 8)
    del wd
    xq4, xs4 = cr.quantize_act(xd, 256, 4)
    y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)

    def timed(fn):
        def one(i):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(st)
            fn()
            e[1].record(st)
            return e
        _, m = timed_loop(one, steps, warmup, torch)
        return sum(a.elapsed_time(b) for a, b in m) / steps

    wp4 = cr.pack_weight_w4a4(wq4)
    tc = timed(lambda: cr.linear_w4a4(None, wq4, ws4, bd, xq=xq4, x_scale=xs4, out=y))
    t4 = timed(lambda: cr.linear_w4a4(xd, wq4, ws4, bd, out=y))
    tpc = timed(lambda: cr.linear_w4a4_packed(None, wp4, ws4, bd, xq=xq4, x_scale=xs4, out=y))
    tp4 = timed(lambda: cr.linear_w4a4_packed(xd, wp4, ws4, bd, out=y))
    t8 = timed(lambda: cr.linear(xd, wq8, ws8, bd, out=y))
    ops = 2.0 * M * N * K
    del wq4, wq8, ws8, wp4, xq4, xs4
    torch.cuda.empty_cache()
    mixed = bench_mixed(cr, wl, torch, M, K, N, bd)
    # cross-check: the same counts of separately timed single-shape linears (serving keeps the
    # W4A4 weights pre-encoded, so the packed path)
    promoted = mixed["w8a8_layers"]
    mixed["sum_of_single_linears_ms"] = (mixed["layers"] - promoted) * tp4 + promoted * t8
    return dict(M=M, K=K, N=N, gemm_us=tc * 1e3, gemm_tops=ops / (tc * 1e-3) / 1e12,
                gemm_frac_int8_peak=ops / (tc * 1e-3) / 1e12 / PEAK_INT8_TOPS,
                gemm_frac_fp6_peak=ops / (tc * 1e-3) / 1e12 / PEAK_FP6_TFLOPS,
                e2e_us=t4 * 1e3, e2e_tops=ops / (t4 * 1e-3) / 1e12,
                packed_gemm_us=tpc * 1e3, packed_e2e_us=tp4 * 1e3, packed_e2e_tops=ops / (tp4 * 1e-3) / 1e12,
                w8a8_e2e_us=t8 * 1e3, mixed_profile=mixed)


def bench_mixed(cr, wl, torch, M, K, N, bias, passes: int = 3):
    """The mixed profile as one timed schedule: MIXED_COUNT linears of the W4A4 shape in instance
    order, the seeded MIXED_PROMOTED of them W8A8 and the rest W4A4 on pre-encoded weights, every
    instance with its own resident weight (drawn on the device), each a full linear from bf16
    activations (a ring of 8 inputs).  Pass 0 warms up; the median of the timed passes is
    reported."""
    from int4_quantized_linear_amd.mixed import MixedSchedule
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    count = wl.MIXED_COUNT
    promoted = wl.mixed_profile_layers(count, wl.MIXED_PROMOTED)
    t0 = time.perf_counter()
    sched = MixedSchedule(M, K, N, count, promoted, lambda i: wl.mixed_weight(i, N, K, dev), bias=bias)
    torch.cuda.synchronize()
    log("mixed: %d instances (%d W8A8) prepared in %.1f s, %.1f GB of weights resident" % (
        count, len(promoted), time.perf_counter() - t0, sched.weight_bytes() / 1e9))
    xs = [wl.mixed_acts(j, M, K, dev) for j in range(8)]
    ys = [torch.empty((M, N), dtype=torch.bfloat16, device=dev) for _ in range(2)]
    per = []
    for rep in range(passes):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(st)
        sched.run(xs, ys)
        e1.record(st)
        e1.synchronize()
        if rep:
            per.append(e0.elapsed_time(e1))
    total = statistics.median(per)
    ops = 2.0 * M * N * K
    log("mixed: %d linears in %.2f ms (%.0f TOP/s)" % (count, total, count * ops / (total * 1e-3) / 1e12))
    del sched, xs, ys
    torch.cuda.empty_cache()
    return dict(layers=count, w8a8_layers=int(len(promoted)), total_ms=total,
                effective_tops=count * ops / (total * 1e-3) / 1e12,
                timing="one timed run of the whole schedule (median of %d passes after a warm-up pass)" % (passes - 1))


def bench_stack(cr, wl, torch, layers: int):
    """All layers' INT8 weights resident; per layer: 4 rotate+quantize of the layer's inputs and
    the 7 linears on the pre-quantized inputs (q/k/v share one, gate/up share one).  Also timed:
    the same layer with the linears that share an input run as one GEMM over their concatenated
    weight rows (q|k|v, gate|up).  Row-wise scales make the concatenation's preparation exactly the
    concatenation of the separate ones, so both schedules compute the same outputs; the 7-linear
    schedule runs on row slices of the concatenated weights."""
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    M = wl.STACK_M
    log("stack: preparing %d layers of weights and inputs on the device" % layers)
    t0 = time.perf_counter()
    kdim = dict(wl.STACK_INPUTS)
    # fused groups in matrix order: the matrices of a group share their input
    groups = []
    for i, (name, K, N) in enumerate(wl.STACK_MATRICES):
        inp = wl.STACK_INPUT_OF[name]
        if groups and groups[-1][0] == inp:
            groups[-1][1].append((i, name, N))
        else:
            groups.append((inp, [(i, name, N)]))
    W, X = [], []
    for L in range(layers):
        fused = []
        for inp, members in groups:
            K = kdim[inp]
            NT = sum(N for _, _, N in members)
            wq = torch.empty((NT, K), dtype=torch.int8, device=dev)
            sw = torch.empty((NT,), dtype=torch.float32, device=dev)
            n0 = 0
            for i, name, N in members:
                cr._call("convrot_prepare_weight", wl.stack_weight(L, i, N, K, dev).data_ptr(), cr.CONVROT_DTYPE_BF16,
                         N, K, 256, 8, wq[n0:n0 + N].data_ptr(), sw[n0:n0 + N].data_ptr(), st.cuda_stream)
                torch.cuda.synchronize()
                n0 += N
            fused.append((inp, K, NT, wq, sw, members))
        W.append(fused)
        X.append({inp: wl.stack_acts(L, j, M, K, dev) for j, (inp, K) in enumerate(wl.STACK_INPUTS)})
    torch.cuda.synchronize()
    log("stack: prepared in %.1f s (%.1f GB of INT8 weights)" % (
        time.perf_counter() - t0, sum(f[3].numel() for g in W for f in g) / 1e9))
    xq = {inp: torch.empty((M, K), dtype=torch.int8, device=dev) for inp, K in wl.STACK_INPUTS}
    xs = {inp: torch.empty((M,), dtype=torch.float32, device=dev) for inp, _ in wl.STACK_INPUTS}
    ys = {inp: torch.empty((M, sum(N for _, _, N in members)), dtype=torch.bfloat16, device=dev)
          for inp, members in groups}
    # one workspace for every GEMM of the layer (stream order serialises them): room for the
    # split-K tail of the GEMMs whose tiles leave the grid's last round partly idle
    shapes = [(K, N) for _, K, N in wl.STACK_MATRICES] + [(f[1], f[2]) for f in W[0]]
    wsz = max(cr.workspace_bytes(M, N, K, 8) for K, N in shapes)
    wsb = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)

    def layer(L, fuse):
        for inp, K in wl.STACK_INPUTS:
            cr._call("convrot_quantize_act", X[L][inp].data_ptr(), cr.CONVROT_DTYPE_BF16, M, K, 256, 8,
                     xq[inp].data_ptr(), xs[inp].data_ptr(), st.cuda_stream)
        for inp, K, NT, wq, sw, members in W[L]:
            y = ys[inp]
            if fuse:
                cr._call("convrot_linear", None, 0, xq[inp].data_ptr(), xs[inp].data_ptr(), M, NT, K, 256,
                         wq.data_ptr(), sw.data_ptr(), None, y.data_ptr(), wsb.data_ptr(), wsz, st.cuda_stream)
                continue
            n0 = 0
            for _, name, N in members:
                # the separate linear writes its own [M, N] output (a contiguous block of y)
                cr._call("convrot_linear", None, 0, xq[inp].data_ptr(), xs[inp].data_ptr(), M, N, K, 256,
                         wq[n0:n0 + N].data_ptr(), sw[n0:n0 + N].data_ptr(), None, y.view(-1)[M * n0:].data_ptr(),
                         wsb.data_ptr(), wsz, st.cuda_stream)
                n0 += N

    def timed(fuse):
        per_pass = []
        settle(lambda i: layer(i % layers, fuse), torch)
        for rep in range(3):                      # pass 0 warms up
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(layers + 1)]
            ev[0].record(st)
            for L in range(layers):
                layer(L, fuse)
                ev[L + 1].record(st)
            torch.cuda.synchronize()
            if rep:
                per_pass.append([ev[i].elapsed_time(ev[i + 1]) for i in range(layers)])
        per_layer = [t for p in per_pass for t in p]
        return statistics.median(per_layer), statistics.median([sum(p) for p in per_pass])

    ops = sum(2.0 * M * N * K for _, K, N in wl.STACK_MATRICES)
    med, total = timed(False)
    fmed, ftotal = timed(True)
    res = dict(layers=layers, M=M, ops_per_layer=ops, median_layer_us=med * 1e3,
               median_layer_tops=ops / (med * 1e-3) / 1e12, total_ms=total,
               frac_int8_peak=ops / (med * 1e-3) / 1e12 / PEAK_INT8_TOPS,
               fused_median_layer_us=fmed * 1e3, fused_median_layer_tops=ops / (fmed * 1e-3) / 1e12,
               fused_total_ms=ftotal, fused_groups=[[name for _, name, _ in m] for _, m in groups])
    del W, X
    torch.cuda.empty_cache()
    return res


SPLIT_SHAPES = [(64, 8192, 5120), (128, 8192, 5120), (32, 25600, 5120), (2048, 1024, 5120)]


def bench_split(cr, torch, steps, warmup):
    """GEMMs whose 256 x 256 tiles leave the persistent grid badly under-filled (mid-size M, the
    layer stack's k/v projection): the pre-quantized INT8 linear without a workspace (whole tiles
    only) and with one (the tail tiles split in K, a second kernel summing the int32 partials).
    Random codes and scales; outputs must be bit-identical."""
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
    g = torch.Generator(device=dev)
    g.manual_seed(7)
    out = {}
    for M, N, K in SPLIT_SHAPES:
        xq = torch.randint(-127, 128, (M, K), dtype=torch.int8, device=dev, generator=g)
        wq = torch.randint(-127, 128, (N, K), dtype=torch.int8, device=dev, generator=g)
        sx = torch.rand(M, device=dev, generator=g) * 0.01
        sw = torch.rand(N, device=dev, generator=g) * 0.01
        y = torch.empty((M, N), dtype=torch.bfloat16, device=dev)
        wsz = cr.workspace_bytes(M, N, K, 8)
        ws = torch.empty(max(wsz, 256), dtype=torch.uint8, device=dev)

        def run(split):
            def one(i):
                e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
                e[0].record(st)
                cr._call("convrot_linear", None, 0, xq.data_ptr(), sx.data_ptr(), M, N, K, 256, wq.data_ptr(),
                         sw.data_ptr(), None, y.data_ptr(), ws.data_ptr() if split else None, wsz if split else 0,
                         st.cuda_stream)
                e[1].record(st)
                return e
            _, m = timed_loop(one, steps, warmup, torch)
            return sum(a.elapsed_time(b) for a, b in m) / steps * 1e3

        t_whole = run(False)
        y_whole = y.clone()
        t_split = run(True)
        torch.cuda.synchronize()
        out["M%d_N%d_K%d" % (M, N, K)] = dict(whole_us=t_whole, split_us=t_split, speedup=t_whole / t_split,
                                              split_tops=2.0 * M * N * K / (t_split * 1e-6) / 1e12,
                                              identical=bool(torch.equal(y, y_whole)))
        log("split-K tail M=%d N=%d K=%d: whole %.1f us, split %.1f us (%.2fx), identical=%s" % (
            M, N, K, t_whole, t_split, t_whole / t_split, out["M%d_N%d_K%d" % (M, N, K)]["identical"]))
        del xq, wq, ws
    return out


def copy_probe(torch):
    """Plain device copy of COPY_PROBE_BYTES (5 launches): the calibration kernel for counters."""
    dev = torch.device("cuda:0")
    n = COPY_PROBE_BYTES // 4
    src = torch.ones(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    for _ in range(5):
        dst.copy_(src)
    torch.cuda.synchronize()
    log("copy probe: 5 copies of %d bytes" % COPY_PROBE_BYTES)


def cpu_baseline(wl, torch):
    """The oracle as it stands on a bounded sample of the prefill workload: all S = 4096 tokens
    against the first R = 8192 of the 16128 output channels (half the work); weights prepared
    untimed as on the GPU; timed = rotate+quantize the tokens, integer GEMM, dequant."""
    import numpy as np

    from oracle import oracle as orc
    S, R = 4096, 8192
    x, w, b = wl.prefill_inputs()
    xs = x[:S].double().numpy()
    wr = w[:R].double().numpy()
    log("cpu baseline: preparing %d weight rows with the oracle (untimed)" % R)
    qw, sw = orc.prepare_weight_i8(wr, 256)
    t0 = time.perf_counter()
    qx, sx = orc.quantize_act_i8(xs, 256)
    acc = orc.gemm_i32(qx, qw)
    y = orc.dequant(acc, sx, sw, b[:R].numpy())
    dt = time.perf_counter() - t0
    assert np.isfinite(y).all()
    K = xs.shape[1]
    ops = 2.0 * S * R * K
    return dict(value=ops / dt / 1e12, unit="TOP/s", cores=orc.num_threads(), kind="oracle",
                sample="%d tokens x %d of 16128 output channels of the 4096x5376x16128 prefill linear "
                       "(rotate+quantize tokens, int64-checked integer GEMM, fp64 dequant; weights prepared "
                       "untimed): %.3g ops in %.1f s" % (S, R, ops, dt))


# --------------------------------------------------------------------------------------------
# counter summary


def _counter_rows(path):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            rows.append((r["Kernel_Name"], r["Counter_Name"], float(r["Counter_Value"])))
    return rows


def _kernel_key(name: str):
    if "gemm_i8_kernel" in name:
        return "gemm_i8"
    if "rotate_quant_kernel" in name:
        return "rotate_quant"
    if "gemv_i8_kernel" in name:
        return "gemv_i8"
    if "gemm_w4a4" in name:
        return "gemm_w4a4"
    if "copyBuffer" in name:
        return "copy"
    return None


def _per_dispatch_kib(path, counter):
    acc = {}
    for name, cname, v in _counter_rows(path):
        k = _kernel_key(name)
        if k and cname == counter:
            acc.setdefault(k, []).append(v)
    return {k: statistics.median(v) for k, v in acc.items()}


PMC_COMMANDS = [
    "cd /tmp && export TMPDIR=/tmp && cd <repo>",
    "rocprofv3 --pmc FETCH_SIZE -d /tmp/pmc_fetch -o run --output-format csv -- "
    "python3 bench.py --only prefill --steps 3 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc WRITE_SIZE -d /tmp/pmc_write -o run --output-format csv -- "
    "python3 bench.py --only prefill --steps 3 --warmup 1 --no-cpu-baseline",
    "rocprofv3 --pmc FETCH_SIZE -d /tmp/pmc_cfetch -o run --output-format csv -- python3 bench.py --only copy",
    "rocprofv3 --pmc WRITE_SIZE -d /tmp/pmc_cwrite -o run --output-format csv -- python3 bench.py --only copy",
    "python3 bench.py --pmc-summary <the four run_counter_collection.csv files, in the order above>",
]


def _kernel_label(name: str) -> str:
    n = name
    for pre in ("void ", "(anonymous namespace)::", "convrot::"):
        n = n.replace(pre, "")
    # keep the template arguments, drop the parameter list
    depth, cut = 0, len(n)
    for i, ch in enumerate(n):
        depth += ch == "<"
        depth -= ch == ">"
        if ch == "(" and depth == 0 and i > 0:
            cut = i
            break
    return n[:cut]


COUNTER_KERNELS = ("gemm_i8_kernel", "gemm_w4a4_kernel", "rotate_quant_kernel", "rotate_quant_fp6_kernel",
                   "tile_fp6_kernel", "gemv_i8_kernel", "gemv_w4a8_kernel", "split_reduce_kernel")


def counter_table(paths):
    """Per-dispatch means of every counter in the given rocprofv3 --pmc CSVs, per library kernel,
    as a markdown table (counters as rows).  Derived rows, per dispatch: MFMA-busy fraction =
    SQ_VALU_MFMA_BUSY_CYCLES / (1024 SIMDs x GRBM_GUI_ACTIVE / 8 XCDs); L2 hit rate =
    TCC_HIT / (TCC_HIT + TCC_MISS); mean L2 read latency seen by the L1 = TCP_TCC_READ_REQ_LATENCY /
    TCP_TCC_READ_REQ (cycles)."""
    acc, by_cfg = {}, {}
    for path in paths:
        with open(path) as f:
            for r in csv.DictReader(f):
                name = r["Kernel_Name"]
                if not any(k in name for k in COUNTER_KERNELS):
                    continue
                v = float(r["Counter_Value"])
                acc.setdefault(_kernel_label(name), {}).setdefault(r["Counter_Name"], []).append(v)
                try:
                    cfg = (_kernel_label(name), int(_col(r, "Grid_Size", "Grid_Size_X")),
                           int(_col(r, "Workgroup_Size", "Workgroup_Size_X")))
                except (KeyError, ValueError):
                    continue
                by_cfg.setdefault(cfg, {}).setdefault(r["Counter_Name"], []).append(v)
    kernels = sorted(acc)
    counters = sorted({c for k in kernels for c in acc[k]})
    mean = {k: {c: statistics.fmean(v) for c, v in acc[k].items()} for k in kernels}
    print("| counter | " + " | ".join("`%s`" % k for k in kernels) + " |")
    print("|---|" + "---|" * len(kernels))
    print("| dispatches | " + " | ".join("%d" % max(len(v) for v in acc[k].values()) for k in kernels) + " |")
    for c in counters:
        print("| %s | " % c + " | ".join("%.4g" % mean[k][c] if c in mean[k] else "" for k in kernels) + " |")

    def derived(label, fn):
        vals = []
        for k in kernels:
            try:
                vals.append(fn(mean[k]))
            except (KeyError, ZeroDivisionError):
                vals.append("")
        if any(v != "" for v in vals):
            print("| *%s* | " % label + " | ".join(v if isinstance(v, str) else "%.3g" % v for v in vals) + " |")

    derived("MFMA-busy fraction", lambda m: m["SQ_VALU_MFMA_BUSY_CYCLES"] / (1024 * m["GRBM_GUI_ACTIVE"] / 8))
    derived("L2 hit rate", lambda m: m["TCC_HIT_sum"] / (m["TCC_HIT_sum"] + m["TCC_MISS_sum"]))
    derived("mean L2 read latency (cycles)", lambda m: m["TCP_TCC_READ_REQ_LATENCY_sum"] / m["TCP_TCC_READ_REQ_sum"])
    if len(by_cfg) > len(kernels):
        # the same kernel at several launch shapes: one row per kernel x grid x workgroup size
        cnames = sorted({c for d in by_cfg.values() for c in d})
        print()
        print("| kernel | grid threads | workgroup threads | dispatches | " + " | ".join(cnames) + " |")
        print("|---|---|---|---|" + "---|" * len(cnames))
        for (k, grid, wg), d in sorted(by_cfg.items()):
            print("| `%s` | %d | %d | %d | " % (k, grid, wg, max(len(v) for v in d.values())) +
                  " | ".join("%.4g" % statistics.median(d[c]) if c in d else "" for c in cnames) + " |")


def _col(row, *names):
    for n in names:
        if n in row and row[n] != "":
            return row[n]
    raise KeyError(names[0])


def trace_table(path):
    """Kernel durations from a rocprofv3 kernel-trace CSV: calls, mean, median, min and max per
    kernel (all of them, longest total first), then per kernel x grid x workgroup size for this
    library's kernels."""
    per, per_cfg = {}, {}
    with open(path) as f:
        for r in csv.DictReader(f):
            name = _kernel_label(r["Kernel_Name"])
            us = (int(_col(r, "End_Timestamp")) - int(_col(r, "Start_Timestamp"))) * 1e-3
            per.setdefault(name, []).append(us)
            if any(k in r["Kernel_Name"] for k in COUNTER_KERNELS):
                grid = int(_col(r, "Grid_Size", "Grid_Size_X"))
                wg = int(_col(r, "Workgroup_Size", "Workgroup_Size_X"))
                per_cfg.setdefault((name, grid, wg), []).append(us)
    print("| kernel | calls | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|")
    for name, v in sorted(per.items(), key=lambda kv: -sum(kv[1])):
        print("| `%s` | %d | %.2f | %.2f | %.2f | %.2f |" % (name, len(v), statistics.fmean(v), statistics.median(v),
                                                             min(v), max(v)))
    print()
    print("| kernel | grid threads | workgroup threads | calls | mean us | median us | min us | max us |")
    print("|---|---|---|---|---|---|---|---|")
    for (name, grid, wg), v in sorted(per_cfg.items(), key=lambda kv: (kv[0][0], -len(kv[1]))):
        print("| `%s` | %d | %d | %d | %.2f | %.2f | %.2f | %.2f |" % (
            name, grid, wg, len(v), statistics.fmean(v), statistics.median(v), min(v), max(v)))


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    f = _per_dispatch_kib(fetch_csv, "FETCH_SIZE")
    w = _per_dispatch_kib(write_csv, "WRITE_SIZE")
    cf = _per_dispatch_kib(copy_fetch_csv, "FETCH_SIZE")["copy"]
    cw = _per_dispatch_kib(copy_write_csv, "WRITE_SIZE")["copy"]
    kib = COPY_PROBE_BYTES / 1024.0
    ff, fw = kib / cf, kib / cw
    out = {"commands": PMC_COMMANDS,
           "calibration": {"kernel": "device copy (__amd_rocclr_copyBuffer) of %d bytes" % COPY_PROBE_BYTES,
                           "fetch_kib_per_dispatch": cf, "write_kib_per_dispatch": cw,
                           "fetch_factor": ff, "write_factor": fw},
           "kernels": {}}
    for k in sorted(set(f) & set(w)):
        if k == "copy":
            continue
        fb, wb = f[k] * 1024 * ff, w[k] * 1024 * fw
        out["kernels"][k + "_prefill" if k in ("gemm_i8", "rotate_quant") else k] = {
            "source_hash": src_hash(KERNEL_SOURCES[k]), "fetch_bytes": fb, "write_bytes": wb,
            "bytes_per_launch": fb + wb, "fetch_kib_raw": f[k], "write_kib_raw": w[k]}
    os.makedirs(os.path.dirname(TRAFFIC_JSON), exist_ok=True)
    with open(TRAFFIC_JSON, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out, indent=1))


# --------------------------------------------------------------------------------------------


def main():
    args = parse()
    if args.pmc_summary:
        pmc_summary(*args.pmc_summary)
        return
    if args.counter_table:
        counter_table(args.counter_table)
        return
    if args.trace_table:
        trace_table(args.trace_table)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this library has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from int4_quantized_linear_amd import convrot as cr
    from int4_quantized_linear_amd import workloads as wl
    cr.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    if args.only == "copy":
        copy_probe(torch)
        return
    res = {}
    if args.only in ("all", "prefill"):
        res["prefill"] = bench_prefill(cr, wl, torch, args.steps, args.warmup)
        p = res["prefill"]
        log("prefill: step %.1f us (rotate+quant %.1f us in the step, %.1f us per graph-replayed launch; GEMM "
            "%.1f us), wall %.1f us" % (p["step_ms"] * 1e3, p["rq_ms"] * 1e3, p["rq_graph_us"], p["gemm_ms"] * 1e3,
                                       p["wall_ms"] * 1e3))
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        res["decode"] = bench_decode(cr, wl, torch, args.steps, args.warmup)
    if args.only in ("all", "w4a4"):
        res["w4a4"] = bench_w4a4(cr, wl, torch, args.steps, args.warmup)
        r4 = res["w4a4"]
        log("w4a4: GEMM %.1f us (%.0f TOP/s), e2e %.1f us; pre-encoded weights: GEMM %.1f us, e2e %.1f us; "
            "W8A8 e2e %.1f us" % (r4["gemm_us"], r4["gemm_tops"], r4["e2e_us"], r4["packed_gemm_us"],
                                   r4["packed_e2e_us"], r4["w8a8_e2e_us"]))
        torch.cuda.empty_cache()
    if args.only in ("all", "stack"):
        res["stack"] = bench_stack(cr, wl, torch, args.stack_layers)
        rs = res["stack"]
        log("stack: median layer %.1f us (%.0f TOP/s) as 7 linears; %.1f us (%.0f TOP/s) with q|k|v and gate|up "
            "as one GEMM each" % (rs["median_layer_us"], rs["median_layer_tops"], rs["fused_median_layer_us"],
                                  rs["fused_median_layer_tops"]))
    if args.only in ("all", "split"):
        res["split"] = bench_split(cr, torch, args.steps, args.warmup)
    cpu = None
    if not args.no_cpu_baseline and args.only in ("all", "prefill"):
        cpu = cpu_baseline(wl, torch)
        log("cpu baseline: %.4f TOP/s on %d threads" % (cpu["value"], cpu["cores"]))

    line = {"metric": "ConvRot linear int8 TOPS @M=4096 + weight GB/s @M=12, % of MI355X roofline",
            "n_gpus": 1, "steps": args.steps, "warmup": args.warmup, "higher_is_better": True,
            "scaling": "weak", "vs_baseline": None, "dtype": "int8", "data": "synthetic"}
    if "prefill" in res:
        p = res["prefill"]
        gemm_tops = p["ops"] / (p["gemm_ms"] * 1e-3) / 1e12
        rq_gbs = p["rq_bytes"] / (p["rq_ms"] * 1e-3) / 1e9
        h = src_hash("gemm_i8.hip")
        line.update({
            "value": p["ops"] / (p["step_ms"] * 1e-3) / 1e12, "unit": "TOP/s", "ms_per_step": p["step_ms"],
            "wall_ms_per_step": p["wall_ms"],
            "config": {"workload": "ConvRot W8A8 linear, prefill attn.qkv_proj-shaped: M=4096 tokens, K=5376 "
                                   "(21 groups of 256), N=16128; bf16 x N(0,1) with 0.5% outlier channels x50; "
                                   "W N(0,0.02); fp32 bias; bf16 out; step = rotate+quantize x, then GEMM+dequant",
                       "M": p["M"], "K": p["K"], "N": p["N"], "group": 256},
            "roofline": {"bound": "mfma", "kernel": "gemm_i8 (int8 MFMA GEMM + dequant epilogue)",
                         "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                         "frac": gemm_tops / PEAK_INT8_TOPS,
                         "traffic": traffic_from_profiles("gemm_i8_prefill", h),
                         "traffic_kind": TRAFFIC_KIND,
                         "algorithmic_bytes": p["gemm_bytes"], "source_hash": h},
            "kernels": {"rotate_quant_us": p["rq_ms"] * 1e3, "rotate_quant_GBps": rq_gbs,
                        "rotate_quant_frac_hbm": rq_gbs / PEAK_HBM_GBS,
                        "rotate_quant_graph_us": p["rq_graph_us"],
                        "rotate_quant_graph_frac_hbm": p["rq_bytes"] / (p["rq_graph_us"] * 1e-6) / 1e9 / PEAK_HBM_GBS,
                        "rotate_quant_traffic": traffic_from_profiles("rotate_quant_prefill",
                                                                      src_hash("rotate_quant.hip")),
                        "gemm_us": p["gemm_ms"] * 1e3, "gemm_TOPs": gemm_tops,
                        "gemm_frac_int8_peak": gemm_tops / PEAK_INT8_TOPS},
        })
    else:
        line.update({"value": None, "unit": "TOP/s", "ms_per_step": None,
                     "config": {"workload": "partial run (--only %s)" % args.only}})
    if "decode" in res:
        line["decode_m12"] = res["decode"]
    if "w4a4" in res:
        line["w4a4"] = res["w4a4"]
    if "stack" in res:
        line["layer_stack"] = res["stack"]
    if "split" in res:
        line["split_k_tail"] = res["split"]
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
