#!/usr/bin/env python3
"""Benchmark of the ConvRot quantized linear on one MI355X.

One step = one ConvRot INT8 linear at the prefill workload (M=4096 tokens, K=5376, N=16128,
bf16 activations with outlier channels, prepared INT8 weights, fp32 bias, bf16 out):
rotate+quantize the activations (KR1), then the INT8 MFMA GEMM with the fused dequant epilogue
(KR2).  Inputs and weights cycle through rings of distinct buffers (>= 1 GiB each) so every
step reads HBM rather than the 256 MB last-level cache.  `value` is whole-step int8 TOP/s.

The same run also measures, with its own timed loops of the same length:
  * decode (M=12) linears on the four Qwen3-VL-32B-like shapes: weight GB/s of the split-K
    GEMV kernel (x pre-quantized) and end-to-end (rotate+quantize + GEMV);
  * the W4A4 linear at M=4096, K=5376, N=10752 and the 20% W8A8 mixed profile;
  * the CPU oracle on a bounded sample of the prefill workload (cpu_baseline).
Per-kernel durations come from HIP events recorded on the stream the kernels run on.
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

PEAK_INT8_TOPS = 5000.0      # MI355X dense int8 MFMA, TOP/s (published)
PEAK_HBM_GBS = 8000.0        # MI355X HBM3E, GB/s (published)
RING_BYTES = 1 << 30


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--only", choices=["all", "prefill", "decode", "w4a4"], default="all",
                    help="restrict the measured workloads (profiling runs)")
    return ap.parse_args()


def ring_count(bytes_each: int) -> int:
    return max(2, -(-RING_BYTES // max(bytes_each, 1)))


def timed_loop(fn, steps: int, warmup: int, torch):
    """Run fn(i) warmup + steps times; returns (wall ms per step, [per-call event lists])."""
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


def ev_ms(a, b):
    return a.elapsed_time(b)


def src_hash(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "int4_quantized_linear_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profiles(kernel_key: str, current_hash: str):
    """HBM bytes per launch from committed rocprofv3 counter summaries, if they were taken on
    the current kernel source; otherwise None."""
    p = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    if not os.path.exists(p):
        return None
    try:
        d = json.load(open(p)).get(kernel_key)
    except (OSError, ValueError):
        return None
    if not d or d.get("source_hash") != current_hash:
        return None
    return d.get("bytes_per_launch")


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
    wss = [ws0] * nw
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
        cr.linear(None, wqs[i % nw], wss[i % nw], bd, group=256, xq=xq, x_scale=xsc, out=y)
        e[2].record(st)
        return e

    wall, marks = timed_loop(step, steps, warmup, torch)
    t_rq = sum(ev_ms(m[0], m[1]) for m in marks) / steps
    t_gemm = sum(ev_ms(m[1], m[2]) for m in marks) / steps
    t_step = sum(ev_ms(m[0], m[2]) for m in marks) / steps
    ops = 2.0 * M * N * K
    rq_bytes = M * K * 2 + M * K + 4 * M
    gemm_bytes = M * K + N * K + 4 * M + 4 * N + 4 * N + 2 * M * N
    return dict(M=M, K=K, N=N, ops=ops, wall_ms=wall, step_ms=t_step, rq_ms=t_rq, gemm_ms=t_gemm,
                rq_bytes=rq_bytes, gemm_bytes=gemm_bytes)


def bench_decode(cr, wl, torch, steps, warmup):
    dev = torch.device("cuda:0")
    st = torch.cuda.current_stream(dev)
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
        ws = torch.empty(wsz, dtype=torch.uint8, device=dev)

        def gemv(i):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(st)
            cr._call("convrot_linear", None, 0, xq.data_ptr(), xsc.data_ptr(), M, N, K, 256,
                     wqs[i % nw].data_ptr(), ws0.data_ptr(), None, y.data_ptr(), ws.data_ptr(), wsz, st.cuda_stream)
            e[1].record(st)
            return e

        def e2e(i):
            e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            e[0].record(st)
            cr._call("convrot_linear", xd.data_ptr(), cr.CONVROT_DTYPE_BF16, None, None, M, N, K, 256,
                     wqs[i % nw].data_ptr(), ws0.data_ptr(), None, y.data_ptr(), ws.data_ptr(), wsz, st.cuda_stream)
            e[1].record(st)
            return e

        _, mg = timed_loop(gemv, steps, warmup, torch)
        _, me = timed_loop(e2e, steps, warmup, torch)
        tg = sum(ev_ms(a, b) for a, b in mg) / steps
        te = sum(ev_ms(a, b) for a, b in me) / steps
        wbytes = N * K + 4 * N
        out["K%d_N%d" % (K, N)] = dict(weight_bytes=wbytes, gemv_us=tg * 1e3, e2e_us=te * 1e3,
                                       weight_GBps=wbytes / (tg * 1e-3) / 1e9,
                                       frac_hbm=wbytes / (tg * 1e-3) / 1e9 / PEAK_HBM_GBS)
        log("decode K=%d N=%d: GEMV %.2f us (%.0f GB/s), e2e %.2f us" % (K, N, tg * 1e3, out["K%d_N%d" % (K, N)]["weight_GBps"], te * 1e3))
        del wqs, wq0
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

    def core(i):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(st)
        cr.linear_w4a4(None, wq4, ws4, bd, xq=xq4, x_scale=xs4, out=y)
        e[1].record(st)
        return e

    def e2e4(i):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(st)
        cr.linear_w4a4(xd, wq4, ws4, bd, out=y)
        e[1].record(st)
        return e

    def e2e8(i):
        e = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
        e[0].record(st)
        cr.linear(xd, wq8, ws8, bd, out=y)
        e[1].record(st)
        return e

    _, mc = timed_loop(core, steps, warmup, torch)
    _, m4 = timed_loop(e2e4, steps, warmup, torch)
    _, m8 = timed_loop(e2e8, steps, warmup, torch)
    tc = sum(ev_ms(a, b) for a, b in mc) / steps
    t4 = sum(ev_ms(a, b) for a, b in m4) / steps
    t8 = sum(ev_ms(a, b) for a, b in m8) / steps
    ops = 2.0 * M * N * K
    promoted = len(wl.mixed_profile_layers())
    mixed_ms = (240 - promoted) * t4 + promoted * t8
    return dict(M=M, K=K, N=N, gemm_us=tc * 1e3, gemm_tops=ops / (tc * 1e-3) / 1e12,
                e2e_us=t4 * 1e3, e2e_tops=ops / (t4 * 1e-3) / 1e12, w8a8_e2e_us=t8 * 1e3,
                mixed_profile=dict(layers=240, w8a8_layers=promoted, total_ms=mixed_ms,
                                   effective_tops=240 * ops / (mixed_ms * 1e-3) / 1e12))


def cpu_baseline(wl, torch):
    """The oracle as it stands on a bounded sample of the prefill workload: S tokens against R
    weight rows (weights prepared untimed, as on the GPU); timed = rotate+quantize the tokens,
    integer GEMM, dequant."""
    import numpy as np

    from oracle import oracle as orc
    S, R = 128, 2048
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
                sample="%d tokens x %d output channels of the 4096x5376x16128 prefill linear "
                       "(rotate+quantize tokens, int GEMM, dequant; weights prepared untimed); %.1f s" % (S, R, dt))


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path (run with --gpus 1)",
              file=sys.stderr)
        sys.exit(2)
    import torch

    from int4_quantized_linear_amd import convrot as cr
    from int4_quantized_linear_amd import workloads as wl
    cr.load()
    assert torch.cuda.is_available(), "bench.py needs a GPU"
    torch.cuda.set_device(0)
    res = {}
    if args.only in ("all", "prefill"):
        res["prefill"] = bench_prefill(cr, wl, torch, args.steps, args.warmup)
        p = res["prefill"]
        log("prefill: step %.1f us (rotate+quant %.1f us, GEMM %.1f us), wall %.1f us" % (
            p["step_ms"] * 1e3, p["rq_ms"] * 1e3, p["gemm_ms"] * 1e3, p["wall_ms"] * 1e3))
        torch.cuda.empty_cache()
    if args.only in ("all", "decode"):
        res["decode"] = bench_decode(cr, wl, torch, args.steps, args.warmup)
    if args.only in ("all", "w4a4"):
        res["w4a4"] = bench_w4a4(cr, wl, torch, args.steps, args.warmup)
        log("w4a4: GEMM %.1f us (%.0f TOP/s), e2e %.1f us" % (res["w4a4"]["gemm_us"], res["w4a4"]["gemm_tops"],
                                                             res["w4a4"]["e2e_us"]))
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
                                   "(21 groups of 256), N=16128; bf16 x with 0.5% outlier channels x50; bias; bf16 out",
                       "M": p["M"], "K": p["K"], "N": p["N"], "group": 256},
            "roofline": {"bound": "mfma", "kernel": "gemm_i8 (int8 MFMA GEMM + dequant epilogue)",
                         "achieved": gemm_tops, "peak": PEAK_INT8_TOPS, "unit": "TOP/s",
                         "frac": gemm_tops / PEAK_INT8_TOPS,
                         "traffic": traffic_from_profiles("gemm_i8_prefill", h), "source_hash": h},
            "kernels": {"rotate_quant_us": p["rq_ms"] * 1e3, "rotate_quant_GBps": rq_gbs,
                        "rotate_quant_frac_hbm": rq_gbs / PEAK_HBM_GBS,
                        "gemm_us": p["gemm_ms"] * 1e3, "gemm_TOPs": gemm_tops,
                        "gemm_frac_int8_peak": gemm_tops / PEAK_INT8_TOPS},
        })
    if "decode" in res:
        line["decode_m12"] = res["decode"]
    if "w4a4" in res:
        line["w4a4"] = res["w4a4"]
    line["cpu_baseline"] = cpu
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
