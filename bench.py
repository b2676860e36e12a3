#!/usr/bin/env python3
"""Benchmark of the Averis linear hot path (forward + dgrad) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input
of the Qwen3-0.6B up-projection shape (l = 8192 tokens, m = 1024, n = 3072,
bf16): both quantized copies of W, split-quant of X (which also forms the
rank-one mean row for the forward GEMM), the forward GEMM, split-quant of the
output gradient D (and its rank-one row), and the dgrad GEMM.  The vanilla-FP4 arm (plain quant of X / D + the same GEMMs without
the mean term) is timed the same way to report the Averis overhead.

Inputs are resident in HBM before timing starts; the timed steps rotate
through enough copies of X and D (> 512 MB) that the 256 MB MALL cannot hold
them, so every step reads its activations from HBM.  The step is timed
three ways: op by op from Python (host clock), as one captured HIP graph per
input copy (host clock), and op by op with the launches queued behind a spin
kernel, timed by events on the launch stream.  The last is the headline: the
device's own step time, free of the host's launch cost; the other two are
reported beside it.

Prints ONE JSON line (see the keys below).
"""

import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from mean_residual_quantized_amd import averis as av  # noqa: E402
from mean_residual_quantized_amd import workloads  # noqa: E402

METRIC = "Averis fwd+dgrad TFLOP/s & split-quant GB/s (frac. roofline); % overhead vs vanilla FP4"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E
F16_MFMA_PEAK_TFLOPS = 2500.0  # dense fp16 MFMA, the instruction the GEMM uses
FP4_MFMA_PEAK_TFLOPS = 10100.0  # dense fp4, for reference only


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--l", type=int, default=8192)
    p.add_argument("--m", type=int, default=1024)
    p.add_argument("--n", type=int, default=3072)
    p.add_argument("--copies", type=int, default=0, help="rotating input copies (0: auto)")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=0,
                   help="oracle sample: tokens (0: the whole step, all l tokens)")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run a 256 MiB device copy and the hot-path kernels a few times each "
                        "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), then exit")
    return p.parse_args()


class Timer:
    """Event pairs on the current stream (the one the library launches on)."""

    def __init__(self):
        self.pairs = {}

    def start(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs.setdefault(name, []).append([e, None])

    def stop(self, name):
        e = torch.cuda.Event(enable_timing=True)
        e.record()
        self.pairs[name][-1][1] = e

    def ms(self, name):
        return [a.elapsed_time(b) for a, b in self.pairs.get(name, [])]


def run_step(x, d, w, ws, t=None, vanilla=False):
    """One pass of the hot path; returns nothing (outputs stay on device)."""
    def tic(n):
        if t:
            t.start(n)

    def toc(n):
        if t:
            t.stop(n)
    tic("wquant")
    wt, wd = av.averis_quant_pair(w, rnd=av.RN, ws=ws["q"])
    toc("wquant")
    if not vanilla:
        # the split also forms the rank-one row 1 (mean W) for the GEMM that
        # takes it, so the GEMM adds it without a mean row of its own
        tic("split_x")
        xr, _, _, rho_x = av.averis_split_quant_rank1(x, wt, seed=0, ws=ws["sq_x"], rho=ws["rho_x"])
        toc("split_x")
        tic("gemm_fwd")
        av.averis_gemm_rank1(xr, rho_x, wt, out_dtype=torch.bfloat16, out=ws["y"])
        toc("gemm_fwd")
        tic("split_d")
        dr, _, _, rho_d = av.averis_split_quant_rank1(d, wd, seed=1, ws=ws["sq_d"], rho=ws["rho_d"])
        toc("split_d")
        tic("gemm_dgrad")
        av.averis_gemm_rank1(dr, rho_d, wd, out_dtype=torch.bfloat16, out=ws["dx"])
        toc("gemm_dgrad")
    else:
        tic("vq_x")
        xq = av.averis_quant(x, seed=0, ws=ws["sq_x"])
        toc("vq_x")
        tic("vgemm_fwd")
        av.averis_gemm_vanilla(xq, wt, out_dtype=torch.bfloat16, out=ws["y"], ws=ws["g"])
        toc("vgemm_fwd")
        tic("vq_d")
        dq = av.averis_quant(d, seed=1, ws=ws["sq_d"])
        toc("vq_d")
        tic("vgemm_dgrad")
        av.averis_gemm_vanilla(dq, wd, out_dtype=torch.bfloat16, out=ws["dx"], ws=ws["g"])
        toc("vgemm_dgrad")


def capture(xs, ds, w, ws, vanilla):
    """One HIP graph per rotating input copy, each holding one whole step
    (every launch of the step, outputs in the graphs' shared pool)."""
    graphs = []
    pool = None
    for i in range(len(xs)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, pool=pool):
            run_step(xs[i], ds[i], w, ws, None, vanilla)
        pool = g.pool()
        graphs.append(g)
    torch.cuda.synchronize()
    return graphs


_SLEEP_CYCLES_PER_MS = None


def hold_gpu(ms):
    """Enqueue a spin kernel of about `ms` milliseconds, so that the launches
    queued behind it run back to back, with no wait on the host."""
    global _SLEEP_CYCLES_PER_MS
    if _SLEEP_CYCLES_PER_MS is None:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda._sleep(1000)
        e0.record()
        torch.cuda._sleep(20_000_000)
        e1.record()
        torch.cuda.synchronize()
        _SLEEP_CYCLES_PER_MS = 20_000_000 / max(e0.elapsed_time(e1), 1e-3)
    torch.cuda._sleep(int(ms * _SLEEP_CYCLES_PER_MS))


def timed(xs, ds, w, ws, steps, warmup, vanilla):
    """Step time three ways (ms/step) and a per-call event timer.

    eager:  one Python call per op, timed on the host around the loop;
    graph:  one captured HIP graph per input copy, replayed;
    queued: the eager launches queued behind a spin kernel and timed with
            events on the launch stream: the device's own step time, with the
            host's launch cost taken out."""
    for i in range(warmup):
        run_step(xs[i % len(xs)], ds[i % len(ds)], w, ws, None, vanilla)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(xs[i % len(xs)], ds[i % len(ds)], w, ws, None, vanilla)
    enqueue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps

    graphs = capture(xs, ds, w, ws, vanilla)
    for i in range(warmup):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        graphs[i % len(graphs)].replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / steps
    del graphs

    hold = 2.0 * enqueue_ms + 2.0
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    hold_gpu(hold)
    e0.record()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(xs[i % len(xs)], ds[i % len(ds)], w, ws, None, vanilla)
    e1.record()
    queued_enqueue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    queued_ms = e0.elapsed_time(e1) / steps
    if queued_enqueue_ms > 0.8 * hold:
        log("bench: warning: enqueue took %.2f ms of a %.2f ms hold" % (queued_enqueue_ms, hold))

    # per-kernel-call durations, events on the launch stream, same rotation,
    # also queued behind a spin kernel
    t = Timer()
    hold_gpu(hold * 1.5)
    for i in range(steps):
        run_step(xs[i % len(xs)], ds[i % len(ds)], w, ws, t, vanilla)
    torch.cuda.synchronize()
    return dict(eager=eager_ms, graph=graph_ms, queued=queued_ms), t


def time_wgrad(xs, ds, ws, steps, warmup):
    """The wgrad pieces, queued behind a spin kernel and timed per call by
    events on the launch stream, rotating through the input copies: the
    transposed residual quants of X and D (their means and residual tensor
    scales come from the splits the forward and dgrad passes run) and the
    wgrad product dW = deq(xt) deq(dt)^T + l mu_X mu_D^T (fp32 out)."""
    l, m = xs[0].shape
    n = ds[0].shape[1]
    xr, _, mx = av.averis_split_quant(xs[0], seed=0, ws=ws["sq_x"])
    dr, _, md = av.averis_split_quant(ds[0], seed=1, ws=ws["sq_d"])
    xt = av.NVFP4.empty(m, l, 1, xs[0].device)
    dt = av.NVFP4.empty(n, l, 1, xs[0].device)
    dw = torch.empty((m, n), dtype=torch.float32, device=xs[0].device)
    wws = torch.empty(av.workspace_bytes(av.OP_WGRAD, m, l, n), dtype=torch.uint8,
                      device=xs[0].device)

    def one(i, t):
        def tic(k):
            if t:
                t.start(k)

        def toc(k):
            if t:
                t.stop(k)
        tic("rt_x")
        av.averis_residual_t_quant(xs[i % len(xs)], mx, xr, seed=0, out=xt)
        toc("rt_x")
        tic("rt_d")
        av.averis_residual_t_quant(ds[i % len(ds)], md, dr, seed=1, out=dt)
        toc("rt_d")
        tic("gemm_wgrad")
        av.averis_gemm_wgrad(xt, dt, mx, md, out=dw, ws=wws)
        toc("gemm_wgrad")

    for i in range(warmup):
        one(i, None)
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for i in range(steps):
        one(i, t)
    torch.cuda.synchronize()
    med = lambda v: float(np.median(v))
    ms = {k: med(t.ms(k)) for k in ("rt_x", "rt_d", "gemm_wgrad")}
    rt_bytes = lambda rows, cols: rows * cols * (2 + 0.5 + 1 / 16)
    flops = 2.0 * l * m * n
    return dict(
        ms=ms,
        rt_gbs={"x": rt_bytes(l, m) / (ms["rt_x"] * 1e-3) / 1e9,
                "d": rt_bytes(l, n) / (ms["rt_d"] * 1e-3) / 1e9},
        gemm_tflops=flops / (ms["gemm_wgrad"] * 1e-3) / 1e12,
        splits_of_tokens=int(av.workspace_bytes(av.OP_WGRAD, m, l, n) // (m * n * 4)),
        note="dW (m x n) = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X mu_D^T, fp32 out; "
             "gemm_wgrad covers the split-K GEMM and the reduce that adds the outer product")


def time_ratio(xs, ds, ws, steps, warmup):
    """Split-quant of X and D with and without the mean-energy ratio, per call
    (events on the launch stream, queued behind a spin kernel, rotating
    copies), and the ratios themselves."""
    def one(i, t):
        for name, src, key in (("x", xs, "sq_x"), ("d", ds, "sq_d")):
            a = src[i % len(src)]
            t.start("plain_" + name)
            av.averis_split_quant(a, seed=0, ws=ws[key])
            t.stop("plain_" + name)
            t.start("ratio_" + name)
            out = av.averis_split_quant_ratio(a, seed=0, ws=ws[key])
            t.stop("ratio_" + name)
            ratios[name] = out[3]

    ratios = {}
    for i in range(warmup):
        one(i, Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for i in range(steps):
        one(i, t)
    torch.cuda.synchronize()
    med = lambda v: float(np.median(v))
    return {name: dict(split_ms=med(t.ms("plain_" + name)), split_with_ratio_ms=med(t.ms("ratio_" + name)),
                       ratio=float(ratios[name][0].item()))
            for name in ("x", "d")}


def time_weight_copies(w, ws, steps, warmup):
    """Both weight copies per call (events on the launch stream, queued behind
    a spin kernel): the two 1-D quantizations (averis_quant_pair) and the
    shared 16x16-tile quantization (averis_quant_pair_2d)."""
    def one(t):
        t.start("pair")
        av.averis_quant_pair(w, rnd=av.RN, ws=ws["q"])
        t.stop("pair")
        t.start("pair_2d")
        av.averis_quant_pair_2d(w, rnd=av.RN, ws=ws["q"])
        t.stop("pair_2d")

    for _ in range(warmup):
        one(Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.2 * steps)
    for _ in range(steps):
        one(t)
    torch.cuda.synchronize()
    return dict(pair_ms=float(np.median(t.ms("pair"))), pair_2d_ms=float(np.median(t.ms("pair_2d"))))


def cpu_baseline(cfg_rows, m, n):
    """The oracle as it stands on a bounded sample: cfg_rows tokens of the
    same workload (split-quant of X and D, both weight copies, the float64
    forward and dgrad GEMMs); reported in TFLOP/s of the sample's GEMMs."""
    from oracle import averis as orc
    cfg = workloads.up_proj(l=cfg_rows, m=m, n=n)
    x, w, d = cfg["x"].float().numpy(), cfg["w"].float().numpy(), cfg["d"].float().numpy()
    t0 = time.perf_counter()
    wq = orc.weight_quant(w, "rn")
    orc.averis_forward(x, wq["fwd"], "sr", 0)
    orc.averis_dgrad(d, wq["dgrad"], "sr", 1)
    dt = time.perf_counter() - t0
    flops = 2 * (2.0 * cfg_rows * m * n)
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = 1
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(blas), kind="oracle",
                sample="%d tokens of the l=8192 workload (m=%d, n=%d), one step: split-quant X and D, "
                       "both weight copies, float64 fwd+dgrad GEMMs; %.1f s; numpy elementwise "
                       "work single-threaded, float64 matmul on %d BLAS threads of %d host cores"
                       % (cfg_rows, m, n, dt, blas, len(os.sched_getaffinity(0))),
                seconds=dt)


COPY_BYTES = 256 << 20


def traffic_probe(args):
    """A device copy of known size (the scale reference for the HBM byte
    counters) followed by three launches of each hot-path kernel."""
    l, m, n = args.l, args.m, args.n
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    cfg = workloads.up_proj(l=l, m=m, n=n)
    x, w, d = cfg["x"].cuda(), cfg["w"].cuda(), cfg["d"].cuda()
    torch.cuda.synchronize()
    for _ in range(3):
        wt, wd = av.averis_quant_pair(w, rnd=av.RN)
        xr, _, mx, rho_x = av.averis_split_quant_rank1(x, wt, seed=0)
        av.averis_gemm_rank1(xr, rho_x, wt, out_dtype=torch.bfloat16)
        dr, _, md, rho_d = av.averis_split_quant_rank1(d, wd, seed=1)
        av.averis_gemm_rank1(dr, rho_d, wd, out_dtype=torch.bfloat16)
        xt = av.averis_residual_t_quant(x, mx, xr, seed=0)
        dt = av.averis_residual_t_quant(d, md, dr, seed=1)
        av.averis_gemm_wgrad(xt, dt, mx, md)
    torch.cuda.synchronize()
    print("traffic probe done: copy %d bytes" % COPY_BYTES, file=sys.stderr)


GEMM_SOURCES = ["gemm.hip", "gemm_ws.hip", "gemm_common.hpp"]


def gemm_source_sha():
    """One hash over the sources of the forward GEMM kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "mean_residual_quantized_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def load_traffic():
    """HBM bytes per forward GEMM launch (k_gemm_ws) from the committed counter
    summary, if it was taken on the current kernel sources (else None)."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        rec = json.load(open(path))
        sha = gemm_source_sha()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_sources_sha256") != sha:
        return None
    return rec


def main():
    args = parse()
    if args.traffic_probe:
        traffic_probe(args)
        return
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    av.lib()
    l, m, n = args.l, args.m, args.n
    log("bench: generating inputs l=%d m=%d n=%d" % (l, m, n))
    cfg = workloads.up_proj(l=l, m=m, n=n)
    x0, w0, d0 = cfg["x"].cuda(), cfg["w"].cuda(), cfg["d"].cuda()
    bytes_per_set = (x0.numel() + d0.numel()) * 2
    copies = args.copies or max(2, int(np.ceil(640e6 / bytes_per_set)))
    xs = [x0] + [x0.clone() for _ in range(copies - 1)]
    ds = [d0] + [d0.clone() for _ in range(copies - 1)]
    dev = x0.device
    ws = dict(
        q=torch.empty(max(av.workspace_bytes(av.OP_QUANT, n, m),
                          av.workspace_bytes(av.OP_QUANT, m, n)), dtype=torch.uint8, device=dev),
        sq_x=torch.empty(av.workspace_bytes(av.OP_SPLIT_QUANT, l, m), dtype=torch.uint8,
                         device=dev),
        sq_d=torch.empty(av.workspace_bytes(av.OP_SPLIT_QUANT, l, n), dtype=torch.uint8,
                         device=dev),
        g=torch.empty(av.workspace_bytes(av.OP_GEMM, l, max(m, n), max(m, n)), dtype=torch.uint8,
                      device=dev),
        y=torch.empty((l, n), dtype=torch.bfloat16, device=dev),
        dx=torch.empty((l, m), dtype=torch.bfloat16, device=dev),
        rho_x=torch.empty((n,), dtype=torch.float32, device=dev),
        rho_d=torch.empty((m,), dtype=torch.float32, device=dev),
    )
    log("bench: %d rotating input copies; warmup %d, steps %d" % (copies, args.warmup, args.steps))
    ta_ms, ta = timed(xs, ds, w0, ws, args.steps, args.warmup, vanilla=False)
    tv_ms, tv = timed(xs, ds, w0, ws, args.steps, args.warmup, vanilla=True)
    log("bench: averis %s, vanilla %s (ms/step)" % (
        " ".join("%s %.4f" % kv for kv in ta_ms.items()),
        " ".join("%s %.4f" % kv for kv in tv_ms.items())))
    log("bench: wgrad pieces")
    wg = time_wgrad(xs, ds, ws, args.steps, args.warmup)
    log("bench: mean-energy ratio")
    mer = time_ratio(xs, ds, ws, args.steps, args.warmup)
    log("bench: weight copies")
    wc = time_weight_copies(w0, ws, args.steps, args.warmup)
    # the headline is the device's step time (launches queued ahead of it)
    ms_a, ms_v = ta_ms["queued"], tv_ms["queued"]

    gemm_flops = 2.0 * l * m * n
    med = lambda v: float(np.median(v)) if v else float("nan")
    comp = {k: med(ta.ms(k)) for k in ["wquant", "split_x", "gemm_fwd", "split_d", "gemm_dgrad"]}
    compv = {k: med(tv.ms(k)) for k in ["vq_x", "vgemm_fwd", "vq_d", "vgemm_dgrad"]}
    sq_bytes = lambda rows, cols: rows * cols * (2 + 0.5 + 1 / 16)   # algorithmic bytes
    gbs = lambda b, ms: b / (ms * 1e-3) / 1e9
    split = {
        "x": dict(ms=comp["split_x"], gbs=gbs(sq_bytes(l, m), comp["split_x"])),
        "d": dict(ms=comp["split_d"], gbs=gbs(sq_bytes(l, n), comp["split_d"])),
    }
    for v in split.values():
        v["frac_hbm"] = v["gbs"] / HBM_PEAK_GBS
    vq = {"x": dict(ms=compv["vq_x"], gbs=gbs(sq_bytes(l, m), compv["vq_x"])),
          "d": dict(ms=compv["vq_d"], gbs=gbs(sq_bytes(l, n), compv["vq_d"]))}
    gemm = {k: dict(ms=comp[k], tflops=gemm_flops / (comp[k] * 1e-3) / 1e12)
            for k in ["gemm_fwd", "gemm_dgrad"]}
    vgemm = {k: dict(ms=compv[k], tflops=gemm_flops / (compv[k] * 1e-3) / 1e12)
             for k in ["vgemm_fwd", "vgemm_dgrad"]}
    t_fwd_a = comp["split_x"] + comp["gemm_fwd"]
    t_fwd_v = compv["vq_x"] + compv["vgemm_fwd"]
    t_bwd_a = comp["split_d"] + comp["gemm_dgrad"]
    t_bwd_v = compv["vq_d"] + compv["vgemm_dgrad"]
    overhead = dict(fwd_pct=100 * (t_fwd_a / t_fwd_v - 1), dgrad_pct=100 * (t_bwd_a / t_bwd_v - 1),
                    step_pct=100 * (ms_a / ms_v - 1))

    # roofline of the dominant kernel: the Averis forward GEMM, one launch of
    # k_gemm_ws (the NT GEMM over the residual codes; the epilogue adds the
    # rank-one row the split formed), timed by the events around the call on
    # the launch stream.  The flops counted are the GEMM's 2lmn.
    g_ms = comp["gemm_fwd"]
    achieved = gemm_flops / (g_ms * 1e-3) / 1e12
    tr = load_traffic()
    traffic = None
    if tr is not None:
        traffic = tr["gemm_fwd"]["fetch_bytes"] + tr["gemm_fwd"]["write_bytes"]
    roofline = dict(bound="mfma", achieved=achieved, peak=F16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / F16_MFMA_PEAK_TFLOPS, traffic=traffic,
                    kernel="k_gemm_ws (averis_gemm_rank1 on the forward operands: warp-specialized "
                           "NVFP4 NT GEMM, exact fp16 dequant -> v_mfma_f32_32x32x16_f16, the rank-one "
                           "row from the split added in the epilogue), M=%d N=%d K=%d, bf16 out"
                           % (l, n, m),
                    frac_of_fp4_peak=achieved / FP4_MFMA_PEAK_TFLOPS)

    out = {
        "metric": METRIC,
        "value": 2 * gemm_flops / (ms_a * 1e-3) / 1e12,
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_a,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 + e4m3 scales) operands, f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": "Qwen3-0.6B-shaped up-proj, Averis fwd+dgrad step",
                   "tokens": l, "m": m, "n": n, "input_dtype": "bf16", "sr": "philox4x32-10, 16 bits",
                   "rotating_input_copies": copies},
        "roofline": roofline,
        "split_quant": split,
        "vanilla_quant": vq,
        "gemm": gemm,
        "vanilla_gemm": vgemm,
        "weight_quant_ms": comp["wquant"],
        "vanilla_ms_per_step": ms_v,
        "step_ms_by_launch": {"averis": ta_ms, "vanilla": tv_ms,
                              "queued": "launches queued behind a spin kernel, events on the "
                                        "launch stream (the headline)",
                              "eager": "one Python call per op, host clock",
                              "graph": "one HIP graph per step, replayed, host clock"},
        "overhead_vs_vanilla": overhead,
        "wgrad": wg,
        "mean_energy_ratio": mer,
        "weight_copies": wc,
        "pages_overhead_context": "2.20% end-to-end over vanilla NVFP4 (hardware not stated)",
    }
    if not args.no_cpu_baseline:
        log("bench: timing the oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(args.cpu_rows or l, m, n)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
