#!/usr/bin/env python3
"""Benchmark of the Averis linear hot path (forward + dgrad) on one MI355X.

One step = one pass of the whole hot path over one batch of synthetic input:
for every linear of the workload, both quantized copies of W, split-quant of
X (which also forms the rank-one mean row for the forward GEMM), the forward
GEMM, split-quant of the output gradient D (and its rank-one row), and the
dgrad GEMM.  The vanilla-FP4 arm (plain quant of X / D + the same GEMMs
without the mean term) is timed the same way to report the Averis overhead.

Workloads (--config):
  4  the Qwen3-0.6B-like block sweep at l = 16384 tokens: q, k, v, o, gate,
     up, down (the headline: the largest workload that fits one GPU)
  1  the up-projection, l = 8192, m = 1024, n = 3072
  2  the down-projection with SwiGLU-like inputs, l = 8192, m = 3072, n = 1024
  3  the MoE-shaped grouped case: 32768 routed rows over 64 experts (Zipf
     popularity), hidden 2048, expert width 768
The headline config is timed first; the others follow as extra fields
(--only-headline skips them).

Inputs are resident in HBM before timing starts; where one step's
activations are smaller than 640 MB the timed steps rotate through enough
copies of them that the 256 MB MALL cannot hold them, so every step reads its
activations from HBM.  The step is timed three ways: op by op from Python
(host clock), as one captured HIP graph per input copy (host clock), and op by
op with the launches queued behind a spin kernel, timed by events on the
launch stream.  The last is the headline: the device's own step time, free of
the host's launch cost.

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
ROTATE_BYTES = 640e6           # > the 256 MB MALL
SQ_BYTES_PER_ELEM = 2 + 0.5 + 1 / 16   # split-quant: bf16 read, codes + scales written

WORKLOAD_NAMES = {
    1: "Qwen3-0.6B-shaped up-proj (l=8192, 1024->3072), Averis fwd+dgrad step",
    2: "Qwen3-0.6B-shaped down-proj with SwiGLU-like inputs (l=8192, 3072->1024), Averis fwd+dgrad step",
    3: "MoE-shaped grouped linear: 32768 routed rows over 64 experts (Zipf 1.1), 2048->768, "
       "Averis fwd+dgrad step",
    4: "Qwen3-0.6B-like block sweep at l=16384: q, k, v, o, gate, up, down, Averis fwd+dgrad step",
}


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def parse():
    p = argparse.ArgumentParser()
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=20)
    p.add_argument("--warmup", type=int, default=5)
    p.add_argument("--config", type=int, default=4, choices=[1, 2, 3, 4],
                   help="headline workload (default 4, the seven-linear block sweep)")
    p.add_argument("--only-headline", action="store_true",
                   help="time the headline config only (no other configs, wgrad, ratio, weight copies)")
    p.add_argument("--copies", type=int, default=0, help="rotating input copies (0: auto)")
    p.add_argument("--streams", type=int, default=2, choices=[1, 2],
                   help="2: each dense linear's dgrad split runs on a second stream, beside "
                        "the forward pass (both arms); 1: every op on the launch stream")
    p.add_argument("--no-cpu-baseline", action="store_true")
    p.add_argument("--cpu-rows", type=int, default=3072,
                   help="oracle sample: tokens of every linear of the headline workload")
    p.add_argument("--traffic-probe", action="store_true",
                   help="run a 256 MiB device copy and three Averis steps of the headline config "
                        "(for rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE), then exit")
    return p.parse_args()


# --------------------------------------------------------------------------
# workloads
# --------------------------------------------------------------------------

class Linear:
    """One linear of a workload: inputs on the device and preallocated
    outputs and workspaces (so the timed steps allocate nothing new)."""

    def __init__(self, name, x, w, d, offsets=None):
        dev = torch.device("cuda")
        self.name = name
        self.x0, self.w, self.d0 = x.to(dev), w.to(dev), d.to(dev)
        self.l, self.m = self.x0.shape
        self.n = self.d0.shape[1]
        self.offsets = None if offsets is None else torch.as_tensor(offsets, dtype=torch.int64,
                                                                    device=dev)
        self.nseg = 1 if offsets is None else len(offsets) - 1
        # the linear whose input this one shares in a transformer block (k and
        # v take q's, up takes gate's): with --shared-input-steps its split is
        # reused, not recomputed
        self.share_src = None
        self.dependents = []   # the linears that take this one's input
        self.last_split = None
        self.cur_w = None      # this step's two weight copies
        ns = 0 if offsets is None else self.nseg
        l, m, n = self.l, self.m, self.n
        wm, wn = (self.w.shape[1], self.w.shape[2]) if self.w.dim() == 3 else self.w.shape
        self.ws = dict(
            q=torch.empty(av.workspace_bytes(av.OP_QUANT, wm, wn, 0, self.w.shape[0]
                                             if self.w.dim() == 3 else 0) + 256,
                          dtype=torch.uint8, device=dev),
            sq_x=torch.empty(max(av.workspace_bytes(av.OP_SPLIT_QUANT, l, m, 0, ns),
                                 av.workspace_bytes(av.OP_QUANT, l, m, 0, ns)),
                             dtype=torch.uint8, device=dev),
            sq_d=torch.empty(max(av.workspace_bytes(av.OP_SPLIT_QUANT, l, n, 0, ns),
                                 av.workspace_bytes(av.OP_QUANT, l, n, 0, ns)),
                             dtype=torch.uint8, device=dev),
            g=torch.empty(av.workspace_bytes(av.OP_GEMM, l, max(m, n), max(m, n), ns),
                          dtype=torch.uint8, device=dev),
            y=torch.empty((l, n), dtype=torch.bfloat16, device=dev),
            dx=torch.empty((l, m), dtype=torch.bfloat16, device=dev),
            rho_x=torch.empty((self.nseg * n,), dtype=torch.float32, device=dev),
            rho_d=torch.empty((self.nseg * m,), dtype=torch.float32, device=dev),
        )
        # the dgrad split's outputs (written on the side stream)
        nsg = self.nseg
        self.ws.update(d_res=av.NVFP4.empty(l, n, nsg, dev), d_mean=av.NVFP4.empty(nsg, n, nsg, dev),
                       d_mu=torch.empty((n,) if offsets is None else (nsg, n), dtype=torch.float32,
                                        device=dev),
                       d_q=av.NVFP4.empty(l, n, nsg, dev))
        self.xs, self.ds = [self.x0], [self.d0]

    def act_bytes(self):
        return (self.x0.numel() + self.d0.numel()) * 2

    def rotate(self, copies):
        self.xs = [self.x0] + [self.x0.clone() for _ in range(copies - 1)]
        self.ds = [self.d0] + [self.d0.clone() for _ in range(copies - 1)]

    def flops(self):
        """GEMM flops of one pass (fwd or dgrad): 2 l m n."""
        return 2.0 * self.l * self.m * self.n


def make_linears(cfg):
    if cfg == 1:
        c = workloads.up_proj()
        return [Linear("up_proj", c["x"], c["w"], c["d"])]
    if cfg == 2:
        c = workloads.down_proj()
        return [Linear("down_proj", c["x"], c["w"], c["d"])]
    if cfg == 3:
        c = workloads.moe()
        return [Linear("moe", c["x"], c["w"], c["d"], offsets=c["offsets"])]
    out = []
    for name in workloads.QWEN3_06B_LINEARS:
        c = workloads.block_linear(name)
        out.append(Linear(name, c["x"], c["w"], c["d"]))
    by_name = {L.name: L for L in out}
    for dst, src in SHARED_INPUTS.items():
        by_name[dst].share_src = by_name[src]
        by_name[src].dependents.append(by_name[dst])
    out[0].ws["qm"] = torch.empty(av.workspace_bytes(av.OP_QUANT_PAIR_MULTI, 0, 0, len(out)),
                                  dtype=torch.uint8, device="cuda")
    return out


# in a transformer block q, k, v read one input, gate and up another
SHARED_INPUTS = {"k": "q", "v": "q", "up": "gate"}


# --------------------------------------------------------------------------
# timing
# --------------------------------------------------------------------------

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


def run_linear(L, i, t, vanilla, shared=False, wq=None, side=None):
    """One linear's forward + dgrad with input copy i.  shared: a linear
    whose input is another's (L.share_src) reuses that linear's split (or
    plain quant) of it from the same step; the Averis GEMM then takes the
    rank-one row the source's split formed for it
    (averis_split_quant_rank1_multi).  wq: both copies of the weight, when
    the step quantized all weights at once.  side: a second stream on which
    the dgrad pass's split of D (independent of the forward pass) runs while
    the main stream does the forward pass; the dgrad GEMM waits for it."""
    def tic(k):
        if t:
            t.start(L.name + "/" + k)

    def toc(k):
        if t:
            t.stop(L.name + "/" + k)
    ws = L.ws
    x, d = L.xs[i % len(L.xs)], L.ds[i % len(L.ds)]
    if wq is None:
        tic("wquant")
        wt, wd = av.averis_quant_pair(L.w, rnd=av.RN, ws=ws["q"])
        toc("wquant")
    else:
        wt, wd = wq
    pending = None
    if side is not None and L.offsets is None:   # (grouped: below)
        fork = torch.cuda.Event()
        fork.record()
        side.wait_event(fork)
        with torch.cuda.stream(side):
            dq, rho_d = split_d(L, d, wd, vanilla)
            join = torch.cuda.Event()
            join.record()
        pending = (join, dq, rho_d)
    if L.offsets is None and shared and L.share_src is not None:
        xr, xmean = L.share_src.last_split
        tic("gemm_fwd")
        if not vanilla:
            av.averis_gemm_rank1(xr, ws["rho_x"], wt, out_dtype=torch.bfloat16, out=ws["y"])
        else:
            av.averis_gemm_vanilla(xr, wt, out_dtype=torch.bfloat16, out=ws["y"], ws=ws["g"])
        toc("gemm_fwd")
        run_dgrad(L, d, wd, t, vanilla, pending)
        return
    if L.offsets is None:
        if not vanilla:
            # the split also forms the rank-one row 1 (mean W) for the GEMM
            # that takes it (and, with shared inputs, for the GEMMs of the
            # linears that read the same input), so no GEMM adds a mean row
            tic("split_x")
            deps = L.dependents if shared else []
            if deps:
                xr, xmean, _, _ = av.averis_split_quant_rank1_multi(
                    x, [wt] + [D.cur_w[0] for D in deps], seed=0, ws=ws["sq_x"],
                    rhos=[ws["rho_x"]] + [D.ws["rho_x"] for D in deps])
                rho_x = ws["rho_x"]
            else:
                xr, xmean, _, rho_x = av.averis_split_quant_rank1(x, wt, seed=0, ws=ws["sq_x"],
                                                                  rho=ws["rho_x"])
            toc("split_x")
            L.last_split = (xr, xmean)
            tic("gemm_fwd")
            av.averis_gemm_rank1(xr, rho_x, wt, out_dtype=torch.bfloat16, out=ws["y"])
            toc("gemm_fwd")
        else:
            tic("split_x")
            xq = av.averis_quant(x, seed=0, ws=ws["sq_x"])
            toc("split_x")
            L.last_split = (xq, None)
            tic("gemm_fwd")
            av.averis_gemm_vanilla(xq, wt, out_dtype=torch.bfloat16, out=ws["y"], ws=ws["g"])
            toc("gemm_fwd")
        run_dgrad(L, d, wd, t, vanilla, pending)
        return
    offs = L.offsets
    if side is not None:
        # the grouped dgrad split on the second stream, beside the forward pass
        fork = torch.cuda.Event()
        fork.record()
        side.wait_event(fork)
        with torch.cuda.stream(side):
            if not vanilla:
                dq, _, _, rho_d = av.averis_split_quant_grouped_rank1(
                    d, offs, wd, seed=1, ws=ws["sq_d"], rho=ws["rho_d"],
                    out=(ws["d_res"], ws["d_mean"], ws["d_mu"]))
            else:
                dq = av.averis_quant_grouped(d, offs, seed=1, ws=ws["sq_d"], out=ws["d_q"])
            join = torch.cuda.Event()
            join.record()
        if not vanilla:
            xr, _, _, rho_x = av.averis_split_quant_grouped_rank1(x, offs, wt, seed=0,
                                                                  ws=ws["sq_x"])
            av.averis_gemm_grouped_rank1(xr, rho_x, wt, offs, out_dtype=torch.bfloat16,
                                         out=ws["y"])
        else:
            xq = av.averis_quant_grouped(x, offs, seed=0, ws=ws["sq_x"])
            av.averis_gemm_grouped(xq, None, wt, offs, out_dtype=torch.bfloat16, out=ws["y"],
                                   ws=ws["g"])
        torch.cuda.current_stream().wait_event(join)
        if not vanilla:
            av.averis_gemm_grouped_rank1(dq, rho_d, wd, offs, out_dtype=torch.bfloat16,
                                         out=ws["dx"])
        else:
            av.averis_gemm_grouped(dq, None, wd, offs, out_dtype=torch.bfloat16, out=ws["dx"],
                                   ws=ws["g"])
        return
    if not vanilla:
        tic("split_x")
        xr, _, _, rho_x = av.averis_split_quant_grouped_rank1(x, offs, wt, seed=0, ws=ws["sq_x"])
        toc("split_x")
        tic("gemm_fwd")
        av.averis_gemm_grouped_rank1(xr, rho_x, wt, offs, out_dtype=torch.bfloat16, out=ws["y"])
        toc("gemm_fwd")
        tic("split_d")
        dr, _, _, rho_d = av.averis_split_quant_grouped_rank1(d, offs, wd, seed=1, ws=ws["sq_d"])
        toc("split_d")
        tic("gemm_dgrad")
        av.averis_gemm_grouped_rank1(dr, rho_d, wd, offs, out_dtype=torch.bfloat16, out=ws["dx"])
        toc("gemm_dgrad")
    else:
        tic("split_x")
        xq = av.averis_quant_grouped(x, offs, seed=0, ws=ws["sq_x"])
        toc("split_x")
        tic("gemm_fwd")
        av.averis_gemm_grouped(xq, None, wt, offs, out_dtype=torch.bfloat16, out=ws["y"],
                               ws=ws["g"])
        toc("gemm_fwd")
        tic("split_d")
        dq = av.averis_quant_grouped(d, offs, seed=1, ws=ws["sq_d"])
        toc("split_d")
        tic("gemm_dgrad")
        av.averis_gemm_grouped(dq, None, wd, offs, out_dtype=torch.bfloat16, out=ws["dx"],
                               ws=ws["g"])
        toc("gemm_dgrad")


def split_d(L, d, wd, vanilla):
    """The dgrad pass's split (or plain quant) of D into the linear's own
    output buffers; returns (quantized D, rank-one row or None)."""
    ws = L.ws
    if not vanilla:
        dr, _, _, rho_d = av.averis_split_quant_rank1(
            d, wd, seed=1, ws=ws["sq_d"], rho=ws["rho_d"],
            out=(ws["d_res"], ws["d_mean"], ws["d_mu"]))
        return dr, rho_d
    return av.averis_quant(d, seed=1, ws=ws["sq_d"], out=ws["d_q"]), None


def gemm_d(L, dq, rho_d, wd, vanilla):
    ws = L.ws
    if not vanilla:
        av.averis_gemm_rank1(dq, rho_d, wd, out_dtype=torch.bfloat16, out=ws["dx"])
    else:
        av.averis_gemm_vanilla(dq, wd, out_dtype=torch.bfloat16, out=ws["dx"], ws=ws["g"])


def run_dgrad(L, d, wd, t, vanilla, pending=None):
    """The dgrad pass of a dense linear (split or plain quant of D, GEMM).
    pending: (join event, quantized D, rank-one row) of a split already
    issued on the side stream; the GEMM waits for it."""
    if pending is not None:
        join, dq, rho_d = pending
        torch.cuda.current_stream().wait_event(join)
        gemm_d(L, dq, rho_d, wd, vanilla)
        return
    if t:
        t.start(L.name + "/split_d")
    dq, rho_d = split_d(L, d, wd, vanilla)
    if t:
        t.stop(L.name + "/split_d")
        t.start(L.name + "/gemm_dgrad")
    gemm_d(L, dq, rho_d, wd, vanilla)
    if t:
        t.stop(L.name + "/gemm_dgrad")


def block_weights(linears):
    """Whether a step quantizes all of its weights in one call: the dense
    linears of a transformer block (all weights are known when a step
    starts)."""
    return len(linears) > 1 and all(L.offsets is None and L.w.dim() == 2 for L in linears)


def run_step(linears, i, t=None, vanilla=False, shared=False, side=None):
    wq = [None] * len(linears)
    if block_weights(linears):
        # both copies of every weight of the block in two launches
        if t:
            t.start("block/wquant")
        wq = av.averis_quant_pair_multi([L.w for L in linears], rnd=av.RN,
                                        ws=linears[0].ws["qm"])
        if t:
            t.stop("block/wquant")
    for L, w in zip(linears, wq):
        L.cur_w = w
    for L, w in zip(linears, wq):
        run_linear(L, i, t, vanilla, shared, w, side)


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


def pct(v, q):
    return float(np.percentile(v, q)) if len(v) else float("nan")


def timed(linears, steps, warmup, vanilla, shared=False, per_call=True, side=None):
    """Step time three ways (ms/step), the per-step device times of the
    queued run, and a per-call event timer.

    eager:  one Python call per op, timed on the host around the loop;
    graph:  one captured HIP graph per input copy, replayed;
    queued: the eager launches queued behind a spin kernel and timed with
            events on the launch stream: the device's own step time, with the
            host's launch cost taken out (an event between steps gives each
            step's own time; the median step, and p10 / p90; queued_mean is
            first event to last over the steps, which a stall of the host
            feeding a full launch queue can lengthen).
    side: the second stream of the dgrad splits (not for the per-call timer,
    whose calls run one after another on the launch stream)."""
    ncopy = max(len(L.xs) for L in linears)
    for i in range(warmup):
        run_step(linears, i, None, vanilla, shared, side)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        run_step(linears, i, None, vanilla, shared, side)
    enqueue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    eager_ms = (time.perf_counter() - t0) * 1e3 / steps

    graphs = []
    pool = None
    for i in range(ncopy):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, pool=pool):
            run_step(linears, i, None, vanilla, shared, side)
        pool = g.pool()
        graphs.append(g)
    torch.cuda.synchronize()
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
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    hold_gpu(hold)
    t0 = time.perf_counter()
    for i in range(steps):
        evs[i].record()
        run_step(linears, i, None, vanilla, shared, side)
    evs[steps].record()
    queued_enqueue_ms = (time.perf_counter() - t0) * 1e3
    torch.cuda.synchronize()
    per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    queued_mean_ms = evs[0].elapsed_time(evs[steps]) / steps
    queued_ms = float(np.median(per_step))
    if queued_enqueue_ms > 0.8 * hold:
        log("bench: warning: enqueue took %.2f ms of a %.2f ms hold" % (queued_enqueue_ms, hold))

    # per-call durations, events on the launch stream, same rotation, also
    # queued behind a spin kernel
    t = Timer()
    if per_call:
        hold_gpu(hold * 2.0)
        for i in range(steps):
            run_step(linears, i, t, vanilla, shared)
        torch.cuda.synchronize()
    return dict(eager=eager_ms, graph=graph_ms, queued=queued_ms, queued_mean=queued_mean_ms,
                queued_p10=pct(per_step, 10), queued_p90=pct(per_step, 90)), t


def stats(v):
    return dict(ms=float(np.median(v)), p10=pct(v, 10), p90=pct(v, 90))


def measure(cfg, linears, steps, warmup, streams=2):
    """Both arms of one workload; returns the summary dict and the timers."""
    act = sum(L.act_bytes() for L in linears)
    copies = max(1, int(np.ceil(ROTATE_BYTES / act)))
    for L in linears:
        L.rotate(copies)
    log("bench: config %d: %d linear(s), %.0f MB of activations per step, %d rotating copies"
        % (cfg, len(linears), act / 1e6, copies))
    side = torch.cuda.Stream() if streams == 2 else None
    ta_ms, ta = timed(linears, steps, warmup, vanilla=False, side=side)
    tv_ms, tv = timed(linears, steps, warmup, vanilla=True, side=side)
    log("bench: config %d: averis %s | vanilla %s (ms/step)" % (
        cfg, " ".join("%s %.4f" % kv for kv in ta_ms.items()),
        " ".join("%s %.4f" % kv for kv in tv_ms.items())))
    flops_step = sum(2 * L.flops() for L in linears)
    per = {}
    tot = {"averis": {}, "vanilla": {}}
    for L in linears:
        rec = {}
        for arm, t in (("averis", ta), ("vanilla", tv)):
            r = {k: stats(t.ms(L.name + "/" + k))
                 for k in ("wquant", "split_x", "gemm_fwd", "split_d", "gemm_dgrad")
                 if t.ms(L.name + "/" + k)}
            for k, v in r.items():
                tot[arm][k] = tot[arm].get(k, 0.0) + v["ms"]
            rec[arm] = r
        a, v = rec["averis"], rec["vanilla"]
        fa = a["split_x"]["ms"] + a["gemm_fwd"]["ms"]
        fv = v["split_x"]["ms"] + v["gemm_fwd"]["ms"]
        ba = a["split_d"]["ms"] + a["gemm_dgrad"]["ms"]
        bv = v["split_d"]["ms"] + v["gemm_dgrad"]["ms"]
        sqx = L.l * L.m * SQ_BYTES_PER_ELEM
        sqd = L.l * L.n * SQ_BYTES_PER_ELEM
        per[L.name] = dict(
            shape=dict(tokens=L.l, k_in=L.m, n_out=L.n, segments=L.nseg),
            averis={k: vv for k, vv in a.items()}, vanilla={k: vv for k, vv in v.items()},
            split_quant_gbs=dict(x=sqx / (a["split_x"]["ms"] * 1e-3) / 1e9,
                                 d=sqd / (a["split_d"]["ms"] * 1e-3) / 1e9),
            vanilla_quant_gbs=dict(x=sqx / (v["split_x"]["ms"] * 1e-3) / 1e9,
                                   d=sqd / (v["split_d"]["ms"] * 1e-3) / 1e9),
            gemm_tflops=dict(fwd=L.flops() / (a["gemm_fwd"]["ms"] * 1e-3) / 1e12,
                             dgrad=L.flops() / (a["gemm_dgrad"]["ms"] * 1e-3) / 1e12,
                             vanilla_fwd=L.flops() / (v["gemm_fwd"]["ms"] * 1e-3) / 1e12,
                             vanilla_dgrad=L.flops() / (v["gemm_dgrad"]["ms"] * 1e-3) / 1e12),
            overhead_pct=dict(fwd=100 * (fa / fv - 1), dgrad=100 * (ba / bv - 1)))
    for arm, t in (("averis", ta), ("vanilla", tv)):
        if t.ms("block/wquant"):
            tot[arm]["wquant"] = stats(t.ms("block/wquant"))["ms"]
    sq_x = sum(L.l * L.m for L in linears) * SQ_BYTES_PER_ELEM
    sq_d = sum(L.l * L.n for L in linears) * SQ_BYTES_PER_ELEM
    A, V = tot["averis"], tot["vanilla"]
    summary = dict(
        workload=WORKLOAD_NAMES[cfg],
        schedule=("each linear's dgrad split on a second stream, beside its forward pass"
                  if side is not None else "every op in order on the launch stream"),
        ms_per_step=ta_ms["queued"], vanilla_ms_per_step=tv_ms["queued"],
        step_p10_p90_ms=[ta_ms["queued_p10"], ta_ms["queued_p90"]],
        vanilla_step_p10_p90_ms=[tv_ms["queued_p10"], tv_ms["queued_p90"]],
        tflops=flops_step / (ta_ms["queued"] * 1e-3) / 1e12,
        vanilla_tflops=flops_step / (tv_ms["queued"] * 1e-3) / 1e12,
        step_ms_by_launch={"averis": ta_ms, "vanilla": tv_ms},
        overhead_pct=dict(
            step=100 * (ta_ms["queued"] / tv_ms["queued"] - 1),
            fwd=100 * ((A["split_x"] + A["gemm_fwd"]) / (V["split_x"] + V["gemm_fwd"]) - 1),
            dgrad=100 * ((A["split_d"] + A["gemm_dgrad"]) / (V["split_d"] + V["gemm_dgrad"]) - 1)),
        split_quant=dict(
            x=dict(ms=A["split_x"], gbs=sq_x / (A["split_x"] * 1e-3) / 1e9),
            d=dict(ms=A["split_d"], gbs=sq_d / (A["split_d"] * 1e-3) / 1e9)),
        vanilla_quant=dict(
            x=dict(ms=V["split_x"], gbs=sq_x / (V["split_x"] * 1e-3) / 1e9),
            d=dict(ms=V["split_d"], gbs=sq_d / (V["split_d"] * 1e-3) / 1e9)),
        gemm=dict(fwd_ms=A["gemm_fwd"], dgrad_ms=A["gemm_dgrad"],
                  tflops=flops_step / ((A["gemm_fwd"] + A["gemm_dgrad"]) * 1e-3) / 1e12,
                  vanilla_tflops=flops_step / ((V["gemm_fwd"] + V["gemm_dgrad"]) * 1e-3) / 1e12),
        weight_quant_ms=A["wquant"],
        weight_quant_calls="one call for all weights (averis_quant_pair_multi)"
        if block_weights(linears) else "one call per weight (averis_quant_pair)",
        per_linear=per,
        rotating_input_copies=copies,
        sum_of_calls_ms=dict(averis=sum(A.values()), vanilla=sum(V.values())),
    )
    for s in (summary["split_quant"], summary["vanilla_quant"]):
        for v in s.values():
            v["frac_hbm"] = v["gbs"] / HBM_PEAK_GBS
    if block_weights(linears):
        summary["block_weight_copies"] = time_block_weight_copies(linears, steps, warmup)
    if any(L.share_src is not None for L in linears):
        # the same step with each shared input split (or quantized) once: k
        # and v reuse q's, up reuses gate's; the one split forms the rank-one
        # rows of all the GEMMs that take it
        sa, _ = timed(linears, steps, warmup, vanilla=False, shared=True, per_call=False,
                      side=side)
        sv, _ = timed(linears, steps, warmup, vanilla=True, shared=True, per_call=False,
                      side=side)
        log("bench: config %d, shared inputs: averis %.4f | vanilla %.4f (ms/step)"
            % (cfg, sa["queued"], sv["queued"]))
        summary["shared_input_once"] = dict(
            shared={L.name: L.share_src.name for L in linears if L.share_src is not None},
            ms_per_step=sa["queued"], vanilla_ms_per_step=sv["queued"],
            step_p10_p90_ms=[sa["queued_p10"], sa["queued_p90"]],
            vanilla_step_p10_p90_ms=[sv["queued_p10"], sv["queued_p90"]],
            tflops=flops_step / (sa["queued"] * 1e-3) / 1e12,
            vanilla_tflops=flops_step / (sv["queued"] * 1e-3) / 1e12,
            overhead_pct=100 * (sa["queued"] / sv["queued"] - 1),
            step_ms_by_launch={"averis": sa, "vanilla": sv})
    return summary, ta, flops_step


def time_wgrad(L, steps, warmup):
    """The wgrad pieces of one linear, queued behind a spin kernel and timed
    per call by events on the launch stream, rotating through the input
    copies: the transposed residual quants of X and D (their means and
    residual tensor scales come from the splits the forward and dgrad passes
    run) and dW = deq(xt) deq(dt)^T + l mu_X mu_D^T (fp32 out)."""
    l, m, n = L.l, L.m, L.n
    xr, _, mx = av.averis_split_quant(L.xs[0], seed=0, ws=L.ws["sq_x"])
    dr, _, md = av.averis_split_quant(L.ds[0], seed=1, ws=L.ws["sq_d"])
    xt = av.NVFP4.empty(m, l, 1, L.x0.device)
    dt = av.NVFP4.empty(n, l, 1, L.x0.device)
    dw = torch.empty((m, n), dtype=torch.float32, device=L.x0.device)
    wws = torch.empty(av.workspace_bytes(av.OP_WGRAD, m, l, n), dtype=torch.uint8,
                      device=L.x0.device)

    def one(i, t):
        t.start("rt_x")
        av.averis_residual_t_quant(L.xs[i % len(L.xs)], mx, xr, seed=0, out=xt)
        t.stop("rt_x")
        t.start("rt_d")
        av.averis_residual_t_quant(L.ds[i % len(L.ds)], md, dr, seed=1, out=dt)
        t.stop("rt_d")
        t.start("gemm_wgrad")
        av.averis_gemm_wgrad(xt, dt, mx, md, out=dw, ws=wws)
        t.stop("gemm_wgrad")

    for i in range(warmup):
        one(i, Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for i in range(steps):
        one(i, t)
    torch.cuda.synchronize()
    ms = {k: stats(t.ms(k)) for k in ("rt_x", "rt_d", "gemm_wgrad")}
    rt = lambda rows, cols, k: rows * cols * SQ_BYTES_PER_ELEM / (ms[k]["ms"] * 1e-3) / 1e9
    return dict(linear=L.name, tokens=l, m=m, n=n, ms=ms,
                rt_gbs={"x": rt(l, m, "rt_x"), "d": rt(l, n, "rt_d")},
                gemm_tflops=2.0 * l * m * n / (ms["gemm_wgrad"]["ms"] * 1e-3) / 1e12,
                note="dW (m x n) = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X mu_D^T, fp32 out; "
                     "gemm_wgrad covers the split-K GEMM and the reduce that adds the outer "
                     "product")


def time_ratio(L, steps, warmup):
    """Split-quant of X and D with and without the mean-energy ratio, per call
    (events on the launch stream, queued behind a spin kernel, rotating
    copies), and the ratios themselves."""
    ratios = {}

    def one(i, t):
        for name, src, key in (("x", L.xs, "sq_x"), ("d", L.ds, "sq_d")):
            a = src[i % len(src)]
            t.start("plain_" + name)
            av.averis_split_quant(a, seed=0, ws=L.ws[key])
            t.stop("plain_" + name)
            t.start("ratio_" + name)
            out = av.averis_split_quant_ratio(a, seed=0, ws=L.ws[key])
            t.stop("ratio_" + name)
            ratios[name] = out[3]

    for i in range(warmup):
        one(i, Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for i in range(steps):
        one(i, t)
    torch.cuda.synchronize()
    med = lambda v: float(np.median(v))
    return dict(linear=L.name, **{
        name: dict(split_ms=med(t.ms("plain_" + name)),
                   split_with_ratio_ms=med(t.ms("ratio_" + name)),
                   ratio=float(ratios[name][0].item()))
        for name in ("x", "d")})


def time_fused_statistics(L, steps, warmup):
    """Column statistics fused into the producer, on one linear: the forward
    GEMM with and without writing the statistics of its bf16 output Y, and
    the split of Y with its own statistics pass (two reads of Y) and from the
    GEMM's statistics (one read), per call (events on the launch stream,
    queued behind a spin kernel)."""
    x = L.xs[0]
    wt, _ = av.averis_quant_pair(L.w, rnd=av.RN)
    xr, _, _, rho = av.averis_split_quant_rank1(x, wt, seed=0)
    y = torch.empty((L.l, L.n), dtype=torch.bfloat16, device=x.device)
    wsy = torch.empty(av.workspace_bytes(av.OP_SPLIT_QUANT, L.l, L.n), dtype=torch.uint8,
                      device=x.device)

    def one(t):
        t.start("gemm")
        av.averis_gemm_rank1(xr, rho, wt, out_dtype=torch.bfloat16, out=y)
        t.stop("gemm")
        t.start("split_two_reads")
        av.averis_split_quant(y, seed=2, ws=wsy)
        t.stop("split_two_reads")
        t.start("gemm_with_stats")
        av.averis_gemm_rank1_stats(xr, rho, wt, ws=wsy, out=y)
        t.stop("gemm_with_stats")
        t.start("split_one_read")
        av.averis_split_quant_from_stats(y, wsy, seed=2)
        t.stop("split_one_read")

    for _ in range(warmup):
        one(Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for _ in range(steps):
        one(t)
    torch.cuda.synchronize()
    ms = {k: stats(t.ms(k)) for k in ("gemm", "gemm_with_stats", "split_two_reads",
                                      "split_one_read")}
    sq = L.l * L.n * SQ_BYTES_PER_ELEM
    return dict(linear=L.name, y_shape=[L.l, L.n], ms=ms,
                split_gbs={"two_reads": sq / (ms["split_two_reads"]["ms"] * 1e-3) / 1e9,
                           "one_read": sq / (ms["split_one_read"]["ms"] * 1e-3) / 1e9},
                producer_plus_split_ms={
                    "separate": ms["gemm"]["ms"] + ms["split_two_reads"]["ms"],
                    "fused": ms["gemm_with_stats"]["ms"] + ms["split_one_read"]["ms"]})


def time_block_weight_copies(linears, steps, warmup):
    """Both copies of every weight of a block: one averis_quant_pair_multi call
    against one averis_quant_pair call per weight (events on the launch
    stream, queued behind a spin kernel)."""
    def one(t):
        t.start("multi")
        av.averis_quant_pair_multi([L.w for L in linears], rnd=av.RN, ws=linears[0].ws["qm"])
        t.stop("multi")
        t.start("per_weight")
        for L in linears:
            av.averis_quant_pair(L.w, rnd=av.RN, ws=L.ws["q"])
        t.stop("per_weight")

    for _ in range(warmup):
        one(Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.5 * steps)
    for _ in range(steps):
        one(t)
    torch.cuda.synchronize()
    return dict(multi_ms=float(np.median(t.ms("multi"))),
                per_weight_calls_ms=float(np.median(t.ms("per_weight"))))


def time_weight_copies(L, steps, warmup):
    """Both weight copies per call (events on the launch stream, queued behind
    a spin kernel): the two 1-D quantizations (averis_quant_pair) and the
    shared 16x16-tile quantization (averis_quant_pair_2d)."""
    def one(t):
        t.start("pair")
        av.averis_quant_pair(L.w, rnd=av.RN, ws=L.ws["q"])
        t.stop("pair")
        t.start("pair_2d")
        av.averis_quant_pair_2d(L.w, rnd=av.RN, ws=L.ws["q"])
        t.stop("pair_2d")

    for _ in range(warmup):
        one(Timer())
    torch.cuda.synchronize()
    t = Timer()
    hold_gpu(5.0 + 0.2 * steps)
    for _ in range(steps):
        one(t)
    torch.cuda.synchronize()
    return dict(linear=L.name, pair_ms=float(np.median(t.ms("pair"))),
                pair_2d_ms=float(np.median(t.ms("pair_2d"))))


# --------------------------------------------------------------------------
# the oracle on the host (reported baseline)
# --------------------------------------------------------------------------

def cpu_baseline(cfg, rows):
    """The oracle as it stands on a bounded sample of the headline workload:
    `rows` tokens of every linear (all other sizes as in the workload):
    split-quant of X and D, both weight copies, the float64 forward and dgrad
    GEMMs.  Reported in TFLOP/s of the sample's GEMMs."""
    from oracle import averis as orc
    if cfg == 4:
        cases = [workloads.block_linear(name, l=rows) for name in workloads.QWEN3_06B_LINEARS]
    elif cfg == 1:
        cases = [workloads.up_proj(l=rows)]
    elif cfg == 2:
        cases = [workloads.down_proj(l=rows)]
    else:
        raise ValueError("the CPU sample covers the dense workloads")
    flops = 0.0
    t0 = time.perf_counter()
    for c in cases:
        x, w, d = c["x"].float().numpy(), c["w"].float().numpy(), c["d"].float().numpy()
        wq = orc.weight_quant(w, "rn")
        orc.averis_forward(x, wq["fwd"], "sr", 0)
        orc.averis_dgrad(d, wq["dgrad"], "sr", 1)
        flops += 2 * 2.0 * x.shape[0] * x.shape[1] * d.shape[1]
    dt = time.perf_counter() - t0
    try:
        import threadpoolctl
        blas = max(i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()) or 1
    except Exception:
        blas = 1
    return dict(value=flops / dt / 1e12, unit="TFLOP/s", cores=int(blas), kind="oracle",
                sample="%d tokens of each of the %d linear(s) of the headline workload (full "
                       "weights), one step: split-quant X and D, both weight copies, float64 "
                       "fwd+dgrad GEMMs; %.1f s; numpy elementwise work single-threaded, float64 "
                       "matmul on %d BLAS threads of %d host cores"
                       % (rows, len(cases), dt, blas, len(os.sched_getaffinity(0))),
                seconds=dt)


# --------------------------------------------------------------------------
# HBM counters (rocprofv3 --pmc) and the roofline record
# --------------------------------------------------------------------------

COPY_BYTES = 256 << 20


def traffic_probe(args):
    """A device copy of known size (the scale reference for the HBM byte
    counters) followed by three Averis steps of the headline config."""
    src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device="cuda").fill_(1.0)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    linears = make_linears(args.config)
    torch.cuda.synchronize()
    for i in range(3):
        run_step(linears, 0, None, vanilla=False)
    torch.cuda.synchronize()
    print("traffic probe done: copy %d bytes, config %d" % (COPY_BYTES, args.config),
          file=sys.stderr)


GEMM_SOURCES = ["gemm.hip", "gemm_ws.hip", "gemm_win.hip", "gemm_common.hpp"]


def gemm_source_sha():
    """One hash over the sources of the GEMM kernel."""
    import hashlib
    h = hashlib.sha256()
    for f in GEMM_SOURCES:
        h.update(open(os.path.join(ROOT, "mean_residual_quantized_amd", "csrc", f), "rb").read())
    return h.hexdigest()


def load_traffic(cfg):
    """HBM bytes per Averis GEMM launch (k_gemm_win) from the committed counter
    summary, if it was taken on the current kernel sources for this workload
    (else None)."""
    path = os.path.join(ROOT, "profiles", "gemm_traffic.json")
    try:
        rec = json.load(open(path))
        sha = gemm_source_sha()
    except (OSError, ValueError):
        return None
    if rec.get("gemm_sources_sha256") != sha or rec.get("config") != cfg:
        return None
    return rec


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: libaveris has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(2)
    av.lib()
    if args.traffic_probe:
        traffic_probe(args)
        return
    cfg = args.config
    log("bench: generating config %d" % cfg)
    linears = make_linears(cfg)
    head, ta, flops_step = measure(cfg, linears, args.steps, args.warmup, args.streams)

    # roofline of the dominant kernel: k_gemm_win, the Averis GEMM (the
    # NVFP4 NT GEMM with the codes staged in LDS, adding the split's rank-one
    # row), over
    # all of its launches in a step: mean flops per launch / mean launch time
    # (events around each call on the launch stream)
    g_calls = [(L, k) for L in linears for k in ("gemm_fwd", "gemm_dgrad")]
    g_ms = sum(float(np.mean(ta.ms(L.name + "/" + k))) for L, k in g_calls)
    nlaunch = len(g_calls)
    achieved = (flops_step / nlaunch) / (g_ms / nlaunch * 1e-3) / 1e12
    tr = load_traffic(cfg)
    traffic = None if tr is None else tr["averis_gemm"]["bytes_per_launch"]
    roofline = dict(bound="mfma", achieved=achieved, peak=F16_MFMA_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=achieved / F16_MFMA_PEAK_TFLOPS, traffic=traffic,
                    kernel="k_gemm_win (averis_gemm_rank1: NVFP4 NT GEMM, 4-bit codes staged in LDS, "
                           "exact fp16 dequant by the MFMA waves -> v_mfma_f32_32x32x16_f16, the "
                           "rank-one row from the "
                           "split added in the epilogue, bf16 out), all %d launches of one step "
                           "(forward and dgrad of every linear)" % nlaunch,
                    launches_per_step=nlaunch, mean_flops_per_launch=flops_step / nlaunch,
                    mean_launch_ms=g_ms / nlaunch,
                    frac_of_fp4_peak=achieved / FP4_MFMA_PEAK_TFLOPS)

    out = {
        "metric": METRIC,
        "value": head["tflops"],
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "nvfp4 (e2m1 + e4m3 scales) operands, f16 MFMA, f32 accumulate",
        "data": "synthetic",
        "config": {"workload": head["workload"], "config_id": cfg,
                   "linears": {L.name: [L.l, L.m, L.n] for L in linears},
                   "input_dtype": "bf16", "sr": "philox4x32-10, 16 bits"},
        "roofline": roofline,
        "headline": head,
        "pages_overhead_context": "2.20% end-to-end over vanilla NVFP4 (hardware not stated)",
    }
    if not args.only_headline:
        others = {}
        for c in (1, 2, 3, 4):
            if c == cfg:
                continue
            for L in linears:
                L.xs, L.ds = [], []
            del linears
            torch.cuda.empty_cache()
            log("bench: generating config %d" % c)
            linears = make_linears(c)
            others[str(c)] = measure(c, linears, args.steps, args.warmup, args.streams)[0]
        out["other_configs"] = others
        # the (f) rows on one linear of the headline workload
        for L in linears:
            L.xs, L.ds = [], []
        del linears
        torch.cuda.empty_cache()
        if cfg == 4:
            c = workloads.block_linear("up")
        elif cfg == 2:
            c = workloads.down_proj()
        else:
            c = workloads.up_proj()
        L = Linear("up" if cfg == 4 else "down_proj" if cfg == 2 else "up_proj",
                   c["x"], c["w"], c["d"])
        act = L.act_bytes()
        L.rotate(max(1, int(np.ceil(ROTATE_BYTES / act))))
        log("bench: wgrad, mean-energy ratio and weight copies on %s" % L.name)
        out["wgrad"] = time_wgrad(L, args.steps, args.warmup)
        out["mean_energy_ratio"] = time_ratio(L, args.steps, args.warmup)
        out["weight_copies"] = time_weight_copies(L, args.steps, args.warmup)
        out["fused_statistics"] = time_fused_statistics(L, args.steps, args.warmup)
    if not args.no_cpu_baseline and cfg != 3:
        log("bench: timing the oracle on the host (bounded sample)")
        out["cpu_baseline"] = cpu_baseline(cfg, args.cpu_rows)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
