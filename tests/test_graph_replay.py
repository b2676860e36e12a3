"""The whole forward + dgrad step captured in one HIP graph and replayed.

Every launch of the library is a plain kernel launch on the caller's stream
(no allocation, copy or memset inside), so a captured step must reproduce the
eager step bit for bit on every replay, also with other eager work and
synchronizations between the replays.  The eager path itself is checked
against the oracle in test_gpu_parity.py."""

import pytest
import torch

from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def step(x, w, d, vanilla, rank1=False, shared=False):
    pair = av.averis_quant_pair_2d if shared else av.averis_quant_pair
    wt, wd = pair(w, rnd=av.RN)
    if rank1:
        xr, xm, xmu, rx = av.averis_split_quant_rank1(x, wt, seed=0)
        y = av.averis_gemm_rank1(xr, rx, wt, out_dtype=torch.bfloat16)
        dr, dm, dmu, rd = av.averis_split_quant_rank1(d, wd, seed=1)
        dx = av.averis_gemm_rank1(dr, rd, wd, out_dtype=torch.bfloat16)
        quants = [wt, wd, xr, xm, dr, dm]
        extra = [xmu, dmu, rx, rd]
    elif vanilla:
        xq = av.averis_quant(x, seed=0)
        dq = av.averis_quant(d, seed=1)
        y = av.averis_gemm_vanilla(xq, wt, out_dtype=torch.bfloat16)
        dx = av.averis_gemm_vanilla(dq, wd, out_dtype=torch.bfloat16)
        quants = [wt, wd, xq, dq]
        extra = []
    else:
        xr, xm, xmu = av.averis_split_quant(x, seed=0)
        y = av.averis_gemm_fwd(xr, xm, wt, out_dtype=torch.bfloat16)
        dr, dm, dmu = av.averis_split_quant(d, seed=1)
        dx = av.averis_gemm_dgrad(dr, dm, wd, out_dtype=torch.bfloat16)
        quants = [wt, wd, xr, xm, dr, dm]
        extra = [xmu, dmu]
    flat = [t for q in quants for t in (q.codes, q.scales, q.tscale)]
    return flat + extra + [y, dx]


@pytest.mark.parametrize("mode", ["fused", "rank1", "vanilla", "rank1_shared_weight"])
@pytest.mark.parametrize("l,m,n", [(1000, 320, 192), (8192, 1024, 3072)])
def test_graph_replays_match_eager(l, m, n, mode):
    cfg = workloads.up_proj(l=l, m=m, n=n)
    x, w, d = cfg["x"].cuda(), cfg["w"].cuda(), cfg["d"].cuda()
    vanilla, rank1 = mode == "vanilla", mode.startswith("rank1")
    shared = mode == "rank1_shared_weight"
    ref = [t.clone() for t in step(x, w, d, vanilla, rank1, shared)]
    torch.cuda.synchronize()

    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step(x, w, d, vanilla, rank1, shared)
    torch.cuda.synchronize()

    other = workloads.up_proj(l=256, m=m, n=n)["x"].cuda()
    for rep in range(3):
        # eager work of the program's own between replays
        av.averis_split_quant(other, seed=rep)
        torch.cuda.synchronize()
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager step" % (rep, i)
    del g
    torch.cuda.synchronize()


@pytest.mark.parametrize("vanilla", [False, True])
def test_two_stream_step_replays_match_eager(vanilla):
    """The step with the dgrad split on a second stream (forked from and
    joined back to the capturing stream by events, its outputs preallocated):
    each replay equals the one-stream eager step bit for bit."""
    cfg = workloads.up_proj(l=2048, m=1024, n=3072)
    x, w, d = cfg["x"].cuda(), cfg["w"].cuda(), cfg["d"].cuda()
    rank1 = not vanilla
    ref = [t.clone() for t in step(x, w, d, vanilla, rank1)]
    side = torch.cuda.Stream()
    l, n = d.shape
    d_res, d_mean = av.NVFP4.empty(l, n), av.NVFP4.empty(1, n)
    d_mu = torch.empty((n,), dtype=torch.float32, device="cuda")
    d_rho = torch.empty((w.shape[0],), dtype=torch.float32, device="cuda")
    d_q = av.NVFP4.empty(l, n)

    def step2():
        wt, wd = av.averis_quant_pair(w, rnd=av.RN)
        fork = torch.cuda.Event()
        fork.record()
        side.wait_event(fork)
        with torch.cuda.stream(side):
            if vanilla:
                dq, rd = av.averis_quant(d, seed=1, out=d_q), None
            else:
                dq, _, _, rd = av.averis_split_quant_rank1(d, wd, seed=1, rho=d_rho,
                                                           out=(d_res, d_mean, d_mu))
            join = torch.cuda.Event()
            join.record()
        if vanilla:
            xq = av.averis_quant(x, seed=0)
            y = av.averis_gemm_vanilla(xq, wt, out_dtype=torch.bfloat16)
            quants, extra = [wt, wd, xq], []
        else:
            xr, xm, xmu, rx = av.averis_split_quant_rank1(x, wt, seed=0)
            y = av.averis_gemm_rank1(xr, rx, wt, out_dtype=torch.bfloat16)
            quants, extra = [wt, wd, xr, xm], [xmu, rx]
        torch.cuda.current_stream().wait_event(join)
        if vanilla:
            dx = av.averis_gemm_vanilla(dq, wd, out_dtype=torch.bfloat16)
            quants, extra = quants + [dq], extra
        else:
            dx = av.averis_gemm_rank1(dq, rd, wd, out_dtype=torch.bfloat16)
            quants, extra = quants + [dq, d_mean], extra + [d_mu, rd]
        flat = [t for q in quants for t in (q.codes, q.scales, q.tscale)]
        return flat + extra + [y, dx]

    eager2 = [t.clone() for t in step2()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = step2()
    torch.cuda.synchronize()
    # step lists [wt, wd, xq, dq] (vanilla) or [wt, wd, xr, xm, dr, dm] and
    # [xmu, dmu, rx, rd]; step2 the same quantized tensors and [xmu, rx, dmu, rd]
    if vanilla:
        order = list(range(12)) + [12, 13]
    else:
        order = list(range(18)) + [18, 20, 19, 21] + [22, 23]
    mapped = [eager2[i] for i in order]
    assert len(mapped) == len(ref)
    for i, (a, b) in enumerate(zip(mapped, ref)):
        assert torch.equal(a, b), "two-stream eager output %d differs from the one-stream step" % i
    for rep in range(3):
        av.averis_split_quant(workloads.up_proj(l=256, m=1024, n=3072)["x"].cuda(), seed=rep)
        torch.cuda.synchronize()
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, eager2)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager step" % (rep, i)
    del g
    torch.cuda.synchronize()


def test_wgrad_graph_replays_match_eager():
    # the transposed residual quants and the split-K wgrad (partials + reduce)
    cfg = workloads.up_proj(l=2048, m=320, n=192)
    x, d = cfg["x"].cuda(), cfg["d"].cuda()
    xr, _, mx = av.averis_split_quant(x, seed=0)
    dr, _, md = av.averis_split_quant(d, seed=1)

    def wstep():
        xt = av.averis_residual_t_quant(x, mx, xr, seed=0)
        dt = av.averis_residual_t_quant(d, md, dr, seed=1)
        dw = av.averis_gemm_wgrad(xt, dt, mx, md)
        return [xt.codes, xt.scales, xt.tscale, dt.codes, dt.scales, dt.tscale, dw]

    ref = [t.clone() for t in wstep()]
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        outs = wstep()
    torch.cuda.synchronize()
    for rep in range(3):
        av.averis_split_quant(workloads.up_proj(l=256, m=320, n=192)["x"].cuda(), seed=rep)
        torch.cuda.synchronize()
        for t in outs:
            t.zero_()
        g.replay()
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(outs, ref)):
            assert torch.equal(a, b), "replay %d, output %d differs from the eager step" % (rep, i)
    del g
    torch.cuda.synchronize()
