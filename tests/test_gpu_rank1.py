"""GPU parity of the rank-one row formed by the split (averis_split_quant_rank1)
and of the GEMM that adds it (averis_gemm_rank1): the split's outputs are
bit for bit those of averis_split_quant; rho = deq(mean) deq(B)^T and
C = deq(A_R) deq(B)^T + 1 rho^T are within 1e-3 of their bounds against the
oracle's float64 values from its own quantized operands."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from tests.parity import assert_gemm_close
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def check(a, w, which, seed=0, rnd="sr", out_dtype=torch.float32):
    """which = 'x' (forward: b = Q4(W^T)) or 'd' (dgrad: b = Q4(W))."""
    r = av.SR if rnd == "sr" else av.RN
    ag, wg = a.cuda(), w.cuda()
    b = av.averis_quant(wg, transpose=(which == "x"), rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    res, mean, mu, rho = av.averis_split_quant_rank1(ag, b, seed=seed, rnd=r)
    r2, m2, mu2 = av.averis_split_quant(ag, seed=seed, rnd=r)
    for x, y in ((res, r2), (mean, m2)):
        for t in ("codes", "scales", "tscale"):
            assert torch.equal(getattr(x, t), getattr(y, t)), t
    assert torch.equal(mu, mu2)
    wq = orc.weight_quant(w.float().numpy(), "rn")
    b_ref = wq["fwd"] if which == "x" else wq["dgrad"]
    s = orc.split_quant(a.float().numpy(), rnd, seed)
    m_deq, b_deq = orc.dequantize(s["mean"])[0], orc.dequantize(b_ref)
    rho_ref = b_deq @ m_deq
    rho_bound = np.abs(b_deq) @ np.abs(m_deq)
    err = np.abs(rho.cpu().numpy().astype(np.float64) - rho_ref)
    assert (err <= TOL * rho_bound + 1e-30).all(), np.max(err / np.maximum(rho_bound, 1e-300))
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=out_dtype)
    ref = orc.gemm(s["residual"], b_ref, s["mean"])
    bound = orc.gemm_abs_bound(s["residual"], b_ref, s["mean"])
    extra = 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0
    cc = c.float().cpu().numpy().astype(np.float64)
    assert_gemm_close(cc, ref, bound, bf16=out_dtype == torch.bfloat16)
    # the same product as the GEMM that sums the rank-one row itself
    fn = av.averis_gemm_fwd if which == "x" else av.averis_gemm_dgrad
    c2 = fn(res, mean, b, out_dtype=torch.float32).cpu().numpy().astype(np.float64)
    assert (np.abs(c2 - cc) <= 2 * TOL * bound + extra * np.abs(ref)).all()
    torch.cuda.synchronize()


@pytest.mark.parametrize("which", ["x", "d"])
def test_tiny(which):
    cfg = workloads.tiny()
    check(cfg[which], cfg["w"], which)


@pytest.mark.parametrize("which", ["x", "d"])
@pytest.mark.parametrize("l,m,n", [
    (2048, 320, 192),    # K % 256 != 0 (per-stage scale loads), ragged tiles
    (1000, 256, 208),    # K % 256 == 0, ragged rows
    (300, 208, 96),      # K % 64 != 0: the general kernel
])
def test_shapes(l, m, n, which):
    cfg = workloads.up_proj(l=l, m=m, n=n)
    check(cfg[which], cfg["w"], which, seed=l)


def test_round_to_nearest_and_bf16_output():
    cfg = workloads.up_proj(l=1024, m=512, n=384)
    check(cfg["x"], cfg["w"], "x", rnd="rn", out_dtype=torch.bfloat16)


@pytest.mark.parametrize("which", ["x", "d"])
def test_full_size_up_proj(which):
    # up-proj: forward K = 1024 (256 x 192 tiles, two rounds), dgrad K = 3072;
    # rho exact against the oracle; the GEMM against the fused-mean GEMM
    cfg = workloads.up_proj()
    a, w = cfg[which], cfg["w"]
    ag = a.cuda()
    b = av.averis_quant(w.cuda(), transpose=(which == "x"), rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    res, mean, mu, rho = av.averis_split_quant_rank1(ag, b)
    r2, m2, _ = av.averis_split_quant(ag)
    assert torch.equal(res.codes, r2.codes) and torch.equal(mean.codes, m2.codes)
    an = a.float().numpy()
    mu_ref = orc.column_mean(an)
    m_deq = orc.dequantize(orc.quantize(mu_ref[None, :], "sr", 0, stream=1))[0]
    wq = orc.weight_quant(w.float().numpy(), "rn")
    b_deq = orc.dequantize(wq["fwd"] if which == "x" else wq["dgrad"])
    err = np.abs(rho.cpu().numpy() - b_deq @ m_deq)
    assert (err <= TOL * (np.abs(b_deq) @ np.abs(m_deq))).all()
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.float32)
    fn = av.averis_gemm_fwd if which == "x" else av.averis_gemm_dgrad
    c2 = fn(res, mean, b, out_dtype=torch.float32)
    rel = ((c - c2).abs().max() / c2.abs().max()).item()
    assert rel < 1e-5, rel


@pytest.mark.parametrize("hidden,inter", [(128, 64), (208, 96)])
def test_grouped_with_an_empty_segment(hidden, inter):
    # per-expert rank-one rows; hidden 208 (K % 64 != 0) takes the general kernel
    cfg = workloads.moe(tokens=256, topk=8, experts=16, hidden=hidden, inter=inter)
    x, w, offs = cfg["x"], cfg["w"], np.array(cfg["offsets"], dtype=np.int64)
    x = torch.cat([x[:offs[2]], x[offs[3]:]])        # segment 2 empty
    offs[3:] -= offs[3] - offs[2]
    nseg = len(offs) - 1
    og = torch.from_numpy(offs).cuda()
    wt = av.averis_quant_batched(w.cuda(), transpose=True)
    res, mean, mu, rho = av.averis_split_quant_grouped_rank1(x.cuda(), og, wt, seed=5)
    r2, m2, mu2 = av.averis_split_quant_grouped(x.cuda(), og, seed=5)
    for a, b in ((res, r2), (mean, m2)):
        for t in ("codes", "scales", "tscale"):
            assert torch.equal(getattr(a, t), getattr(b, t)), t
    assert torch.equal(mu, mu2)
    c = av.averis_gemm_grouped_rank1(res, rho, wt, og)
    g = orc.split_quant_grouped(x.float().numpy(), offs, "sr", 5)
    wrefs = [orc.weight_quant(w[e].float().numpy(), "rn")["fwd"] for e in range(nseg)]
    n = w.shape[2]
    rho_c = rho.cpu().numpy().reshape(nseg, n)
    for s in range(nseg):
        m_deq, b_deq = orc.dequantize(g["mean"][s])[0], orc.dequantize(wrefs[s])
        err = np.abs(rho_c[s] - b_deq @ m_deq)
        assert (err <= TOL * (np.abs(b_deq) @ np.abs(m_deq)) + 1e-30).all(), s
    assert not rho_c[2].any()
    ref = orc.gemm_grouped(g["residual"], wrefs, g["mean"])
    bound = np.concatenate([orc.gemm_abs_bound(g["residual"][s], wrefs[s], g["mean"][s])
                            for s in range(nseg)])
    cc = c.cpu().numpy().astype(np.float64)
    assert_gemm_close(cc, ref, bound)
    torch.cuda.synchronize()


def test_no_tokens_gives_a_zero_row():
    x = torch.zeros((0, 128), dtype=torch.bfloat16, device="cuda")
    w = workloads.tiny()["w"].cuda()
    b = av.averis_quant(w, transpose=True, rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    res, mean, mu, rho = av.averis_split_quant_rank1(x, b)
    assert rho.shape == (64,) and not rho.any() and not mu.any()
    c = av.averis_gemm_rank1(res, rho, b)
    assert c.shape == (0, 64)


@pytest.mark.parametrize("l,m,n", [(1000, 256, 200), (512, 512, 384)])
def test_bf16_output_strides_and_ragged_columns(l, m, n):
    # the staged epilogue's element-wise stores (odd strides, ragged last tile)
    cfg = workloads.up_proj(l=l, m=m, n=n)
    ag, wg = cfg["x"].cuda(), cfg["w"].cuda()
    b = av.averis_quant(wg, transpose=True, rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    res, mean, mu, rho = av.averis_split_quant_rank1(ag, b, seed=3)
    ref = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.bfloat16)
    big = torch.full((l, n + 3), float("nan"), dtype=torch.bfloat16, device="cuda")
    out = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.bfloat16, out=big[:, 1:n + 1])
    assert torch.equal(out, ref)
    assert torch.isnan(big[:, 0]).all() and torch.isnan(big[:, n + 1:]).all()


@pytest.mark.parametrize("case", ["qkv", "four_small"])
def test_several_rank1_operands_in_one_split(case):
    """averis_split_quant_rank1_multi: the split and each operand's rank-one
    row are those of averis_split_quant_rank1 with that operand alone, bit for
    bit (q, k and v of a block at a ragged token count; four small operands
    with ragged row counts, the mean's columns not a multiple of 1024)."""
    g = np.random.default_rng(23)
    if case == "qkv":
        l, m, ns = 1000, 1024, (2048, 1024, 1024)
    else:
        l, m, ns = 300, 144, (16, 48, 32, 80)
    a = workloads.mean_biased_activation(np.random.default_rng(5), l, m).cuda()
    bs = []
    for i, n in enumerate(ns):
        w = torch.from_numpy((g.standard_normal((m, n)) * (i + 1) / np.sqrt(m)).astype(np.float32))
        bs.append(av.averis_quant(w.cuda(), transpose=True, rnd=av.RN, sr_stream=av.STREAM_WEIGHT))
    res, mean, mu, rhos = av.averis_split_quant_rank1_multi(a, bs, seed=3)
    for b, rho in zip(bs, rhos):
        r1, m1, mu1, rho1 = av.averis_split_quant_rank1(a, b, seed=3)
        for x, y in ((res, r1), (mean, m1)):
            for t in ("codes", "scales", "tscale"):
                assert torch.equal(getattr(x, t), getattr(y, t)), t
        assert torch.equal(mu, mu1)
        assert torch.equal(rho, rho1)
    torch.cuda.synchronize()
