"""Full-size parity at the block-sweep and MoE configurations, on sampled
rows: the Qwen3-0.6B-like block of seven linears at l = 16384 tokens through
the timed path (split-quant with the rank-one row, GEMM adding it, bf16
output), and the 64-expert grouped case (32768 routed rows) through the
grouped entry points.  Means, tensor scales, mean codes and weight copies are
compared whole; residual codes on sampled row ranges (the oracle quantizes
only those, with the tensor-wide amax); GEMM outputs on the same rows within
1e-3 of the bound (plus bf16 rounding of the output)."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu

TOL = 1e-3
BF16_REL = 2.0 ** -8


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def f32(t):
    return t.float().cpu().numpy()


def same(gpu_q, ref, rows=None, seg=0):
    g = gpu_q.cpu()
    codes, scales = g["codes"], g["scales"]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(scales, ref["scales"])
    assert g["tscale"][2 * seg] == ref["s_enc"] and g["tscale"][2 * seg + 1] == ref["s_dec"]


def close(c_rows, ref, bound, bf16):
    c = c_rows.astype(np.float64)
    err = np.abs(c - ref)
    ok = err <= TOL * bound + (BF16_REL * np.abs(ref) if bf16 else 0.0)
    assert ok.all(), "max normalised error %.3g" % np.max(err / np.maximum(bound, 1e-300))


@pytest.mark.parametrize("name", list(workloads.QWEN3_06B_LINEARS))
def test_block_linear_sampled(name):
    cfg = workloads.block_linear(name)
    x, w, d = cfg["x"], cfg["w"], cfg["d"]
    l = x.shape[0]
    seed = list(workloads.QWEN3_06B_LINEARS).index(name)
    print("block linear %s: l=%d, %s -> %s" % (name, l, x.shape[1], d.shape[1]), flush=True)
    wt, wd = av.averis_quant_pair(w.cuda(), rnd=av.RN)
    wq = orc.weight_quant(f32(w), "rn")
    same(wt, wq["fwd"])
    same(wd, wq["dgrad"])
    ranges = [(0, 16), (l // 2 + 5, l // 2 + 21), (l - 16, l)]
    for a, b, b_ref, s in ((x, wt, wq["fwd"], seed), (d, wd, wq["dgrad"], seed + 100)):
        res, mean, mu, rho = av.averis_split_quant_rank1(a.cuda(), b, seed=s)
        c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.bfloat16)
        an = f32(a)
        mu_ref = orc.column_mean(an)
        np.testing.assert_array_equal(mu.cpu().numpy(), mu_ref)
        amax = np.max(np.abs(orc.residual(an, mu_ref)))
        mean_ref = orc.quantize(mu_ref[None, :], "sr", s, stream=1)
        same(mean, mean_ref)
        m_deq, b_deq = orc.dequantize(mean_ref)[0], orc.dequantize(b_ref)
        err = np.abs(rho.cpu().numpy() - b_deq @ m_deq)
        assert (err <= TOL * (np.abs(b_deq) @ np.abs(m_deq))).all()
        cc = c.float().cpu().numpy()
        rho_ref = m_deq @ b_deq.T
        for r0, r1 in ranges:
            q = orc.quantize(orc.residual(an[r0:r1], mu_ref), "sr", s, stream=0, row0=r0, amax=amax)
            same(res, q, rows=slice(r0, r1))
            a_deq = orc.dequantize(q)
            ref = a_deq @ b_deq.T + rho_ref[None, :]
            bound = np.abs(a_deq) @ np.abs(b_deq).T + (np.abs(m_deq) @ np.abs(b_deq).T)[None, :]
            close(cc[r0:r1], ref, bound, bf16=True)
    torch.cuda.synchronize()


def test_moe_full_size_sampled():
    cfg = workloads.moe()       # 4096 tokens x top-8 over 64 experts, hidden 2048, inter 768
    x, w, d, offs = cfg["x"], cfg["w"], cfg["d"], cfg["offsets"]
    nseg = len(offs) - 1
    print("the MoE case: %d rows, %d experts" % (x.shape[0], nseg), flush=True)
    og = torch.from_numpy(offs).cuda()
    counts = np.diff(offs)
    live = [e for e in range(nseg) if counts[e] > 0]
    picks = sorted({live[0], live[len(live) // 2], live[-1]})
    wg = w.cuda()
    for a, transpose, s in ((x, True, 7), (d, False, 8)):
        res, mean, mu = av.averis_split_quant_grouped(a.cuda(), og, seed=s)
        bq = av.averis_quant_batched(wg, transpose=transpose)
        c = av.averis_gemm_grouped(res, mean, bq, og, out_dtype=torch.bfloat16)
        an = f32(a)
        mu_g = mu.cpu().numpy()
        cc = c.float().cpu().numpy()
        n = bq.rows // nseg
        for e in range(nseg):
            r0, r1 = int(offs[e]), int(offs[e + 1])
            mu_ref = orc.column_mean(an[r0:r1]) if r1 > r0 else np.zeros(an.shape[1], np.float32)
            np.testing.assert_array_equal(mu_g[e], mu_ref)
            if e not in picks:
                continue
            r = orc.residual(an[r0:r1], mu_ref)
            amax = np.max(np.abs(r))
            mean_ref = orc.quantize(mu_ref[None, :], "sr", s, stream=1, row0=e)
            same(mean, mean_ref, rows=slice(e, e + 1), seg=e)
            wsrc = f32(w[e])
            b_ref = orc.weight_quant(wsrc, "rn")["fwd" if transpose else "dgrad"]
            same(bq, b_ref, rows=slice(e * n, (e + 1) * n), seg=e)
            t0, t1 = r0, min(r1, r0 + 16)
            q = orc.quantize(r[t0 - r0:t1 - r0], "sr", s, stream=0, row0=t0, amax=amax)
            same(res, q, rows=slice(t0, t1), seg=e)
            a_deq, b_deq = orc.dequantize(q), orc.dequantize(b_ref)
            m_deq = orc.dequantize(mean_ref)[0]
            ref = a_deq @ b_deq.T + (m_deq @ b_deq.T)[None, :]
            bound = np.abs(a_deq) @ np.abs(b_deq).T + (np.abs(m_deq) @ np.abs(b_deq).T)[None, :]
            close(cc[t0:t1], ref, bound, bf16=True)
    torch.cuda.synchronize()
