"""Full-size parity at every workload, through the entry points and seeds the
benchmark times (split-quant forming the rank-one row, the GEMM adding it,
bf16 output; X with seed 0, D with seed 1).

* up-proj and down-proj (8192 tokens): the fp32 mean, every residual code and
  scale byte, the tensor scales, the mean codes, both weight copies, the
  rank-one row, and whole GEMM outputs -- the timed bf16 launch and fp32
  output of both GEMM paths -- against the oracle's float64 product.
* the vanilla arm at the up-proj size: every code and scale byte of plain
  Q4(X) and Q4(D), whole forward and dgrad outputs.
* the block sweep (seven linears at 16384 tokens) and the MoE case (32768
  routed rows over 64 experts): every byte of the split (per segment for
  MoE) and of the weight copy the GEMM takes; GEMM outputs on sampled rows.

The oracle's quantization runs over row blocks in worker processes
(tests/parity.py): each block is one oracle call with the tensor's amax and
its first global row, which is how a whole-tensor call treats those rows."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads
from tests.parity import GEMM_TOL, OraclePool, assert_gemm_close, assert_quant_equal

pytestmark = pytest.mark.gpu

SEED = {"x": 0, "d": 1}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


@pytest.fixture(scope="module")
def pool():
    p = OraclePool()
    yield p
    p.close()


def f32(t):
    return t.float().cpu().numpy()


def oracle_split(pool, an, seed, row0=0, mean_row=0):
    """mu, Q4(a - 1 mu) (stream 0), Q4(mu) (stream 1) of one segment."""
    mu = orc.column_mean(an)
    r = orc.residual(an, mu)
    res = pool.quantize(r, "sr", seed, 0, row0=row0)
    mean = orc.quantize(mu[None, :], "sr", seed, stream=1, row0=mean_row)
    return mu, res, mean


def check_rho(rho, mean_ref, b_ref):
    m_deq, b_deq = orc.dequantize(mean_ref)[0], orc.dequantize(b_ref)
    err = np.abs(np.asarray(rho, dtype=np.float64) - b_deq @ m_deq)
    assert (err <= GEMM_TOL * (np.abs(b_deq) @ np.abs(m_deq)) + 1e-30).all()


@pytest.mark.parametrize("which", ["x", "d"])
@pytest.mark.parametrize("cfg_name", ["up_proj", "down_proj"])
def test_dense_full_size(pool, cfg_name, which):
    cfg = getattr(workloads, cfg_name)()
    a, w = cfg[which], cfg["w"]
    seed = SEED[which]
    print("%s %s: %s, seed %d" % (cfg_name, which, tuple(a.shape), seed), flush=True)
    wt, wd = av.averis_quant_pair(w.cuda(), rnd=av.RN)
    wq = orc.weight_quant(f32(w), "rn")
    assert_quant_equal(wt, wq["fwd"])
    assert_quant_equal(wd, wq["dgrad"])
    b, b_ref = (wt, wq["fwd"]) if which == "x" else (wd, wq["dgrad"])
    res, mean, mu, rho = av.averis_split_quant_rank1(a.cuda(), b, seed=seed)
    mu_ref, res_ref, mean_ref = oracle_split(pool, f32(a), seed)
    np.testing.assert_array_equal(mu.cpu().numpy(), mu_ref)
    assert_quant_equal(res, res_ref)
    assert_quant_equal(mean, mean_ref)
    check_rho(rho.cpu().numpy(), mean_ref, b_ref)
    ref = orc.gemm(res_ref, b_ref, mean_ref)
    bound = orc.gemm_abs_bound(res_ref, b_ref, mean_ref)
    tag = "%s %s" % (cfg_name, which)
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.bfloat16)
    assert_gemm_close(c, ref, bound, bf16=True, label=tag + " rank-one GEMM, bf16")
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.float32)
    assert_gemm_close(c, ref, bound, label=tag + " rank-one GEMM, fp32")
    fn = av.averis_gemm_fwd if which == "x" else av.averis_gemm_dgrad
    c = fn(res, mean, b, out_dtype=torch.float32)
    assert_gemm_close(c, ref, bound, label=tag + " fused GEMM, fp32")
    torch.cuda.synchronize()


@pytest.mark.parametrize("which", ["x", "d"])
def test_vanilla_full_size_up_proj(pool, which):
    cfg = workloads.up_proj()
    a, w = cfg[which], cfg["w"]
    seed = SEED[which]
    print("vanilla up_proj %s: %s" % (which, tuple(a.shape)), flush=True)
    wt, wd = av.averis_quant_pair(w.cuda(), rnd=av.RN)
    wq = orc.weight_quant(f32(w), "rn")
    b, b_ref = (wt, wq["fwd"]) if which == "x" else (wd, wq["dgrad"])
    q = av.averis_quant(a.cuda(), seed=seed)
    q_ref = pool.quantize(f32(a), "sr", seed, 0)         # the oracle's vanilla_quant
    assert_quant_equal(q, q_ref)
    ref, bound = orc.gemm(q_ref, b_ref), orc.gemm_abs_bound(q_ref, b_ref)
    c = av.averis_gemm_vanilla(q, b, out_dtype=torch.float32)
    assert_gemm_close(c, ref, bound, label="vanilla %s fp32" % which)
    c = av.averis_gemm_vanilla(q, b, out_dtype=torch.bfloat16)
    assert_gemm_close(c, ref, bound, bf16=True, label="vanilla %s bf16" % which)
    torch.cuda.synchronize()


def sample_rows(l, n=8, width=16):
    starts = np.linspace(0, l - width, n).astype(np.int64)
    starts[3] += 5                      # one range not aligned to 16
    return [(int(s), int(s) + width) for s in starts]


@pytest.mark.parametrize("which", ["x", "d"])
@pytest.mark.parametrize("name", list(workloads.QWEN3_06B_LINEARS))
def test_block_linear_full_size(pool, name, which):
    cfg = workloads.block_linear(name)
    a, w = cfg[which], cfg["w"]
    seed = SEED[which]
    l = a.shape[0]
    print("block linear %s %s: %s" % (name, which, tuple(a.shape)), flush=True)
    wt, wd = av.averis_quant_pair(w.cuda(), rnd=av.RN)
    wq = orc.weight_quant(f32(w), "rn")
    b, b_ref = (wt, wq["fwd"]) if which == "x" else (wd, wq["dgrad"])
    assert_quant_equal(b, b_ref)
    res, mean, mu, rho = av.averis_split_quant_rank1(a.cuda(), b, seed=seed)
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.bfloat16).float().cpu().numpy()
    c32 = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.float32).cpu().numpy()
    mu_ref, res_ref, mean_ref = oracle_split(pool, f32(a), seed)
    np.testing.assert_array_equal(mu.cpu().numpy(), mu_ref)
    assert_quant_equal(res, res_ref)
    assert_quant_equal(mean, mean_ref)
    check_rho(rho.cpu().numpy(), mean_ref, b_ref)
    b_deq, m_deq = orc.dequantize(b_ref), orc.dequantize(mean_ref)[0]
    rows = np.concatenate([np.arange(r0, r1) for r0, r1 in sample_rows(l)])
    a_deq = orc.dequantize(dict(res_ref, codes=res_ref["codes"][rows],
                                scales=res_ref["scales"][rows]))
    ref = a_deq @ b_deq.T + (m_deq @ b_deq.T)[None, :]
    bound = np.abs(a_deq) @ np.abs(b_deq).T + (np.abs(m_deq) @ np.abs(b_deq).T)[None, :]
    assert_gemm_close(c[rows], ref, bound, bf16=True, label="%s %s bf16 rows" % (name, which))
    assert_gemm_close(c32[rows], ref, bound, label="%s %s fp32 rows" % (name, which))
    torch.cuda.synchronize()


@pytest.mark.parametrize("which", ["x", "d"])
def test_moe_full_size(pool, which):
    cfg = workloads.moe()       # 4096 tokens x top-8 over 64 experts, hidden 2048, inter 768
    a, w, offs = cfg[which], cfg["w"], cfg["offsets"]
    seed = SEED[which]
    nseg = len(offs) - 1
    print("MoE %s: %s over %d experts" % (which, tuple(a.shape), nseg), flush=True)
    og = torch.from_numpy(offs).cuda()
    wt, wd = av.averis_quant_pair(w.cuda(), rnd=av.RN)
    b = wt if which == "x" else wd
    res, mean, mu, rho = av.averis_split_quant_grouped_rank1(a.cuda(), og, b, seed=seed)
    c = av.averis_gemm_grouped_rank1(res, rho, b, og, out_dtype=torch.bfloat16)
    cc = c.float().cpu().numpy()
    rc, mc, bc = res.cpu(), mean.cpu(), b.cpu()
    mu_g, rho_g = mu.cpu().numpy(), rho.cpu().numpy()
    an, wn = f32(a), f32(w)
    n = b.rows // nseg
    counts = np.diff(offs)
    live = [e for e in range(nseg) if counts[e] > 0]
    by_size = sorted(live, key=lambda e: counts[e])
    picks = sorted({live[0], live[-1], by_size[0], by_size[len(by_size) // 2], by_size[-1]})
    # the oracle: each expert's weight copy and each segment's split, all
    # quantizations in one parallel map
    wsrc = [wn[e] if which == "d" else np.ascontiguousarray(wn[e].T) for e in range(nseg)]
    mus, calls = {}, [(wsrc[e], "rn", 0, 2, 0, None) for e in range(nseg)]
    for e in live:
        r0, r1 = int(offs[e]), int(offs[e + 1])
        mus[e] = orc.column_mean(an[r0:r1])
        calls.append((orc.residual(an[r0:r1], mus[e]), "sr", seed, 0, r0, None))
    out = pool.quantize_many(calls)
    b_refs, res_refs = out[:nseg], dict(zip(live, out[nseg:]))
    for e in range(nseg):
        r0, r1 = int(offs[e]), int(offs[e + 1])
        b_ref = b_refs[e]
        assert_quant_equal(bc, b_ref, seg=e, rows=slice(e * n, (e + 1) * n))
        if r1 == r0:
            assert not mu_g[e].any() and not rho_g[e * n:(e + 1) * n].any()
            assert rc["tscale"][2 * e] == 1.0 and rc["tscale"][2 * e + 1] == 1.0
            continue
        mu_ref, res_ref = mus[e], res_refs[e]
        mean_ref = orc.quantize(mu_ref[None, :], "sr", seed, stream=1, row0=e)
        np.testing.assert_array_equal(mu_g[e], mu_ref)
        assert_quant_equal(rc, res_ref, seg=e, rows=slice(r0, r1))
        assert_quant_equal(mc, mean_ref, seg=e, rows=slice(e, e + 1))
        check_rho(rho_g[e * n:(e + 1) * n], mean_ref, b_ref)
        if e in picks:
            t1 = min(r1 - r0, 32)
            q = dict(res_ref, codes=res_ref["codes"][:t1], scales=res_ref["scales"][:t1])
            a_deq, b_deq = orc.dequantize(q), orc.dequantize(b_ref)
            m_deq = orc.dequantize(mean_ref)[0]
            ref = a_deq @ b_deq.T + (m_deq @ b_deq.T)[None, :]
            bound = np.abs(a_deq) @ np.abs(b_deq).T + (np.abs(m_deq) @ np.abs(b_deq).T)[None, :]
            assert_gemm_close(cc[r0:r0 + t1], ref, bound, bf16=True,
                              label="MoE %s expert %d (%d rows)" % (which, e, r1 - r0))
    torch.cuda.synchronize()
