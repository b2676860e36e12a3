"""Column statistics fused into the producer ([Lighthouse] §2.2 cost note and
§4.2): averis_gemm_rank1_stats writes the column statistics of its bf16
output in its epilogue and averis_split_quant_from_stats splits that output
with one read.  Checked through the C ABI:

* the GEMM's output is averis_gemm_rank1's, bit for bit;
* the split from the statistics is averis_split_quant of the same tensor, bit
  for bit (the fp32 mean, codes, scale bytes, tensor scales, mean codes, and
  the rank-one row of the next GEMM), and on the tiny case also the oracle's;
* on hand-built operands whose outputs span a huge range the mean's fp64
  sum is not certified exact for some columns and one 256-row tile is not
  exact on its own either, so the exact re-summation of both kinds runs.
Shapes: the tiny case, the up-proj and down-proj sizes, a ragged one."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads
from tests.parity import assert_quant_equal

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def same_nvfp4(g, r):
    for t in ("codes", "scales", "tscale"):
        assert torch.equal(getattr(g, t), getattr(r, t)), t


def check_producer(xr, rho, wt, seed, nxt=None):
    """GEMM with and without statistics, then both splits of its output."""
    c_ref = av.averis_gemm_rank1(xr, rho, wt, out_dtype=torch.bfloat16)
    c, ws = av.averis_gemm_rank1_stats(xr, rho, wt)
    assert torch.equal(c, c_ref)
    got = av.averis_split_quant_from_stats(c, ws, seed=seed)
    ref = av.averis_split_quant(c, seed=seed)
    same_nvfp4(got[0], ref[0])
    same_nvfp4(got[1], ref[1])
    assert torch.equal(got[2], ref[2])
    if nxt is not None:
        c2, ws2 = av.averis_gemm_rank1_stats(xr, rho, wt)
        g1 = av.averis_split_quant_from_stats(c2, ws2, seed=seed, b=nxt)
        r1 = av.averis_split_quant_rank1(c2, nxt, seed=seed)
        same_nvfp4(g1[0], r1[0])
        assert torch.equal(g1[2], r1[2])
        assert torch.equal(g1[3], r1[3])
    torch.cuda.synchronize()
    return c, got


@pytest.mark.parametrize("case", ["tiny", "up_proj", "down_proj", "ragged"])
def test_split_from_gemm_statistics_equals_split(case):
    if case == "tiny":
        cfg = workloads.tiny()                                # X 64x128 -> Y 64x64
    elif case == "ragged":
        cfg = workloads.up_proj(l=1000, m=320, n=208)
    else:
        cfg = getattr(workloads, case)()
    x, w = cfg["x"].cuda(), cfg["w"].cuda()
    print("%s: X %s, W %s" % (case, tuple(x.shape), tuple(w.shape)), flush=True)
    wt, wd = av.averis_quant_pair(w, rnd=av.RN)
    xr, _, _, rho = av.averis_split_quant_rank1(x, wt, seed=0)
    # the next layer's weight (n x n2), forward copy, for the rank-one form
    n = w.shape[1]
    w2 = workloads.weight(workloads.rng_for(9, 1), n, 96).cuda()
    nxt = av.averis_quant(w2, transpose=True, rnd=av.RN, sr_stream=av.STREAM_WEIGHT)
    c, got = check_producer(xr, rho, wt, seed=5, nxt=nxt)
    if case == "tiny":
        s = orc.split_quant(c.float().cpu().numpy(), "sr", 5)
        np.testing.assert_array_equal(got[2].cpu().numpy(), s["mu"])
        assert_quant_equal(got[0], s["residual"])
        assert_quant_equal(got[1], s["mean"])


def nvfp4_from_bytes(codes, scales):
    rows, half = codes.shape
    return av.NVFP4(torch.from_numpy(codes).cuda(), torch.from_numpy(scales).cuda(),
                    torch.tensor([1.0, 1.0], dtype=torch.float32, device="cuda"), rows, 2 * half)


def test_uncertified_columns_of_a_gemm_output():
    # Hand-built operands (tensor scales 1).  A row 300: six (code 7) in the
    # first 16-block with the largest E4M3 scale 448 (0x7E); every other A
    # row: one 0.5 (code 1) in the second block with the smallest scale 2^-9
    # (0x01).  Every B row: sixes at scale 448 in block 0, halves at 2^-9 in
    # block 1.  So C[300, :] is about 2^26.8 and every other
    # entry is 2^-20 exactly: each column's fp64 sum over 1000 rows is not
    # certified exact, the 256-row tile holding row 300 is not exact on its
    # own (its rows are re-summed) and the other tiles are (their partials
    # are added exactly).
    m, k, n = 1000, 128, 208
    ac = np.zeros((m, k // 2), np.uint8)
    asc = np.full((m, k // 16), 0x01, np.uint8)
    ac[300, :8] = 0x77
    asc[300, 0] = 0x7E
    for r in range(m):
        if r != 300:
            e = 16 + r % 16
            ac[r, e // 2] = 0x01 if e % 2 == 0 else 0x10
    bc = np.zeros((n, k // 2), np.uint8)
    bsc = np.full((n, k // 16), 0x01, np.uint8)
    bc[:, :8] = 0x77
    bsc[:, 0] = 0x7E
    bc[:, 8:16] = 0x11
    a, b = nvfp4_from_bytes(ac, asc), nvfp4_from_bytes(bc, bsc)
    rho = torch.zeros((n,), dtype=torch.float32, device="cuda")
    c, got = check_producer(a, rho, b, seed=3)
    cc = c.float().cpu().numpy().astype(np.float64)
    # 16 * 36 * 448^2 = 441 * 2^18 needs 9 significant bits: bf16 keeps 440 * 2^18
    assert cc[300, 0] == 440 * 2.0 ** 18 and cc[0, 0] == 2.0 ** -20
    cert = lambda t: t.shape[0] * np.abs(t).max() <= 2.0 ** (52 + np.frexp(np.abs(t).min())[1] - 1 - 7)
    assert not cert(cc[:, 0])            # the column: not certified
    assert not cert(cc[256:512, 0])      # the tile holding row 300: not on its own either
    assert cert(cc[0:256, 0])            # the first tile: exact on its own
    # the mean is the correctly rounded one (oracle)
    np.testing.assert_array_equal(got[2].cpu().numpy(), orc.column_mean(c.float().cpu().numpy()))
