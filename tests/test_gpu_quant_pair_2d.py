"""GPU parity of averis_quant_pair_2d (both GEMM copies of a weight from one
quantization in 16 x 16 tiles) against the oracle's weight_quant_2d, bit for
bit, and of the Averis GEMMs that take those copies, within 1e-3 of their
bounds."""

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


def same(gpu, ref, rows=None, seg=0):
    g = gpu.cpu()
    codes, scales = g["codes"], g["scales"]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(scales, ref["scales"])
    assert g["tscale"][2 * seg] == ref["s_enc"] and g["tscale"][2 * seg + 1] == ref["s_dec"]


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_full_size_weight_matches_oracle(rnd):
    w = workloads.up_proj()["w"]                 # 1024 x 3072 bf16
    r = av.RN if rnd == "rn" else av.SR
    wt, wd = av.averis_quant_pair_2d(w.cuda(), seed=3, rnd=r)
    ref = orc.weight_quant_2d(w.float().numpy(), rnd, 3)
    same(wt, ref["fwd"])
    same(wd, ref["dgrad"])


@pytest.mark.parametrize("rows,cols", [(304, 208), (16, 16), (64, 64), (80, 1040), (2000, 48)])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
def test_ragged_tiles_and_dtypes(rows, cols, dtype):
    rng = np.random.default_rng(rows * 5 + cols)
    # tile magnitudes over four decades, so the tile scales differ
    mag = 10.0 ** rng.uniform(-2, 2, size=((rows + 15) // 16, (cols + 15) // 16))
    base = rng.standard_normal((rows, cols)) * np.repeat(np.repeat(mag, 16, 0), 16, 1)[:rows, :cols]
    w = torch.from_numpy(base.astype(np.float32)).to(dtype)
    wn = w.float().numpy()
    for rnd, r in (("rn", av.RN), ("sr", av.SR)):
        wt, wd = av.averis_quant_pair_2d(w.cuda(), seed=rows, rnd=r)
        ref = orc.weight_quant_2d(wn, rnd, rows)
        same(wt, ref["fwd"])
        same(wd, ref["dgrad"])


def test_row_stride_and_batch_of_experts():
    rng = np.random.default_rng(12)
    e, m, n = 3, 128, 96
    big = torch.from_numpy(rng.standard_normal((e, m, n + 32)).astype(np.float32)).to(torch.bfloat16)
    w = big.cuda()[:, :, :n]                     # row stride n + 32, batch stride m (n + 32)
    wt, wd = av.averis_quant_pair_2d(w, seed=9, rnd=av.SR)
    wn = big[:, :, :n].float().numpy()
    for b in range(e):
        ref = orc.weight_quant_2d(wn[b], "sr", 9, row0=b * m)
        same(wt, ref["fwd"], rows=slice(b * n, (b + 1) * n), seg=b)
        same(wd, ref["dgrad"], rows=slice(b * m, (b + 1) * m), seg=b)


def test_zero_weight():
    w = torch.zeros((32, 48), dtype=torch.bfloat16, device="cuda")
    wt, wd = av.averis_quant_pair_2d(w)
    for q in (wt, wd):
        assert not q.codes.any() and not q.scales.any()
        assert q.tscale.tolist() == [1.0, 1.0]


@pytest.mark.parametrize("which", ["x", "d"])
def test_averis_gemms_take_the_shared_copies(which):
    # forward: X (l x m) against W^T's copy; dgrad: D (l x n) against W's copy
    cfg = workloads.up_proj(l=512, m=256, n=384)
    a, w = cfg[which], cfg["w"]
    wt, wd = av.averis_quant_pair_2d(w.cuda(), seed=1, rnd=av.RN)
    b = wt if which == "x" else wd
    res, mean, mu, rho = av.averis_split_quant_rank1(a.cuda(), b, seed=4, rnd=av.SR)
    c = av.averis_gemm_rank1(res, rho, b, out_dtype=torch.float32)
    wq = orc.weight_quant_2d(w.float().numpy(), "rn", 1)
    b_ref = wq["fwd"] if which == "x" else wq["dgrad"]
    s = orc.split_quant(a.float().numpy(), "sr", 4)
    ref = orc.gemm(s["residual"], b_ref, s["mean"])
    bound = orc.gemm_abs_bound(s["residual"], b_ref, s["mean"])
    cc = c.cpu().numpy().astype(np.float64)
    assert_gemm_close(cc, ref, bound)
