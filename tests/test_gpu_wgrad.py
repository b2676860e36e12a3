"""GPU parity of the wgrad path: the transposed residual quant (bit for bit
against the oracle) and dW = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X mu_D^T
(within 1e-3 of the bound |deq xt| |deq dt|^T + l |mu_X| |mu_D|^T, against the
oracle's float64 product of its own quantized operands)."""

import numpy as np
import pytest
import torch

from oracle import averis as orc
from tests.parity import assert_gemm_close
from mean_residual_quantized_amd import averis as av
from mean_residual_quantized_amd import workloads

pytestmark = pytest.mark.gpu

GEMM_TOL = 1e-3


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    av.lib()


def f32(t):
    return t.float().cpu().numpy()


def assert_quant_equal(gpu, ref, rows=None):
    g = gpu.cpu()
    codes, scales = g["codes"], g["scales"]
    if rows is not None:
        codes, scales = codes[rows], scales[rows]
    np.testing.assert_array_equal(codes, ref["codes"])
    np.testing.assert_array_equal(scales, ref["scales"])
    assert g["tscale"][0] == ref["s_enc"] and g["tscale"][1] == ref["s_dec"]


def assert_close(c_gpu, ref, bound, extra=0.0):
    # elementwise against the bound, and normwise for fp32 output
    assert_gemm_close(c_gpu, ref, bound, bf16=extra > 0)


def gpu_side(x, d, seed_x, seed_d, r, out_dtype=torch.float32):
    xg, dg = x.cuda(), d.cuda()
    xr, _, mx = av.averis_split_quant(xg, seed=seed_x, rnd=r)
    dr, _, md = av.averis_split_quant(dg, seed=seed_d, rnd=r)
    xt = av.averis_residual_t_quant(xg, mx, xr, seed=seed_x, rnd=r)
    dt = av.averis_residual_t_quant(dg, md, dr, seed=seed_d, rnd=r)
    dw = av.averis_gemm_wgrad(xt, dt, mx, md, out_dtype=out_dtype)
    return xt, dt, mx, md, dw


def check(x, d, seed_x=0, seed_d=1, rnd="sr", out_dtype=torch.float32):
    r = av.SR if rnd == "sr" else av.RN
    xt, dt, mx, md, dw = gpu_side(x, d, seed_x, seed_d, r, out_dtype)
    ref = orc.averis_wgrad(f32(x), f32(d), rnd, seed_x, seed_d)
    np.testing.assert_array_equal(mx.cpu().numpy(), ref["mu_x"])
    np.testing.assert_array_equal(md.cpu().numpy(), ref["mu_d"])
    assert_quant_equal(xt, ref["xt"])
    assert_quant_equal(dt, ref["dt"])
    bound = orc.wgrad_abs_bound(ref["xt"], ref["dt"], ref["mu_x"], ref["mu_d"], x.shape[0])
    extra = 2.0 ** -8 if out_dtype == torch.bfloat16 else 0.0
    assert_close(dw, ref["dw"], bound, extra)
    torch.cuda.synchronize()


def mean_biased(l, m, seed, dtype=torch.bfloat16):
    rng = np.random.default_rng(seed)
    a = rng.standard_normal((l, m)) * 0.5 + (3 * rng.standard_normal(m) + 1.5)[None, :]
    return torch.from_numpy(a.astype(np.float32)).to(dtype)


def test_tiny():
    cfg = workloads.tiny()
    check(cfg["x"], cfg["d"])


@pytest.mark.parametrize("rnd", ["rn", "sr"])
@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("l,m,n", [
    (1008, 208, 96),     # l % 64 != 0: one partial, general GEMM path
    (2048, 320, 192),    # four splits of 512 tokens (256-wide scale groups)
    (1152, 256, 208),    # two splits of 576 tokens (per-stage scale loads), ragged n tile
    (16, 16, 16),        # one token block
    (1056, 64, 48),      # token count a multiple of 32, not of 128: a partial tile of tokens
])
def test_shapes_and_paths(l, m, n, dtype, rnd):
    check(mean_biased(l, m, l + m, dtype), mean_biased(l, n, l + n + 1, dtype), seed_x=l,
          seed_d=n, rnd=rnd)


def test_bf16_output_and_row_stride():
    x, d = mean_biased(2048, 320, 5), mean_biased(2048, 192, 6)
    check(x, d, out_dtype=torch.bfloat16)
    xt, dt, mx, md, dw = gpu_side(x, d, 0, 1, av.SR)
    big = torch.full((320, 200), float("nan"), device="cuda")
    av.averis_gemm_wgrad(xt, dt, mx, md, out=big[:, :192])
    assert torch.equal(big[:, :192], dw)
    assert torch.isnan(big[:, 192:]).all()


def test_constant_columns_leave_the_outer_product():
    rng = np.random.default_rng(3)
    mu = (3 * rng.standard_normal(64) + 1.5).astype(np.float32)
    x = torch.from_numpy(np.tile(mu, (512, 1)))
    d = mean_biased(512, 48, 4, torch.float32)
    check(x, d)
    xt, dt, mx, md, dw = gpu_side(x, d, 0, 1, av.SR)
    assert not (xt.codes & 0x77).any()


def test_no_tokens():
    x = torch.zeros((0, 64), dtype=torch.bfloat16, device="cuda")
    d = torch.zeros((0, 32), dtype=torch.bfloat16, device="cuda")
    xr, _, mx = av.averis_split_quant(x)
    dr, _, md = av.averis_split_quant(d)
    xt = av.averis_residual_t_quant(x, mx, xr)
    dt = av.averis_residual_t_quant(d, md, dr)
    assert xt.tscale.tolist() == [1.0, 1.0]
    dw = av.averis_gemm_wgrad(xt, dt, mx, md)
    assert dw.shape == (64, 32) and not dw.any()


def test_repeat_calls_give_the_same_bits():
    x, d = mean_biased(2048, 320, 7), mean_biased(2048, 192, 8)
    xt, dt, mx, md, dw = gpu_side(x, d, 0, 1, av.SR)
    for _ in range(3):
        assert torch.equal(av.averis_gemm_wgrad(xt, dt, mx, md), dw)


def test_full_size_up_proj_sampled():
    # up-proj shapes: X 8192 x 1024, D 8192 x 3072, dW 1024 x 3072 (four
    # splits of 2048 tokens); sampled rows of the transposed residuals are
    # exact, and dW on the sampled rows and columns is within tolerance
    cfg = workloads.up_proj()
    x, d = cfg["x"], cfg["d"]
    l = x.shape[0]
    xt, dt, mx, md, dw = gpu_side(x, d, 0, 1, av.SR)
    dwc = dw.cpu().numpy().astype(np.float64)
    deq = {}
    for name, a, q, mu_g, idx in (("x", x, xt, mx, [0, 1, 517, 1023]),
                                  ("d", d, dt, md, [0, 191, 192, 2048, 3071])):
        an = f32(a)
        mu = orc.column_mean(an)
        np.testing.assert_array_equal(mu_g.cpu().numpy(), mu)
        r = orc.residual(an, mu)
        amax = np.max(np.abs(r))
        rows = []
        for i in idx:
            ref = orc.quantize(np.ascontiguousarray(r[:, i:i + 1].T), "sr", 0 if name == "x" else 1,
                               stream=3, row0=i, amax=amax)
            assert_quant_equal(q, ref, rows=slice(i, i + 1))
            rows.append(orc.dequantize(ref)[0])
        deq[name] = (np.array(rows), mu.astype(np.float64), idx)
    (xr, mux, ix), (dr, mud, jd) = deq["x"], deq["d"]
    ref = xr @ dr.T + l * np.outer(mux[ix], mud[jd])
    bound = np.abs(xr) @ np.abs(dr).T + l * np.outer(np.abs(mux[ix]), np.abs(mud[jd]))
    got = dwc[np.ix_(ix, jd)]
    err = np.abs(got - ref)
    assert (err <= GEMM_TOL * bound).all(), np.max(err / bound)
