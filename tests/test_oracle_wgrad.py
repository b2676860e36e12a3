"""Pins of the oracle's wgrad (reading: the split applied to both operands of
dW = X^T D; the pages give only the forward and dgrad equations)."""

import math

import numpy as np

from oracle import averis as orc
from oracle import formats
from mean_residual_quantized_amd import workloads


def exact_split(a):
    """float64 column means (fsum / l) and residuals a - 1 mu, no rounding to fp32."""
    a = np.asarray(a, dtype=np.float64)
    mu = np.array([math.fsum(a[:, j]) / a.shape[0] for j in range(a.shape[1])])
    return mu, a - mu[None, :]


def test_combination_without_quantization_is_xt_d():
    # with exact means and residuals the residual cross terms vanish and the
    # combination reproduces X^T D (the l factor and the outer product's
    # orientation are what this pins)
    rng = np.random.default_rng(0)
    l, m, n = 96, 24, 40
    x = rng.standard_normal((l, m)) * 2 + rng.standard_normal(m)[None, :] * 3
    d = rng.standard_normal((l, n)) * 0.1 + rng.standard_normal(n)[None, :]
    mx, xr = exact_split(x)
    md, dr = exact_split(d)
    dw = orc.wgrad_combine(xr.T, dr.T, mx, md, l)
    np.testing.assert_allclose(dw, x.T @ d, rtol=1e-12, atol=1e-9)
    # dropping the mean term leaves a visible error on mean-biased data
    assert np.abs(orc.wgrad_combine(xr.T, dr.T, 0 * mx, md, l) - x.T @ d).max() > 1.0


def test_constant_columns_leave_only_the_mean_term():
    # X with constant columns: X_R = 0, so Q4(X_R^T) is all zero codes and
    # dW = l mu nu^T from the fp32 means (or from the dequantized FP4 means)
    cfg = workloads.tiny()
    mu = (3 * np.random.default_rng(1).standard_normal(128) + 1.5).astype(np.float32)
    x = np.tile(mu, (64, 1))
    d = cfg["d"].float().numpy()
    out = orc.averis_wgrad(x, d, "sr", 3, 4)
    assert not (formats.unpack_nibbles(out["xt"]["codes"]) & 7).any()
    np.testing.assert_array_equal(out["mu_x"], mu)
    np.testing.assert_array_equal(out["dw"], 64.0 * np.outer(mu.astype(np.float64), out["mu_d"]))
    q = orc.averis_wgrad(x, d, "sr", 3, 4, mean="q4")
    mq = orc.split_quant(x, "sr", 3)["mean"]
    nq = orc.split_quant(d, "sr", 4)["mean"]
    np.testing.assert_array_equal(q["dw"], 64.0 * np.outer(orc.dequantize(mq)[0], orc.dequantize(nq)[0]))


def test_transposed_residual_quant_is_per_column_quant_of_the_residual():
    # row j of Q4(X_R^T) holds column j of the residual, blocked along the
    # tokens, with one tensor scale for the whole residual (the same amax as
    # the forward's residual)
    cfg = workloads.tiny()
    x = cfg["x"].float().numpy()
    s = orc.split_quant(x, "sr", 2)
    xt = orc.residual_t_quant(x, s["mu"], "sr", 2)
    assert xt["codes"].shape == (128, 32) and xt["scales"].shape == (128, 4)
    assert xt["s_enc"] == s["residual"]["s_enc"]
    r = orc.residual(x, s["mu"])
    j = 17
    col = orc.quantize(np.ascontiguousarray(r.T), "rn", 0, stream=3)
    # the block scales do not depend on rounding; they are those of the column's 16-blocks
    np.testing.assert_array_equal(xt["scales"][j], col["scales"][j])
    amax_b = np.abs(r[:, j].reshape(4, 16)).max(axis=1)
    s_b = np.minimum(((amax_b / np.float32(6)).astype(np.float32) * xt["s_enc"]).astype(np.float32),
                     np.float32(448))
    np.testing.assert_array_equal(xt["scales"][j], formats.e4m3_encode(s_b))


def test_quantized_wgrad_close_to_exact_product():
    # Q4 error is bounded: the quantized wgrad of the tiny case stays near X^T D;
    # FP4 means in the outer product do worse than the fp32 ones on this
    # mean-biased input (their error is not averaged over the tokens)
    cfg = workloads.tiny()
    x, d = cfg["x"].float().numpy(), cfg["d"].float().numpy()
    exact = x.astype(np.float64).T @ d.astype(np.float64)
    rel = lambda a: np.linalg.norm(a - exact) / np.linalg.norm(exact)
    for rnd in ("rn", "sr"):
        out = orc.averis_wgrad(x, d, rnd, 0, 1)
        assert rel(out["dw"]) < 0.05
        assert rel(orc.averis_wgrad(x, d, rnd, 0, 1, mean="q4")["dw"]) > 3 * rel(out["dw"])
        bound = orc.wgrad_abs_bound(out["xt"], out["dt"], out["mu_x"], out["mu_d"], x.shape[0])
        assert (bound >= np.abs(out["dw"]) - 1e-9).all()


def test_sr_wgrad_is_unbiased_over_seeds():
    # SR rounds each residual element up with probability equal to its
    # fractional position, independently for X and D (different seeds), so the
    # seed average of dW tends to X^T D, up to the small bias of the clamp at
    # 6 (it acts only where a block's E4M3 scale rounded down); with RN in
    # place of SR the average would stay as far off as one sample
    cfg = workloads.tiny()
    x, d = cfg["x"].float().numpy(), cfg["d"].float().numpy()
    exact = x.astype(np.float64).T @ d.astype(np.float64)
    one = orc.averis_wgrad(x, d, "sr", 0, 1000)["dw"]
    acc = np.zeros_like(exact)
    n = 64
    for s in range(n):
        acc += orc.averis_wgrad(x, d, "sr", s, 1000 + s)["dw"]
    err_one = np.linalg.norm(one - exact)
    err_avg = np.linalg.norm(acc / n - exact)
    # independent errors shrink as 1/sqrt(n) = 1/8; allow for the spread
    assert err_avg < 0.25 * err_one


def test_wgrad_abs_bound_brute_force_tiny():
    # the wgrad parity tests divide the error by this bound: pin it to a
    # triple loop over hand-decoded bytes of the transposed residuals,
    # sum_t |xt_it| |dt_jt| + l |mu_x,i| |mu_d,j|
    from tests.test_oracle_gemm import decode_by_hand
    cfg = workloads.tiny()
    x, d = cfg["x"].float().numpy(), cfg["d"].float().numpy()
    l = x.shape[0]
    out = orc.averis_wgrad(x, d, "sr", 0, 1)
    xt, dt = out["xt"], out["dt"]
    bound = orc.wgrad_abs_bound(xt, dt, out["mu_x"], out["mu_d"], l)
    assert bound.shape == (x.shape[1], d.shape[1])
    rng = np.random.default_rng(9)
    for i, j in zip(rng.integers(0, x.shape[1], 25), rng.integers(0, d.shape[1], 25)):
        ref = sum(abs(decode_by_hand(xt, i, t)) * abs(decode_by_hand(dt, j, t)) for t in range(l))
        ref += l * abs(float(out["mu_x"][i])) * abs(float(out["mu_d"][j]))
        assert abs(bound[i, j] - ref) <= 1e-12 * ref, (i, j)
        # and the product it bounds, from the same bytes
        val = sum(decode_by_hand(xt, i, t) * decode_by_hand(dt, j, t) for t in range(l))
        val += l * float(out["mu_x"][i]) * float(out["mu_d"][j])
        assert abs(out["dw"][i, j] - val) <= 1e-12 * ref, (i, j)
