"""The GEMM acceptance test itself, checked on the CPU with outputs the oracle
computes and then perturbs: it must reject an error just above its limit, a
dropped 16-block of one row, and a missing rank-one row, and accept an error
just below its limit.  Also: the pooled oracle quantization equals the
whole-tensor call."""

import numpy as np
import pytest

from oracle import averis as orc
from mean_residual_quantized_amd import workloads
from tests.parity import (GEMM_TOL, OraclePool, assert_elementwise, assert_gemm_close,
                          assert_normwise, gemm_errors)


def case(l=64, m=3072, n=256, seed=0):
    """An up-proj-like dgrad product at K = 3072 (the widest K of the
    workloads), small enough for the float64 oracle to be instant."""
    cfg = workloads.up_proj(l=l, m=n, n=m)
    d, w = cfg["d"].float().numpy(), cfg["w"].float().numpy()
    wq = orc.weight_quant(w, "rn")
    s = orc.split_quant(d, "sr", seed)
    ref = orc.gemm(s["residual"], wq["dgrad"], s["mean"])
    bound = orc.gemm_abs_bound(s["residual"], wq["dgrad"], s["mean"])
    return s, wq["dgrad"], ref, bound


def test_each_limit_is_sharp():
    _, _, ref, bound = case()
    i, j = np.unravel_index(np.argmax(np.abs(ref)), ref.shape)
    for tight, scale in ((assert_elementwise, bound[i, j]), (assert_normwise, np.abs(ref).max())):
        args = (lambda c: (c, ref, bound)) if tight is assert_elementwise else (lambda c: (c, ref))
        below = ref.copy()
        below[i, j] += 0.99 * GEMM_TOL * scale
        tight(*args(below))
        above = ref.copy()
        above[i, j] -= 1.01 * GEMM_TOL * scale
        with pytest.raises(AssertionError):
            tight(*args(above))


def test_normwise_limit_catches_what_the_bound_allows():
    # where cancellation makes the bound large next to max|C|, an error under
    # 1e-3 of the bound can still exceed 1e-3 of the output's scale
    _, _, ref, bound = case()
    peak = np.abs(ref).max()
    i, j = np.unravel_index(np.argmax(bound), ref.shape)
    assert bound[i, j] > 1.1 * peak
    c = ref.copy()
    c[i, j] += 1.01 * GEMM_TOL * peak
    elem, norm = gemm_errors(c, ref, bound)
    assert elem < GEMM_TOL < norm
    with pytest.raises(AssertionError):
        assert_gemm_close(c, ref, bound)
    c[i, j] = ref[i, j] + 0.99 * GEMM_TOL * peak
    assert_gemm_close(c, ref, bound)


def test_a_dropped_block_or_mean_row_fails():
    s, b, ref, bound = case()
    a = orc.dequantize(s["residual"])
    bd = orc.dequantize(b)
    # one row loses one 16-element block of its contraction
    dropped = ref.copy()
    dropped[5] -= a[5, 160:176] @ bd[:, 160:176].T
    with pytest.raises(AssertionError):
        assert_gemm_close(dropped, ref, bound)
    # the rank-one mean row is left out
    with pytest.raises(AssertionError):
        assert_gemm_close(orc.gemm(s["residual"], b), ref, bound)


def test_bf16_rounding_allowance():
    _, _, ref, bound = case()
    import torch
    c = torch.from_numpy(ref.astype(np.float32)).to(torch.bfloat16)
    assert_gemm_close(c, ref, bound, bf16=True)
    with pytest.raises(AssertionError):
        assert_gemm_close(c, ref, bound)   # not within 1e-3 of max|C| unrounded


def test_pooled_quantize_equals_whole_tensor_call():
    cfg = workloads.up_proj(l=1100, m=64, n=96)
    x = cfg["x"].float().numpy()
    mu = orc.column_mean(x)
    r = orc.residual(x, mu)
    whole = orc.quantize(r, "sr", 3, stream=0)
    pool = OraclePool(procs=3)
    try:
        parts = pool.quantize(r, "sr", 3, 0, block=128)
    finally:
        pool.close()
    for key in ("codes", "scales"):
        np.testing.assert_array_equal(parts[key], whole[key])
    assert parts["s_enc"] == whole["s_enc"] and parts["s_dec"] == whole["s_dec"]
