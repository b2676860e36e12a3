"""Pins for the oracle's mean, residual and Q4: a worked example derived by
hand from the stated definitions, exact round trips, exact column sums,
and the invariants the method implies ([Lighthouse] §2.1-§2.2)."""

from fractions import Fraction

import numpy as np
import pytest

from oracle import averis, formats
from mean_residual_quantized_amd import workloads

F32 = np.float32


# ---- worked example (derived by hand, see the comments) -----------------
#
# One row, two 16-blocks.  amax = 6 -> S_enc = 2688/6 = 448, S_dec = 1/448.
# Block A: amax_b = 6 -> s_b = (6/6)*448 = 448 -> E4M3 0x7E (1.75*2^8), so
# e_b = 448/448 = 1 and v = T.  RN with ties to the even index:
#   6->7, 3->5, -1.25 (tie 1|1.5)->idx2 neg=0xA, 0.25 (tie 0|0.5)->0,
#   0.75 (tie)->2, 5 (tie 4|6)->6, 2.5 (tie 2|3)->4, -0.1->0 neg=0x8,
#   1.75 (tie)->4, 3.5 (tie)->6, 0->0, -6->0xF, 1->2, 0.5->1, 4.5->6,
#   -2.9->5 neg=0xD.
# Block B: amax_b = f32(0.3); f32(f32(0.3)/6) = 0.0500000007..;
#   * 448 -> f32 22.3999996; E4M3 quantum in [16, 32) is 2 -> 11.2 -> 11 ->
#   22 = 0x5B.  e_b = f32(448/22) = 20.3636..; v = [6.109, -3.054, 1.018,
#   2.444, 0...] -> 6 saturates (the scale rounded down) -> 7; -3.05 -> 0xD;
#   1.02 -> 2; 2.44 -> 4; zeros -> 0.
BLOCK_A = [6, 3, -1.25, 0.25, 0.75, 5, 2.5, -0.1, 1.75, 3.5, 0, -6, 1.0, 0.5, 4.5, -2.9]
BLOCK_B = [0.3, -0.15, 0.05, 0.12] + [0] * 12
PACKED_A = [0x57, 0x0A, 0x62, 0x84, 0x64, 0xF0, 0x12, 0xD6]
PACKED_B = [0xD7, 0x42, 0, 0, 0, 0, 0, 0]


def test_worked_example_rn():
    t = np.array([BLOCK_A + BLOCK_B], dtype=np.float32)
    q = averis.quantize(t, "rn")
    assert q["s_enc"] == F32(448.0)
    assert q["s_dec"] == F32(1.0) / F32(448.0)
    assert list(q["scales"][0]) == [0x7E, 0x5B]
    assert list(q["codes"][0]) == PACKED_A + PACKED_B


def test_roundtrip_exact_on_grid_times_power_of_two():
    # One anchor element 2688 * 2^-p makes amax = 2688 / 2^p, so S_enc = 2^p
    # and S_dec = 2^-p exactly.  Every other block holds grid values g * 2^t
    # with block amax 6 * 2^t: its scale is the E4M3 power of two 2^(t+p),
    # its factor e_b = 2^-t is exact, v = g, and deq(Q4(x)) == x exactly.
    rng = np.random.default_rng(5)
    for p, ts in [(0, [-8, -3, 0, 2]), (6, [-9, -4, 0, 2]), (-4, [-5, 0, 3, 4])]:
        g = np.array(formats.E2M1_GRID)[rng.integers(0, 8, size=(len(ts), 64))]
        g *= np.where(rng.random(g.shape) < 0.5, -1, 1)
        g[:, ::16] = 6.0
        x = g * np.exp2(np.array(ts, dtype=np.float64))[:, None]
        anchor = np.zeros((1, 64))
        anchor[0, 0] = 2688.0 * 2.0 ** -p
        x = np.concatenate([anchor, x]).astype(np.float32)
        for rnd in ("rn", "sr"):
            q = averis.quantize(x, rnd, seed=3)
            assert q["s_enc"] == 2.0 ** p and q["s_dec"] == 2.0 ** -p
            np.testing.assert_array_equal(averis.dequantize(q), x.astype(np.float64))


def test_column_mean_equals_exact_rational_mean():
    x = workloads.tiny()["x"].numpy()
    mu = averis.column_mean(x)
    for j in range(x.shape[1]):
        exact = sum(Fraction(float(v)) for v in x[:, j]) / x.shape[0]
        # float32 of (the float64 nearest the exact sum) / l, two roundings
        s64 = float(sum(Fraction(float(v)) for v in x[:, j]))   # correctly rounded
        assert mu[j] == F32(s64 / x.shape[0])
        assert abs(Fraction(float(mu[j])) - exact) <= Fraction(float(np.spacing(abs(mu[j]))))


def test_column_mean_exact_with_wide_dynamic_range():
    # a float64 running sum in row order loses the first 1.0 (2^60 + 1 needs
    # 61 bits) and would give 0.2; the exact mean is 0.4
    x = np.zeros((5, 16), dtype=np.float32)
    x[:, 0] = [2.0 ** 60, 1.0, -(2.0 ** 60), 1.0, 0.0]
    mu = averis.column_mean(x)
    assert mu[0] == F32(2.0 / 5)


def test_constant_columns_give_zero_residual():
    # X = 1 mu^T: residual is exactly 0, every residual code has magnitude 0,
    # S_enc = 1, block scales 0; the mean carries the whole tensor
    rng = np.random.default_rng(6)
    mu = (3 * rng.standard_normal(48) + 1.5).astype(np.float32)
    x = np.tile(mu, (37, 1))
    s = averis.split_quant(x, "sr", seed=11)
    np.testing.assert_array_equal(s["mu"], mu)
    r = s["residual"]
    assert r["s_enc"] == 1 and r["s_dec"] == 1
    assert not r["scales"].any()
    assert not (r["codes"] & 0x77).any()
    np.testing.assert_array_equal(averis.dequantize(r), 0.0)


def test_single_token_is_a_constant_column_case():
    x = np.random.default_rng(7).standard_normal((1, 32)).astype(np.float32)
    s = averis.split_quant(x, "rn")
    np.testing.assert_array_equal(s["mu"], x[0])
    assert not (s["residual"]["codes"] & 0x77).any()


def test_residual_column_mean_is_zero_before_quantization():
    x = workloads.tiny()["x"].numpy()
    mu = averis.column_mean(x)
    r = averis.residual(x, mu)
    l = x.shape[0]
    col = np.array([float(sum(Fraction(float(v)) for v in r[:, j])) for j in range(x.shape[1])])
    # each f32 subtraction errs by at most half an ulp of its result
    bound = 0.5 * np.spacing(np.abs(r).astype(np.float32)).astype(np.float64).sum(axis=0)
    bound += l * 0.5 * np.spacing(np.abs(mu)).astype(np.float64)   # mean rounded to f32
    assert np.all(np.abs(col) <= bound)
    # and the split removes the mean: far smaller than the raw column sums
    assert np.max(np.abs(col)) < 1e-3 * np.max(np.abs(x.sum(axis=0)))


def test_split_shrinks_the_tensor_scale_on_mean_biased_input():
    x = workloads.tiny()["x"].numpy()
    s = averis.split_quant(x, "rn")
    v = averis.vanilla_quant(x, "rn")
    # residual amax is smaller than the raw amax, so S_enc is larger
    assert s["residual"]["s_enc"] > 1.5 * v["s_enc"]


def test_all_zero_tensor():
    q = averis.quantize(np.zeros((3, 32), np.float32), "sr", seed=1)
    assert q["s_enc"] == 1 and q["s_dec"] == 1
    assert not q["scales"].any() and not q["codes"].any()


def test_negative_zero_keeps_sign():
    t = np.zeros((1, 16), np.float32)
    t[0, 0] = 1.0
    t[0, 1] = -0.0
    t[0, 2] = -1e-9
    q = averis.quantize(t, "rn")
    c = formats.unpack_nibbles(q["codes"])[0]
    assert c[1] == 0x8 and c[2] == 0x8 and c[3] == 0x0


def test_rejects_ragged_cols():
    with pytest.raises(ValueError):
        averis.quantize(np.zeros((2, 24), np.float32))


def test_sr_depends_only_on_global_index():
    # quantizing a segment with row0 gives the same codes as the matching rows
    # of the whole tensor when the scales are shared
    x = np.random.default_rng(8).standard_normal((20, 64)).astype(np.float32)
    amax = np.max(np.abs(x))
    whole = averis.quantize(x, "sr", seed=99)
    part = averis.quantize(x[7:13], "sr", seed=99, row0=7, amax=amax)
    np.testing.assert_array_equal(part["codes"], whole["codes"][7:13])
    np.testing.assert_array_equal(part["scales"], whole["scales"][7:13])


def test_grouped_matches_per_segment_split():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((40, 32)) + 2).astype(np.float32)
    offsets = [0, 10, 10, 33, 40]                 # includes an empty segment
    g = averis.split_quant_grouped(x, offsets, "sr", seed=5)
    for s in range(4):
        r0, r1 = offsets[s], offsets[s + 1]
        if r1 == r0:
            assert not g["mu"][s].any()
            assert g["mean"][s]["s_enc"] == 1
            continue
        mu = averis.column_mean(x[r0:r1])
        np.testing.assert_array_equal(g["mu"][s], mu)
        q = averis.quantize(averis.residual(x[r0:r1], mu), "sr", 5, stream=0, row0=r0)
        np.testing.assert_array_equal(g["residual"][s]["codes"], q["codes"])
