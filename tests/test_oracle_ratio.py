"""Pins of the oracle's mean-energy ratio R = ||mu||_2 / sqrt(||A||_F^2 / l)
(reading of the monitor [Lighthouse] §7 recommends: E||X||^2 as the operand's
sum of squares, N as its row count)."""

import math

import numpy as np

from oracle import averis as orc
from mean_residual_quantized_amd import workloads


def test_hand_example():
    # X = [[1, 2], [3, 4]]: mu = (2, 3), ||mu||^2 = 13, ||X||_F^2 = 30, l = 2
    x = np.array([[1, 2], [3, 4]], dtype=np.float32)
    assert orc.mean_energy_ratio(x) == math.sqrt(13 / 15)


def test_constant_rows_give_one_and_zero_mean_columns_give_zero():
    rng = np.random.default_rng(0)
    mu = rng.standard_normal(48).astype(np.float32)
    assert abs(orc.mean_energy_ratio(np.tile(mu, (7, 1))) - 1.0) < 1e-15
    # columns made of +v / -v pairs have an exact zero mean
    v = rng.standard_normal((5, 48)).astype(np.float32)
    assert orc.mean_energy_ratio(np.concatenate([v, -v])) == 0.0


def test_degenerate_inputs():
    assert orc.mean_energy_ratio(np.zeros((0, 16), np.float32)) == 0.0
    assert orc.mean_energy_ratio(np.zeros((9, 16), np.float32)) == 0.0
    # a single row is its own mean
    assert abs(orc.mean_energy_ratio(np.arange(16, dtype=np.float32)[None, :] - 3) - 1.0) < 1e-15


def test_pythagorean_split_and_scale_invariance():
    # ||A||_F^2 = l ||mu||^2 + ||A - 1 mu||_F^2 (the residual's columns sum to
    # zero), so R^2 = ||mu||^2 / (||mu||^2 + ||A_R||_F^2 / l); checked with the
    # residual formed in float64 from the exact rational mean of each column
    from fractions import Fraction
    cfg = workloads.tiny()
    x = cfg["x"].float().numpy()
    l = x.shape[0]
    mu = [Fraction(sum(Fraction(float(v)) for v in x[:, j])) / l for j in range(x.shape[1])]
    mu2 = sum(m * m for m in mu)
    res2 = sum((Fraction(float(x[i, j])) - mu[j]) ** 2 for i in range(l) for j in range(x.shape[1]))
    ref = math.sqrt(mu2 / (mu2 + res2 / l))
    r = orc.mean_energy_ratio(x)
    assert abs(r - ref) < 1e-14
    assert 0.5 < r < 1.0               # the tiny case is mean-dominated
    # a power-of-two scale leaves every float exact, so R is unchanged
    assert orc.mean_energy_ratio(x * np.float32(8)) == r
    # the mean-free residual of the split has R near zero
    assert orc.mean_energy_ratio(orc.residual(x, orc.column_mean(x))) < 1e-6


def test_grouped_is_per_segment():
    cfg = workloads.tiny()
    x = cfg["x"].float().numpy()
    offs = [0, 10, 10, 64]
    r = orc.mean_energy_ratio_grouped(x, offs)
    assert r[1] == 0.0
    assert r[0] == orc.mean_energy_ratio(x[:10]) and r[2] == orc.mean_energy_ratio(x[10:])
