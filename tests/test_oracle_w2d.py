"""Pins of the oracle's shared 16x16-block weight quantization (reading: one
quantized W serves both GEMMs, so the dgrad operand is exactly the transpose
of the forward one; [Lighthouse] §2.2 writes it so)."""

import numpy as np
import pytest

from oracle import averis as orc
from oracle import formats


def weight(m, n, seed):
    """A weight with per-tile magnitudes spread over four decades."""
    rng = np.random.default_rng(seed)
    w = rng.standard_normal((m, n)).astype(np.float32)
    tile_scale = 10.0 ** rng.uniform(-2, 2, size=(m // 16, n // 16))
    return (w * np.repeat(np.repeat(tile_scale, 16, 0), 16, 1)).astype(np.float32)


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_forward_copy_is_the_exact_transpose(rnd):
    w = weight(64, 48, 1)
    q = orc.weight_quant_2d(w, rnd=rnd, seed=7)
    assert q["fwd"]["codes"].shape == (48, 32) and q["dgrad"]["codes"].shape == (64, 24)
    assert q["fwd"]["scales"].shape == (48, 4) and q["dgrad"]["scales"].shape == (64, 3)
    np.testing.assert_array_equal(orc.dequantize(q["fwd"]), orc.dequantize(q["dgrad"]).T)


def test_one_scale_per_tile():
    q = orc.weight_quant_2d(weight(48, 32, 2))
    s = q["dgrad"]["scales"].reshape(3, 16, 2)
    assert (s == s[:, :1, :]).all()
    t = q["fwd"]["scales"].reshape(2, 16, 3)
    assert (t == t[:, :1, :]).all()
    np.testing.assert_array_equal(s[:, 0, :], t[:, 0, :].T)


def diagonal_max(m, n, seed):
    """Every row and every column of each 16x16 tile holds the tile's largest
    magnitude (on the tile's diagonal), so the 1-D blocks of both orientations
    have the tile's maximum."""
    rng = np.random.default_rng(seed)
    w = np.empty((m, n), dtype=np.float32)
    for bi in range(m // 16):
        for bj in range(n // 16):
            big = np.float32(10.0 ** rng.uniform(-1, 1))
            tile = rng.uniform(-0.9, 0.9, size=(16, 16)) * big
            for t in range(16):
                tile[t, t] = big if rng.random() < 0.5 else -big
            w[16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16] = tile
    return w


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_reduces_to_the_1d_quantization_when_every_run_holds_the_tile_max(rnd):
    # then each 16-run's own maximum is the tile's, and the 2-D quantization
    # must agree with the 1-D one byte for byte (same SR index and stream)
    w = diagonal_max(48, 64, 3)
    q = orc.weight_quant_2d(w, rnd=rnd, seed=11)
    d1 = orc.quantize(w, rnd, 11, stream=2)
    np.testing.assert_array_equal(q["dgrad"]["codes"], d1["codes"])
    np.testing.assert_array_equal(q["dgrad"]["scales"], d1["scales"])
    assert q["dgrad"]["s_enc"] == d1["s_enc"] and q["dgrad"]["s_dec"] == d1["s_dec"]
    if rnd == "rn":
        f1 = orc.quantize(np.ascontiguousarray(w.T), "rn", 11, stream=2)
        np.testing.assert_array_equal(q["fwd"]["codes"], f1["codes"])
        np.testing.assert_array_equal(q["fwd"]["scales"], f1["scales"])


@pytest.mark.parametrize("rnd", ["rn", "sr"])
def test_constant_weight_is_exact(rnd):
    # c = 2688 / 4096: S_enc = 4096 and S_dec = 1 / 4096 are exact, the tile
    # scale is E4M3's largest (448) and every value encodes as E2M1's 6, so
    # 6 * 448 / 4096 = c comes back exactly
    w = np.full((32, 48), -0.65625, dtype=np.float32)
    q = orc.weight_quant_2d(w, rnd=rnd, seed=5)
    assert (q["dgrad"]["scales"] == formats.e4m3_encode(np.float32(448.0))).all()
    np.testing.assert_array_equal(orc.dequantize(q["dgrad"]), w.astype(np.float64))
    np.testing.assert_array_equal(orc.dequantize(q["fwd"]), w.T.astype(np.float64))


def test_stochastic_rounding_is_unbiased():
    # the mean over seeds of the SR dequantization approaches W; the RN error,
    # which is systematic, does not shrink
    w = weight(32, 32, 4)
    acc = np.zeros(w.shape)
    seeds = 64
    for s in range(seeds):
        acc += orc.dequantize(orc.weight_quant_2d(w, rnd="sr", seed=s)["dgrad"])
    err_sr = np.abs(acc / seeds - w).sum()
    err_rn = np.abs(orc.dequantize(orc.weight_quant_2d(w, rnd="rn")["dgrad"]) - w).sum()
    assert err_sr < 0.35 * err_rn


def test_zero_weight_and_bad_shapes():
    q = orc.weight_quant_2d(np.zeros((16, 16), np.float32))
    assert not orc.dequantize(q["fwd"]).any() and q["dgrad"]["s_enc"] == 1.0
    with pytest.raises(ValueError):
        orc.weight_quant_2d(np.zeros((16, 24), np.float32))
