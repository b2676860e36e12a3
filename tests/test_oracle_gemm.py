"""Pins for the oracle's split GEMMs ([Lighthouse] §2.2 forward and backward):
a brute-force triple loop over codes decoded by hand, the algebra of the
unquantized split, and the rank-one structure of a constant-column input."""

import numpy as np

from oracle import averis
from mean_residual_quantized_amd import workloads

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]


def decode_by_hand(q, i, k):
    """Value of element (i, k) of a quantized tensor, straight from its bytes."""
    byte = int(q["codes"][i, k // 2])
    code = byte & 0xF if k % 2 == 0 else byte >> 4
    mag = GRID[code & 7]
    c = int(q["scales"][i, k // 16])
    e, m = (c >> 3) & 15, c & 7
    scale = m * 2.0 ** -9 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7)
    return (-mag if code & 8 else mag) * scale * float(q["s_dec"])


def test_split_gemm_brute_force_tiny():
    cfg = workloads.tiny()
    x, w = cfg["x"].numpy(), cfg["w"].numpy()          # 64x128, 128x64
    wq = averis.weight_quant(w, "rn")
    s, y = averis.averis_forward(x, wq["fwd"], "sr", seed=0)
    a, b, mu = s["residual"], wq["fwd"], s["mean"]
    rows, k = x.shape
    n = w.shape[1]
    rng = np.random.default_rng(0)
    for i, j in zip(rng.integers(0, rows, 40), rng.integers(0, n, 40)):
        acc = 0.0
        for kk in range(k):
            bjk = decode_by_hand(b, j, kk)
            acc += decode_by_hand(a, i, kk) * bjk + decode_by_hand(mu, 0, kk) * bjk
        assert abs(acc - y[i, j]) <= 1e-12 * max(1.0, abs(acc)), (i, j)


def test_dgrad_brute_force_tiny():
    cfg = workloads.tiny()
    d, w = cfg["d"].numpy(), cfg["w"].numpy()          # D 64x64, W 128x64
    wq = averis.weight_quant(w, "rn")
    s, dx = averis.averis_dgrad(d, wq["dgrad"], "sr", seed=0)
    assert dx.shape == (64, 128)
    a, b, mu = s["residual"], wq["dgrad"], s["mean"]
    rng = np.random.default_rng(1)
    for i, j in zip(rng.integers(0, 64, 30), rng.integers(0, 128, 30)):
        acc = sum((decode_by_hand(a, i, kk) + decode_by_hand(mu, 0, kk)) * decode_by_hand(b, j, kk)
                  for kk in range(64))
        assert abs(acc - dx[i, j]) <= 1e-12 * max(1.0, abs(acc))


def test_weight_copies_have_the_right_orientation():
    w = np.random.default_rng(2).standard_normal((48, 32)).astype(np.float32)
    wq = averis.weight_quant(w, "rn")
    assert wq["fwd"]["codes"].shape == (32, 24)        # n x m/2, blocks along m
    assert wq["dgrad"]["codes"].shape == (48, 16)      # m x n/2, blocks along n
    # both dequantize to within the NVFP4 error of the same W
    for deq, ref in [(averis.dequantize(wq["fwd"]).T, w), (averis.dequantize(wq["dgrad"]), w)]:
        assert np.max(np.abs(deq - ref)) <= 0.3 * np.max(np.abs(w))
        assert np.corrcoef(deq.ravel(), ref.ravel())[0, 1] > 0.98


def test_unquantized_split_equals_plain_matmul():
    # the split itself is exact algebra: 1 mu^T W + (X - 1 mu^T) W = X W
    x = workloads.tiny()["x"].numpy().astype(np.float64)
    w = workloads.tiny()["w"].numpy().astype(np.float64)
    mu = x.mean(axis=0)
    y = np.ones((x.shape[0], 1)) @ (mu[None, :] @ w) + (x - mu[None, :]) @ w
    np.testing.assert_allclose(y, x @ w, rtol=1e-12, atol=1e-12 * np.abs(x @ w).max())


def test_constant_columns_rows_equal_mean_times_weight():
    rng = np.random.default_rng(3)
    mu = (3 * rng.standard_normal(64) + 1.5).astype(np.float32)
    x = np.tile(mu, (20, 1))
    wq = averis.weight_quant(rng.standard_normal((64, 48)).astype(np.float32) / 8, "rn")
    s, y = averis.averis_forward(x, wq["fwd"], "sr", seed=4)
    row = averis.dequantize(s["mean"]) @ averis.dequantize(wq["fwd"]).T
    np.testing.assert_array_equal(y, np.repeat(row, 20, axis=0))
    assert np.abs(row).max() > 0


def test_split_preserves_the_tail_better_than_vanilla():
    # the pages' argument ([Abstract]; [Lighthouse] §1.1): block scales set by
    # mean-driven extremes compress the tail; quantizing X - 1 mu^T instead
    # keeps it.  The residual's quantization error is far below the error of
    # quantizing X itself.
    cfg = workloads.up_proj(l=512, m=256, n=128)
    x = cfg["x"].float().numpy()
    s = averis.split_quant(x, "sr", seed=0)
    xr = averis.residual(x, s["mu"]).astype(np.float64)
    e_split = np.linalg.norm(averis.dequantize(s["residual"]) - xr)
    e_van = np.linalg.norm(averis.dequantize(averis.vanilla_quant(x, "sr", seed=0)) - x)
    assert e_split < 0.5 * e_van, (e_split, e_van)


def test_grouped_gemm_is_row_concatenation():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((30, 32)) + 1).astype(np.float32)
    offsets = [0, 12, 12, 30]
    ws = [averis.weight_quant(rng.standard_normal((32, 16)).astype(np.float32), "rn")["fwd"]
          for _ in range(3)]
    g = averis.split_quant_grouped(x, offsets, "sr", seed=2)
    y = averis.gemm_grouped(g["residual"], ws, g["mean"])
    assert y.shape == (30, 16)
    for s in range(3):
        r0, r1 = offsets[s], offsets[s + 1]
        if r1 > r0:
            np.testing.assert_array_equal(y[r0:r1], averis.gemm(g["residual"][s], ws[s], g["mean"][s]))
