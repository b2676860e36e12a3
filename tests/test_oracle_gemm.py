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


def q4_exact_rows(rng, rows, cols, t, anchor_p):
    """A (rows x cols) float64 matrix that Q4 (blocks of 16 along the rows)
    maps to itself, RN or SR: element (0, 0) is the anchor 2688 * 2^-p, alone
    in its block, which makes the tensor's amax 2688 * 2^-p and so S_enc = 2^p
    and S_dec = 2^-p exactly; every other element is g * 2^t with g on the
    E2M1 grid, and each other 16-run along a row holds one +-6 * 2^t (on the
    diagonal i = j mod 16), so its scale is the E4M3 power of two 2^(t + p) and
    its factor e_b = 2^-t is exact.  Needs -9 <= t + p <= 8.  Columns hold the
    same pattern (the diagonal runs down them too), so the transpose is Q4-exact
    along its rows as well, except for the anchor's column run, which is zero
    apart from the anchor."""
    g = np.array(GRID)[rng.integers(0, 7, size=(rows, cols))]   # |g| <= 4 off the diagonal
    g *= np.where(rng.random((rows, cols)) < 0.5, -1.0, 1.0)
    i, j = np.indices((rows, cols))
    g[(i % 16) == (j % 16)] = np.where(rng.random(((i % 16) == (j % 16)).sum()) < 0.5, -6.0, 6.0)
    m = g * 2.0 ** t
    m[0, :16] = 0.0
    m[:16, 0] = 0.0
    m[0, 0] = 2688.0 * 2.0 ** -anchor_p
    return m


def test_split_gemm_is_exact_when_q4_is_the_identity():
    # [Lighthouse] §2.2: Y = 1 (mean_q W_q) + X_R,q W_q.  On inputs whose mean,
    # residual and weight Q4 maps to themselves (and whose every product and
    # sum is exact in float64) the oracle's split forward and dgrad must equal
    # X W and D W^T exactly: this pins, through the oracle's own functions, the
    # mean, the residual, the rank-one row added to every output row, and the
    # orientation of both weight copies.
    rng = np.random.default_rng(11)
    l, m, n = 64, 64, 48
    w = q4_exact_rows(rng, m, n, -1, 9)                       # anchor 5.25, others <= 3
    # residual: row pairs +v, -v, so every column sums to exactly zero
    v = q4_exact_rows(rng, l // 2, m, -2, 8)                  # anchor 10.5, others <= 1.5
    r = np.empty((l, m))
    r[0::2], r[1::2] = v, -v
    mu = q4_exact_rows(rng, 1, m, 0, 7)[0]                    # anchor 21, others <= 6
    x = (r + mu[None, :]).astype(np.float32)
    assert np.array_equal(x.astype(np.float64), r + mu[None, :])   # exact in float32
    for rnd in ("rn", "sr"):
        wq = averis.weight_quant(w.astype(np.float32), rnd)
        np.testing.assert_array_equal(averis.dequantize(wq["fwd"]), w.T)
        np.testing.assert_array_equal(averis.dequantize(wq["dgrad"]), w)
        s, y = averis.averis_forward(x, wq["fwd"], rnd, seed=5)
        np.testing.assert_array_equal(s["mu"], mu.astype(np.float32))
        np.testing.assert_array_equal(averis.dequantize(s["residual"]), r)
        np.testing.assert_array_equal(averis.dequantize(s["mean"])[0], mu)
        np.testing.assert_array_equal(y, x.astype(np.float64) @ w)
        # dgrad: D (l x n) = its residual + 1 nu^T, dX = D W^T
        vd = q4_exact_rows(rng, l // 2, n, -3, 9)
        rd = np.empty((l, n))
        rd[0::2], rd[1::2] = vd, -vd
        nu = q4_exact_rows(rng, 1, n, -1, 8)[0]
        d = (rd + nu[None, :]).astype(np.float32)
        sd, dx = averis.averis_dgrad(d, wq["dgrad"], rnd, seed=6)
        np.testing.assert_array_equal(averis.dequantize(sd["residual"]), rd)
        np.testing.assert_array_equal(dx, d.astype(np.float64) @ w.T)
    # dropping the rank-one row (or adding it twice) breaks the equality
    wq = averis.weight_quant(w.astype(np.float32), "rn")
    s, y = averis.averis_forward(x, wq["fwd"], "rn", seed=5)
    no_mean = averis.gemm(s["residual"], wq["fwd"])
    assert not np.array_equal(no_mean, x.astype(np.float64) @ w)


def test_gemm_abs_bound_brute_force_tiny():
    # every GEMM parity test divides the error by this bound: pin it to a
    # triple loop over hand-decoded bytes, sum_k |a_ik| |b_jk| + |mean_k| |b_jk|
    cfg = workloads.tiny()
    x, d, w = cfg["x"].numpy(), cfg["d"].numpy(), cfg["w"].numpy()
    wq = averis.weight_quant(w, "rn")
    rng = np.random.default_rng(7)
    for a_in, b in ((x, wq["fwd"]), (d, wq["dgrad"])):
        s = averis.split_quant(a_in, "sr", seed=3)
        a, mu = s["residual"], s["mean"]
        bound = averis.gemm_abs_bound(a, b, mu)
        plain = averis.gemm_abs_bound(a, b)
        rows, k = a_in.shape
        n = b["codes"].shape[0]
        assert bound.shape == (rows, n)
        for i, j in zip(rng.integers(0, rows, 25), rng.integers(0, n, 25)):
            with_mean = no_mean = 0.0
            for kk in range(k):
                bjk = abs(decode_by_hand(b, j, kk))
                no_mean += abs(decode_by_hand(a, i, kk)) * bjk
                with_mean += abs(decode_by_hand(mu, 0, kk)) * bjk
            with_mean += no_mean
            assert abs(bound[i, j] - with_mean) <= 1e-12 * with_mean, (i, j)
            assert abs(plain[i, j] - no_mean) <= 1e-12 * no_mean, (i, j)
        # the bound dominates the product it measures
        c = averis.gemm(a, b, mu)
        assert (np.abs(c) <= bound * (1 + 1e-12)).all()


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
