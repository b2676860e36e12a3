"""Pins for oracle.formats: torch's float8_e4m3fn cast (an independent codec),
the E2M1 rounding boundaries written out by hand, and the statistical
properties that define stochastic rounding."""

import numpy as np
import pytest
import torch

from oracle import formats
from oracle.philox import sr_draw16


def torch_e4m3(x):
    t = torch.from_numpy(np.asarray(x, dtype=np.float32))
    return t.clamp(max=448.0).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_all_codes_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    mine = formats.e4m3_decode(codes)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(mine), nan)
    np.testing.assert_array_equal(mine[~nan], ref[~nan])


def test_e4m3_encode_midpoints_and_neighbours_match_torch():
    vals = np.sort(formats.e4m3_decode(np.arange(0, 0x7F, dtype=np.uint8)))  # 0 .. 448
    mids = (vals[:-1] + vals[1:]) / 2
    pts = np.concatenate([vals, mids]).astype(np.float32)
    # the midpoints and one float32 ulp either side of each
    cand = np.concatenate([pts, np.nextafter(pts, np.float32(np.inf)),
                           np.nextafter(pts, np.float32(0))])
    cand = cand[(cand >= 0) & np.isfinite(cand)]
    cand = np.concatenate([cand, np.float32([2.0 ** -10, 2.0 ** -11, 1e-30, 447.9, 448.0, 460.0,
                                             464.0, 1e4, 3e38])])
    np.testing.assert_array_equal(formats.e4m3_encode(cand), torch_e4m3(cand))


def test_e4m3_encode_random_matches_torch():
    rng = np.random.default_rng(1)
    x = np.exp2(rng.uniform(-14, 10, size=2_000_000)).astype(np.float32)
    np.testing.assert_array_equal(formats.e4m3_encode(x), torch_e4m3(x))


def test_e4m3_spot_values():
    # RNE with subnormals kept, saturation at 448
    got = formats.e4m3_encode(np.float32([2.0 ** -10, 1.0625, 1.1875, 460.0, 2.0 ** -9 * 1.5]))
    assert list(got) == [0x00, 0x38, 0x3A, 0x7E, 0x02]


# ---- E2M1 --------------------------------------------------------------

GRID = [0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0]
# RN decision boundaries between neighbours and the index a tie goes to (even)
BOUNDS = [(0.25, 0), (0.75, 2), (1.25, 2), (1.75, 4), (2.5, 4), (3.5, 6), (5.0, 6)]


def rn_by_boundaries(a):
    """Index of |v| by walking the hand-written boundary table."""
    idx = 0
    for b, tie_idx in BOUNDS:
        if a > b:
            idx = BOUNDS.index((b, tie_idx)) + 1
        elif a == b:
            return tie_idx
    return idx


def test_e2m1_rn_against_boundary_table():
    rng = np.random.default_rng(2)
    v = np.concatenate([rng.uniform(-7, 7, 20000).astype(np.float32),
                        np.float32([b for b, _ in BOUNDS] + [-b for b, _ in BOUNDS] + GRID),
                        np.float32([6.0, 6.5, 100.0, -0.0, 0.0, 1e-30])])
    codes = formats.e2m1_round_rn(v)
    for x, c in zip(v, codes):
        want = rn_by_boundaries(min(abs(float(x)), 6.0))
        assert c & 7 == want, (x, c)
        assert (c >> 3) == (1 if np.signbit(x) else 0)


def test_e2m1_decode_values():
    assert list(formats.e2m1_decode(np.arange(16))) == GRID + [-g for g in GRID]


def test_pack_unpack_roundtrip_and_order():
    c = np.array([[1, 2, 3, 4, 15, 0, 8, 7]], dtype=np.uint8)
    p = formats.pack_nibbles(c)
    assert list(p[0]) == [0x21, 0x43, 0x0F, 0x78]
    np.testing.assert_array_equal(formats.unpack_nibbles(p), c)


# ---- SR ----------------------------------------------------------------

def test_sr_on_grid_values_never_move():
    v = np.float32(GRID + [-g for g in GRID])
    for u in [0, 1, 32767, 65535]:
        np.testing.assert_array_equal(formats.e2m1_round_sr(v, np.full(v.shape, u)),
                                      formats.e2m1_round_rn(v))


def test_sr_result_is_a_neighbour_and_threshold_rule():
    rng = np.random.default_rng(3)
    v = rng.uniform(-6, 6, 50000).astype(np.float32)
    u = rng.integers(0, 65536, v.shape)
    c = formats.e2m1_round_sr(v, u)
    a = np.abs(v).astype(np.float64)
    got = np.array(GRID)[c & 7]
    lo = np.array([max(g for g in GRID if g <= x) for x in a])
    hi = np.array([min([g for g in GRID if g > x] or [6.0]) for x in a])
    assert np.all((got == lo) | (got == hi))
    # the draw that first rounds up: u >= 2^16 (1 - frac), compared exactly
    # with Python fractions on the float32 inputs
    from fractions import Fraction
    for x, uu, g in zip(a[:4000], u[:4000], got[:4000]):
        lo_x = max(gv for gv in GRID if gv <= x)
        hi_x = min([gv for gv in GRID if gv > x] or [6.0])
        if x >= 6.0 or x == lo_x:
            assert g == lo_x or x >= 6.0
            continue
        frac = (Fraction(float(x)) - Fraction(lo_x)) / (Fraction(hi_x) - Fraction(lo_x))
        assert (g == hi_x) == (int(2 ** 22 * frac) + 64 * int(uu) >= 2 ** 22), (x, uu)


def test_sr_exact_up_count_over_all_draws():
    # over all 2^16 draws, exactly floor(2^16 frac) round up (closed form)
    from fractions import Fraction
    rng = np.random.default_rng(11)
    vals = np.concatenate([rng.uniform(0, 6, 40), [1e-6, 0.2500001, 0.74999994, 5.9999995, 3.0000002]])
    u = np.arange(65536)
    for x in vals.astype(np.float32):
        c = formats.e2m1_round_sr(np.full(u.shape, x, dtype=np.float32), u)
        lo_x = max(gv for gv in GRID if gv <= float(x))
        hi_x = min([gv for gv in GRID if gv > float(x)] or [6.0])
        if float(x) >= 6.0:
            continue
        frac = (Fraction(float(x)) - Fraction(lo_x)) / (Fraction(hi_x) - Fraction(lo_x))
        n_up = int(np.count_nonzero(np.array(GRID)[c & 7] == hi_x)) if hi_x != lo_x else 0
        assert n_up == int(frac * 65536), (x, n_up, frac)
        # and the draws that round up are exactly the largest ones
        if n_up:
            assert np.all(np.array(GRID)[c[-n_up:] & 7] == hi_x)


def test_sr_up_frequency_and_unbiased_over_seeds():
    # E[deq(SR(v))] = v up to the 2^-16 draw resolution
    vals = np.float32([0.1, 0.37, 0.8, 1.2, 1.9, 2.25, 3.3, 4.9, 5.99, -0.6, -2.7])
    nseed = 4096
    idx = np.arange(vals.size, dtype=np.uint64)
    acc = np.zeros(vals.size)
    acc2 = np.zeros(vals.size)
    for s in range(nseed):
        d = formats.e2m1_decode(formats.e2m1_round_sr(vals, sr_draw16(s, 0, idx)))
        acc += d
        acc2 += d * d
    mean = acc / nseed
    sd = np.sqrt(np.maximum(acc2 / nseed - mean ** 2, 1e-12))
    gap = 2.0
    assert np.all(np.abs(mean - vals) <= 4 * sd / np.sqrt(nseed) + gap * 2.0 ** -16)


def test_sr_saturates_above_six():
    v = np.float32([6.0, 6.1, 9.0, -7.5])
    c = formats.e2m1_round_sr(v, np.zeros(4, dtype=np.int64))
    assert list(c) == [0x7, 0x7, 0x7, 0xF]
