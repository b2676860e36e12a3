"""The exact column-sum arithmetic the split-quant kernels fall back on
(csrc/exact_sum.hpp: a 64-bit integer in units of the column's grid where the
sum fits, else a 320-bit integer in units of 2^-149, either rounded once),
built for the host with g++ and checked against Python's exact rationals:
fp32 values over the whole exponent range with cancellation, subnormals and
the largest magnitudes, and exact fp64 partial sums mixed with fp32 values.
Python's float(Fraction) is the correctly rounded value, as math.fsum."""

import os
import shutil
import struct
import subprocess
from fractions import Fraction

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "mean_residual_quantized_amd", "csrc")


@pytest.fixture(scope="module")
def driver(tmp_path_factory):
    cxx = shutil.which("g++")
    if cxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path_factory.mktemp("exact") / "exact_sum_driver")
    subprocess.run([cxx, "-O2", "-std=c++17", "-Wno-unknown-pragmas", "-I" + CSRC,
                    os.path.join(ROOT, "tests", "host", "exact_sum_driver.cpp"), "-o", exe],
                   check=True)
    return exe


def run(exe, cases):
    lines = []
    for f32s, f64s in cases:
        b32 = np.asarray(f32s, dtype=np.float32).view(np.uint32)
        b64 = np.asarray(f64s, dtype=np.float64).view(np.uint64)
        lines.append(" ".join([str(len(b32)), str(len(b64))] + ["%x" % v for v in b32] +
                              ["%x" % v for v in b64]))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.splitlines()
    return [struct.unpack("<d", int(ln.split()[0], 16).to_bytes(8, "little"))[0] for ln in out]


def run_grid(exe, cases):
    """The 64-bit grid sum of each case (None where its grid does not fit)."""
    lines = []
    for f32s, f64s in cases:
        b32 = np.asarray(f32s, dtype=np.float32).view(np.uint32)
        b64 = np.asarray(f64s, dtype=np.float64).view(np.uint64)
        lines.append(" ".join([str(len(b32)), str(len(b64))] + ["%x" % v for v in b32] +
                              ["%x" % v for v in b64]))
    out = subprocess.run([exe], input="\n".join(lines) + "\n", capture_output=True, text=True,
                         check=True).stdout.splitlines()
    res = []
    for ln in out:
        t = ln.split()[1]
        res.append(None if t == "x" else struct.unpack("<d", int(t, 16).to_bytes(8, "little"))[0])
    return res


def exact(f32s, f64s):
    s = sum((Fraction(float(v)) for v in np.asarray(f32s, dtype=np.float32)), Fraction(0))
    s += sum((Fraction(float(v)) for v in f64s), Fraction(0))
    return float(s)


def random_f32(rng, n, lo=-149, hi=127):
    """fp32 values m * 2^e, m uniform in [1, 2), e uniform in [lo, hi), random
    signs (exponents below -126 give subnormals)."""
    m = 1.0 + rng.random(n)
    e = rng.integers(lo, hi, size=n)
    v = np.ldexp(m, e)
    v = np.where(rng.random(n) < 0.5, -v, v).astype(np.float32)
    return v[np.isfinite(v)]


def test_fp32_sums_are_correctly_rounded(driver):
    rng = np.random.default_rng(0)
    cases = []
    for n in (1, 2, 7, 64, 500):
        for lo, hi in ((-149, 127), (-30, 30), (-149, -120), (100, 127)):
            cases.append((random_f32(rng, n, lo, hi), []))
    # cancellation down to a single low bit, and the ends of the range
    big = np.float32(2.0 ** 127)
    cases.append(([big, 1.0, -big, np.float32(2.0 ** -149)], []))
    cases.append(([3e38, 3e38, 3e38, -3e38, 1e-45], []))
    cases.append(([2.0 ** 100, 1.0, -(2.0 ** 100), 1.0, 0.0], []))
    cases.append(([1.0] * 3 + [np.float32(2.0 ** -24)] * 5, []))
    cases.append(([], []))
    got = run(driver, cases)
    for (f32s, f64s), g in zip(cases, got):
        assert g == exact(f32s, f64s), (list(f32s)[:4], g)


def test_exact_fp64_partials_mix_with_fp32_values(driver):
    # the fallback adds the chunks' exact fp64 partial sums and the rows of the
    # chunks whose own partial was not exact
    rng = np.random.default_rng(1)
    cases = []
    for _ in range(40):
        parts = []
        for _ in range(rng.integers(1, 9)):
            lo = int(rng.integers(-140, 60))
            chunk = random_f32(rng, int(rng.integers(1, 64)), lo, lo + 20)
            chunk = chunk[np.abs(chunk) >= np.ldexp(np.float32(1), -149)]
            chunk = chunk * np.float32(2.0 ** int(rng.integers(0, 40)))
            fr = sum((Fraction(float(v)) for v in chunk), Fraction(0))
            if float(fr) == fr:            # an exact fp64 partial, as a certified chunk gives
                parts.append(float(fr))
        rows = random_f32(rng, int(rng.integers(0, 50)), -149, 127)
        cases.append((rows, parts))
    # a partial spanning the full fp64 mantissa and a subnormal-unit partial
    cases.append(([np.float32(-(2.0 ** -149))], [float(2 ** 60 + 1) * 2.0 ** -149, 2.0 ** -149]))
    cases.append(([], [-(2.0 ** 158), 2.0 ** 158, 3.0 * 2.0 ** -149]))
    got = run(driver, cases)
    for (f32s, f64s), g in zip(cases, got):
        assert g == exact(f32s, f64s)


def test_grid_sum_is_correctly_rounded_where_it_fits(driver):
    # the 64-bit path the fallback takes first: every value a multiple of the
    # grid of the smallest nonzero magnitude, the total below 2^62 grid units;
    # with fp32's 24-bit significands, n values spanning s binades need about
    # s + 24 + log2(n) bits: 54-60 here, so the double result is rounded (and a
    # plain fp64 running sum is not exact)
    rng = np.random.default_rng(2)
    cases = []
    for n, span in ((2, 35), (10, 32), (40, 29)):
        for _ in range(4):
            lo = int(rng.integers(-100, 40))
            # large values near the top of the span, two small ones at its foot
            v = np.concatenate([random_f32(rng, n, lo + span - 4, lo + span),
                                random_f32(rng, 2, lo, lo + 1)])
            cases.append((v, []))
    # values that cancel to a few grid units, and ties of the final rounding:
    # 2^53 + 1 grid units is exactly halfway between two doubles
    g = np.float32(2.0 ** -20)
    cases.append(([np.float32(2.0 ** 20), g, np.float32(-(2.0 ** 20))], []))
    cases.append(([np.float32(2.0 ** 33), g], []))                      # ties to even: down
    cases.append(([np.float32(2.0 ** 33), np.float32(3 * 2.0 ** -20)], []))   # ties to even: up
    cases.append(([np.float32(1.0), np.float32(2.0 ** -24), np.float32(2.0 ** -24)], [2.0 ** 29]))
    # exact fp64 partials on the grid mixed with fp32 values
    for _ in range(20):
        vals = random_f32(rng, 200, -5, 22)
        parts = []
        for k in range(0, 200, 40):
            fr = sum((Fraction(float(x)) for x in vals[k:k + 40]), Fraction(0))
            if float(fr) == fr:
                parts.append(float(fr))
        # the grid comes from the smallest magnitude of every value summed,
        # partials included (the kernel takes it over all of a column's chunks)
        cases.append((np.append(vals[:20], vals[np.argmin(np.abs(vals))]), parts))
    got = run_grid(driver, cases)
    wide = run(driver, cases)
    fitted = rounded = 0
    for (f32s, f64s), g64, w in zip(cases, got, wide):
        if g64 is None:
            continue
        fitted += 1
        fr = sum((Fraction(float(v)) for v in np.asarray(f32s, dtype=np.float32)), Fraction(0))
        fr += sum((Fraction(float(v)) for v in f64s), Fraction(0))
        rounded += float(fr) != fr
        assert g64 == exact(f32s, f64s), (list(f32s)[:4], g64)
        assert g64 == w
    assert fitted >= len(cases) - 4
    assert rounded >= 5       # the cases test the final rounding, not only exact sums
    # and where the grid does not fit, the driver says so: a 2^70 span
    assert run_grid(driver, [([np.float32(2.0 ** 50), np.float32(2.0 ** -30)], [])]) == [None]
