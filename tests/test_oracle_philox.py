"""Pins for oracle.philox: rocRAND's independent Philox4x32-10 engine, plus
the draw layout and a uniformity check of the 16-bit draws."""

import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.philox import MASK32, philox4x32_10, sr_draw16

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc):
        pytest.skip("hipcc not available to build the rocRAND reference")
    exe = str(tmp_path_factory.mktemp("rr") / "rocrand_philox_ref")
    src = os.path.join(HERE, "pins", "rocrand_philox_ref.cpp")
    # host-only program; HIP mode is needed for rocRAND's headers
    subprocess.run([hipcc, "-x", "hip", "--offload-arch=gfx950", "-O1", src, "-o", exe],
                   check=True, capture_output=True)

    def run(seed, stream, gs):
        out = subprocess.run([exe, str(seed), str(stream)] + [str(g) for g in gs],
                             check=True, capture_output=True, text=True).stdout
        return np.array([[int(w) for w in line.split()] for line in out.strip().splitlines()],
                        dtype=np.uint64)
    return run


@pytest.mark.parametrize("seed", [0, 1, 0x123456789ABCDEF0, 0xFFFFFFFFFFFFFFFF])
@pytest.mark.parametrize("stream", [0, 1, 2])
def test_philox_matches_rocrand(rocrand_ref, seed, stream):
    rng = np.random.default_rng(seed & 0xFFFF)
    gs = [0, 1, 2, 7, 2**32 - 1, 2**32, 2**40 + 3] + list(rng.integers(0, 2**45, size=9))
    ref = rocrand_ref(seed, stream, gs)
    g = np.array(gs, dtype=np.uint64)
    mine = np.stack(philox4x32_10(g & np.uint64(MASK32), g >> np.uint64(32), stream, 0,
                                  seed & MASK32, seed >> 32), axis=-1).astype(np.uint64)
    np.testing.assert_array_equal(mine, ref)


def test_draw_layout_uses_each_half_word_once(rocrand_ref):
    # element idx -> word (idx >> 1) & 3, half idx & 1, block g = idx >> 3
    seed, stream = 0xDEADBEEF12345, 1
    ref = rocrand_ref(seed, stream, [5])[0]
    idx = np.arange(40, 48, dtype=np.uint64)          # g = 5
    u = sr_draw16(seed, stream, idx)
    expect = []
    for w in range(4):
        expect += [int(ref[w]) & 0xFFFF, int(ref[w]) >> 16]
    np.testing.assert_array_equal(u, np.array(expect, dtype=np.uint32))


def test_draws_depend_on_seed_stream_index():
    idx = np.arange(4096, dtype=np.uint64)
    a = sr_draw16(7, 0, idx)
    assert not np.array_equal(a, sr_draw16(8, 0, idx))
    assert not np.array_equal(a, sr_draw16(7, 1, idx))
    np.testing.assert_array_equal(a[100:200], sr_draw16(7, 0, idx[100:200]))


def test_draws_uniform_chi2():
    # 2^18 draws in 256 bins of the top byte: chi^2 with 255 dof
    u = sr_draw16(42, 0, np.arange(2**18, dtype=np.uint64))
    counts = np.bincount(u >> 8, minlength=256)
    exp = len(u) / 256
    chi2 = float(((counts - exp) ** 2 / exp).sum())
    assert 180 < chi2 < 340, chi2
    assert u.max() < 65536
