"""Element and scale codecs for the NVFP4-style Q4 operator (oracle side).

TEST INFRASTRUCTURE ONLY (see oracle/__init__.py).

[Lighthouse] §3.1 fixes the element format as E2M1 (NVFP4); [NVFP4-outliers]
says NVFP4 uses two-level ("hierarchical") microscaling.  The pages give no
bit-level rules, so the readings below are the oracle's:

* E2M1 magnitudes, index 0..7: {0, 0.5, 1, 1.5, 2, 3, 4, 6}; a code is
  sign << 3 | index, so a negative value that rounds to 0 keeps its sign (0x8).
* Round-to-nearest (RN): nearest grid point; a value exactly half-way between
  two grid points goes to the even index; |v| >= 6 saturates to 6.
* Stochastic rounding (SR): with lo the largest grid point <= |v|, hi the
  next one and frac = (|v| - lo) / (hi - lo), the element's 16-bit draw u
  rounds up iff floor(2^22 frac) + 2^6 u >= 2^22 (a 22-bit dither added to
  the fraction of the step, with the draw in its top 16 bits).  Exactly
  floor(2^16 frac) of the 2^16 draws round up (P(up) = floor(2^16 frac) /
  2^16, a bias below 2^-16 of a gap); |v| == lo never moves; |v| >= 6
  saturates to 6.
* Block scales are E4M3FN (bias 7, no infinities, max 448, subnormals kept,
  smallest 2^-9), round-to-nearest-even, saturating at 448.
"""

import numpy as np

E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
E4M3_MAX = 448.0


def e4m3_encode(s):
    """Encode non-negative values to E4M3FN byte codes (RNE, saturate at 448)."""
    s = np.asarray(s, dtype=np.float64)
    if np.any(s < 0) or not np.all(np.isfinite(s)):
        raise ValueError("e4m3_encode expects finite non-negative values")
    s = np.minimum(s, E4M3_MAX)
    codes = np.zeros(s.shape, dtype=np.int64)
    nz = s > 0
    mant, ex = np.frexp(s[nz])                  # s = mant * 2^ex, mant in [0.5, 1)
    e = ex.astype(np.int64) - 1                 # s in [2^e, 2^(e+1))
    sub = e < -6
    # subnormal binade: quantum 2^-9, code = number of quanta (8 -> 2^-6, normal)
    q_sub = np.rint(s[nz] * 2.0 ** 9)           # exact scaling; rint is ties-to-even
    # normal binades: quantum 2^(e-3), q in [8, 16]
    q_nrm = np.rint(np.ldexp(s[nz], (3 - e)))
    carry = q_nrm >= 16
    e_n = np.where(carry, e + 1, e)
    q_n = np.where(carry, 8.0, q_nrm)
    c_nrm = ((e_n + 7) << 3) | (q_n.astype(np.int64) - 8)
    codes[nz] = np.where(sub, q_sub.astype(np.int64), c_nrm)
    return codes.astype(np.uint8)


def e4m3_decode(c):
    """Decode E4M3FN byte codes (sign bit honoured; 0x7F/0xFF are NaN)."""
    c = np.asarray(c, dtype=np.int64)
    e = (c >> 3) & 15
    m = c & 7
    mag = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((c & 0x7F) == 0x7F, np.nan, mag)
    return np.where(c & 0x80, -mag, mag)


def e2m1_decode(code):
    """Value of 4-bit E2M1 codes (float64)."""
    code = np.asarray(code, dtype=np.int64)
    mag = E2M1_GRID[code & 7]
    return np.where(code & 8, -mag, mag)


def e2m1_round_rn(v):
    """RN codes for float32 values v (already multiplied by the block factor)."""
    v = np.asarray(v, dtype=np.float32)
    a = np.abs(v).astype(np.float64)
    dist = np.abs(a[..., None] - E2M1_GRID)            # (..., 8), exact
    idx = np.argmin(dist, axis=-1)                    # first (lowest) index on ties
    # a tie is always between neighbours i, i+1; move to the even one
    nxt = np.minimum(idx + 1, 7)
    d_idx = np.take_along_axis(dist, idx[..., None], -1)[..., 0]
    d_nxt = np.take_along_axis(dist, nxt[..., None], -1)[..., 0]
    idx = np.where((idx % 2 == 1) & (nxt != idx) & (d_nxt == d_idx), nxt, idx)
    idx = np.where(a >= 6.0, 7, idx)
    sign = np.signbit(v).astype(np.int64)
    return ((sign << 3) | idx).astype(np.uint8)


def e2m1_round_sr(v, u16):
    """SR codes for float32 values v with per-element 16-bit draws u16.

    lo is the largest grid point <= |v|, hi the next one, and
    frac = (|v| - lo) / (hi - lo) in [0, 1).  The 16-bit draw u rounds up iff
        floor(2^22 frac) + 2^6 u >= 2^22,
    i.e. iff u >= 2^16 (1 - frac): over the 2^16 draws, exactly
    floor(2^16 frac) of them round up, so the rounding is unbiased to within
    2^-16 of a step.  A value on the grid never moves; |v| >= 6 gives 6.
    """
    v = np.asarray(v, dtype=np.float32)
    u = np.asarray(u16, dtype=np.float64)
    a = np.abs(v).astype(np.float64)
    lo = np.searchsorted(E2M1_GRID, a, side="right") - 1   # largest grid point <= a
    lo = np.clip(lo, 0, 7)
    hi = np.minimum(lo + 1, 7)
    g_lo = E2M1_GRID[lo]
    gap = np.where(hi > lo, E2M1_GRID[hi] - g_lo, 1.0)     # a power of two
    # (a - g_lo) is exact in float64 and the scaling by 2^22 / gap is a power
    # of two, so f22 is the exact floor
    f22 = np.floor((a - g_lo) * (4194304.0 / gap))
    up = (f22 + 64.0 * u >= 4194304.0) & (hi > lo)
    idx = np.where(a >= 6.0, 7, lo + up.astype(np.int64))
    sign = np.signbit(v).astype(np.int64)
    return ((sign << 3) | idx).astype(np.uint8)


def pack_nibbles(codes):
    """Pack 4-bit codes along the last axis: byte j = code[2j] | code[2j+1] << 4."""
    codes = np.asarray(codes, dtype=np.uint8)
    return (codes[..., 0::2] | (codes[..., 1::2] << 4)).astype(np.uint8)


def unpack_nibbles(packed):
    """Inverse of pack_nibbles."""
    packed = np.asarray(packed, dtype=np.uint8)
    out = np.empty(packed.shape[:-1] + (packed.shape[-1] * 2,), dtype=np.uint8)
    out[..., 0::2] = packed & 0x0F
    out[..., 1::2] = packed >> 4
    return out
