// Exact summation of fp32 values and of exact fp64 partial sums of them, in
// a signed 320-bit integer, rounded once to the nearest double.
//
// Every fp32 value is an integer multiple of 2^-149 below 2^128, so a sum of
// up to 2^31 of them is an integer multiple of 2^-149 of magnitude below
// 2^159, which a 320-bit two's-complement integer in units of 2^-149 holds
// exactly.  An fp64 value that is itself an exact sum of fp32 values is such
// a multiple too, so it can be added exactly as well.  The final rounding is
// to nearest, ties to even: the correctly rounded sum (what math.fsum gives).
//
// Host and device: the same functions are compiled into the kernels and, for
// the tests, into a host program.
#pragma once

#include <stdint.h>

#if defined(__HIPCC__)
#include <hip/hip_runtime.h>
#define AVERIS_HD __host__ __device__
#else
#define AVERIS_HD
#endif

namespace averis {

constexpr int kWideWords = 10;

// acc += (neg ? -1 : 1) * mant * 2^s  (mant < 2^53, 0 <= s, s + 53 < 320)
AVERIS_HD inline void wide_add_bits(uint32_t (&acc)[kWideWords], uint64_t mant, int s, bool neg) {
  const int w = s >> 5, b = s & 31;
  // mant << b spans at most 84 bits: three words
  const uint64_t lo = mant << b;
  const uint32_t hi = b ? (uint32_t)(mant >> (64 - b)) : 0u;
  const uint32_t part[3] = {(uint32_t)lo, (uint32_t)(lo >> 32), hi};
  uint64_t carry = 0;
  if (!neg) {
#pragma unroll
    for (int i = 0; i < kWideWords; ++i) {
      const int k = i - w;
      const uint32_t add = (k >= 0 && k < 3) ? part[k] : 0u;
      const uint64_t sum = (uint64_t)acc[i] + add + carry;
      acc[i] = (uint32_t)sum;
      carry = sum >> 32;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kWideWords; ++i) {
      const int k = i - w;
      const uint32_t sub = (k >= 0 && k < 3) ? part[k] : 0u;
      const uint64_t d = (uint64_t)acc[i] - sub - carry;
      acc[i] = (uint32_t)d;
      carry = (d >> 32) ? 1u : 0u;
    }
  }
}

// acc += v (any finite fp32 value)
AVERIS_HD inline void wide_add_f32(uint32_t (&acc)[kWideWords], float v) {
  const uint32_t bits = __builtin_bit_cast(uint32_t, v);
  const uint32_t e = (bits >> 23) & 0xFFu, m = bits & 0x7FFFFFu;
  if (e == 0 && m == 0) return;
  // value = mant * 2^(shift - 149)
  const uint64_t mant = e ? (m | 0x800000u) : m;
  const int shift = e ? (int)e - 1 : 0;
  wide_add_bits(acc, mant, shift, (bits >> 31) != 0);
}

// acc += v, v a finite fp64 value that is an integer multiple of 2^-149
// below 2^159 in magnitude (an exact sum of fp32 values)
AVERIS_HD inline void wide_add_f64(uint32_t (&acc)[kWideWords], double v) {
  const uint64_t bits = __builtin_bit_cast(uint64_t, v);
  const int e = (int)((bits >> 52) & 0x7FFu);
  uint64_t mant = bits & ((1ull << 52) - 1);
  if (e == 0 && mant == 0) return;
  if (e) mant |= 1ull << 52;
  // value = mant * 2^(e - 1075) = mant * 2^(s) units of 2^-149, s = e - 926
  // (e = 0, an fp64 subnormal, is not a multiple of 2^-149 and does not occur)
  int s = e - 926;
  if (s < 0) {
    mant >>= -s;   // the dropped bits are zero for a multiple of 2^-149
    s = 0;
  }
  wide_add_bits(acc, mant, s, (bits >> 63) != 0);
}

AVERIS_HD inline void wide_add(uint32_t (&acc)[kWideWords], const uint32_t* other) {
  uint64_t carry = 0;
#pragma unroll
  for (int i = 0; i < kWideWords; ++i) {
    const uint64_t sum = (uint64_t)acc[i] + other[i] + carry;
    acc[i] = (uint32_t)sum;
    carry = sum >> 32;
  }
}

// bits [lo, lo + 64) of the magnitude (bits past the top read as 0)
AVERIS_HD inline uint64_t wide_bits64(const uint32_t (&a)[kWideWords], int lo) {
  uint64_t r = 0;
#pragma unroll
  for (int i = 0; i < kWideWords; ++i) {
    const int off = 32 * i - lo;   // position of word i's bit 0 in the result
    if (off >= 64 || off <= -32) continue;
    const uint64_t wv = a[i];
    r |= off >= 0 ? (wv << off) : (wv >> -off);
  }
  return r;
}

// the accumulated value rounded to the nearest double, ties to even
// (destroys acc)
AVERIS_HD inline double wide_to_double(uint32_t (&a)[kWideWords]) {
  const bool neg = a[kWideWords - 1] >> 31;
  if (neg) {   // magnitude: two's complement negation
    uint64_t carry = 1;
#pragma unroll
    for (int i = 0; i < kWideWords; ++i) {
      const uint64_t v = (uint64_t)(~a[i]) + carry;
      a[i] = (uint32_t)v;
      carry = v >> 32;
    }
  }
  int p = -1;   // highest set bit
#pragma unroll
  for (int i = 0; i < kWideWords; ++i)
    if (a[i]) p = 32 * i + 31 - __builtin_clz(a[i]);
  if (p < 0) return 0.0;
  double r;
  if (p < 53) {
    r = __builtin_ldexp((double)wide_bits64(a, 0), -149);   // exact
  } else {
    uint64_t mant = wide_bits64(a, p - 52) & ((1ull << 53) - 1);
    const bool round = (wide_bits64(a, p - 53) & 1ull) != 0;
    bool sticky = false;
    for (int b = 0; b < p - 53; b += 64) {
      const int n = p - 53 - b;
      const uint64_t chunk = wide_bits64(a, b);
      sticky = sticky || (n >= 64 ? chunk != 0 : (chunk & ((1ull << n) - 1)) != 0);
    }
    int ex = p - 52 - 149;
    if (round && (sticky || (mant & 1ull))) {
      mant += 1;
      if (mant >> 53) {
        mant >>= 1;
        ex += 1;
      }
    }
    r = __builtin_ldexp((double)mant, ex);
  }
  return neg ? -r : r;
}

// ---------------------------------------------------------------------------
// A narrower exact path for a column whose values all lie on one grid: every
// value is a multiple of 2^gexp (gexp from the column's smallest nonzero
// magnitude) and every partial sum is below 2^62 units of it, so the sum in
// units of 2^gexp is exact in a signed 64-bit integer, in any order.
// ---------------------------------------------------------------------------

// exponent of the grid that every value of a column lies on, from its
// smallest nonzero magnitude mnz (p = 7 for bf16 values, 23 for fp32): a
// value with binary exponent e (in [2^(e-1), 2^e)) and p fraction bits is a
// multiple of 2^(e - 1 - p), and e >= that of mnz
AVERIS_HD inline int value_grid_exp(float mnz, int p) {
  int e;
  (void)__builtin_frexp((double)mnz, &e);
  return e - 1 - p;
}

// whether n values of magnitude <= amax on the grid 2^gexp sum exactly in a
// signed 64-bit integer (a margin of one bit for the rounding of n * amax)
AVERIS_HD inline bool grid_sum_fits(double n, double amax, int gexp) {
  return n * amax <= __builtin_ldexp(1.0, 61 + gexp);
}

// v / 2^gexp as an integer (v an exact multiple of 2^gexp, |v / 2^gexp| < 2^62)
AVERIS_HD inline int64_t grid_int64(double v, int gexp) {
  const double t = __builtin_ldexp(v, -gexp);                 // an integer-valued double
  const double hi = __builtin_floor(t * 0x1p-32);             // exact
  const double lo = t - hi * 0x1p32;                          // exact, in [0, 2^32)
  return (int64_t)((uint64_t)(int64_t)(int32_t)hi << 32) + (int64_t)(uint32_t)lo;
}

// n 2^gexp rounded once to the nearest double, ties to even (the scale by
// 2^gexp is exact: the results here are far from the fp64 range's ends)
AVERIS_HD inline double grid_int64_to_double(int64_t n, int gexp) {
  const double hi = (double)(int32_t)(n >> 32) * 0x1p32;      // exact
  const double lo = (double)(uint32_t)(uint64_t)n;            // exact
  return __builtin_ldexp(hi + lo, gexp);                      // one rounding
}

}  // namespace averis
