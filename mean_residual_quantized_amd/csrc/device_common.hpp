// Device helpers shared by the libaveris kernels (gfx950): counter-based RNG
// and the E4M3 scale codec of the NVFP4-style Q4 (the E2M1 element rounding,
// RN and SR, is done by the hardware conversion instructions).
//
// Every operation that decides a code or a scale byte is a single IEEE fp32
// operation with round-to-nearest-even, in the order the format definition
// states (no contraction; this file is built with -ffp-contract=off).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace averis {

// ---------------------------------------------------------------------------
// Philox4x32-10 (Salmon et al., "Parallel random numbers: as easy as 1, 2, 3",
// SC'11): 10 rounds of two 32x32->64-bit multiplies and key mixing.  Each call
// gives 128 bits = eight 16-bit draws, for elements 8g .. 8g+7: element j
// takes word j >> 1, its low half for even j and its high half for odd j.
// ---------------------------------------------------------------------------
struct u32x4 {
  uint32_t x, y, z, w;
};

__device__ __forceinline__ u32x4 philox10(uint32_t c0, uint32_t c1, uint32_t c2, uint32_t c3,
                                           uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)c0 * 0xD2511F53u;
    const uint64_t p1 = (uint64_t)c2 * 0xCD9E8D57u;
    // three-input xors as one v_bitop3_b32 each (truth table 0x96 = a ^ b ^ c)
    const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
    const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
    c1 = (uint32_t)p1;
    c3 = (uint32_t)p0;
    c0 = n0;
    c2 = n2;
    k0 += 0x9E3779B9u;
    k1 += 0xBB67AE85u;
  }
  return {c0, c1, c2, c3};
}

// ---------------------------------------------------------------------------
// E4M3FN scale codec: bias 7, 3 mantissa bits, max 448, subnormals m * 2^-9.
// ---------------------------------------------------------------------------

// s: finite, >= 0, already capped at 448.  Round-to-nearest-even.
__device__ __forceinline__ uint32_t e4m3_encode(float s) {
  if (s < 0.015625f) {                       // below 2^-6: subnormal quanta of 2^-9
    return (uint32_t)__builtin_rintf(s * 512.0f);   // exact scaling; 8 -> 2^-6 = 0x08
  }
  const uint32_t b = __float_as_uint(s);
  // round the 23-bit mantissa to 3 bits, ties to even, carrying into the exponent
  const uint32_t r = (b + 0x7FFFFu + ((b >> 20) & 1u)) & ~0xFFFFFu;
  const uint32_t e = (r >> 23) - 127u + 7u;
  const uint32_t code = (e << 3) | ((r >> 20) & 7u);
  return code > 0x7Eu ? 0x7Eu : code;
}

__device__ __forceinline__ float e4m3_decode(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;            // m * 2^-9
  return __uint_as_float(((e + 120u) << 23) | (m << 20));  // (1 + m/8) 2^(e-7)
}

// ---------------------------------------------------------------------------
// Tensor scale from the tensor's max magnitude.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void tensor_scales(float amax, float& s_enc, float& s_dec) {
  float e = 1.0f;
  if (amax > 0.0f) {
    e = 2688.0f / amax;
    if (!__builtin_isfinite(e)) e = 1.0f;
  }
  s_enc = e;
  s_dec = 1.0f / e;
}

// amax / 6 rounded to nearest even, as the IEEE division gives it: from the
// rounded reciprocal and one FMA correction, which reproduces the quotient
// for every finite amax >= 2^-125 (checked against the division for every
// fp32 value); smaller inputs (subnormal quotients) take the division.
__device__ __forceinline__ float div6(float amax) {
  if (__builtin_expect(amax < 0x1p-125f, 0)) return amax / 6.0f;
  const float c = 1.0f / 6.0f;
  const float q = amax * c;
  return __builtin_fmaf(__builtin_fmaf(-q, 6.0f, amax), c, q);
}

// E4M3 scale byte of a block (no element factor): the first steps of
// block_scale
__device__ __forceinline__ uint32_t block_scale_code(float amax_b, float s_enc) {
  float s = div6(amax_b);
  s = s * s_enc;
  s = __builtin_fminf(s, 448.0f);
  return e4m3_encode(s);
}

// Element factors of a tensor scale: tab[code] = s_enc / e4m3_decode(code)
// (0 for code 0), the division block_scale does, for every code a block can
// get (0 .. 0x7E); filled by the first 127 threads of a workgroup.
__device__ __forceinline__ void fill_eb_table(float s_enc, float* tab) {
  const uint32_t t = threadIdx.x;
  if (t < 127) {
    const float d = e4m3_decode(t);
    tab[t] = d > 0.0f ? s_enc / d : 0.0f;
  }
}

// Block scale byte and element factor from the block's max magnitude.
__device__ __forceinline__ void block_scale(float amax_b, float s_enc, uint32_t& code, float& e_b) {
  float s = div6(amax_b);
  s = s * s_enc;
  s = __builtin_fminf(s, 448.0f);
  code = e4m3_encode(s);
  const float d = e4m3_decode(code);
  e_b = d > 0.0f ? s_enc / d : 0.0f;
}

// bf16 bits -> fp32 (exact)
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Order-preserving map of fp32 to uint32 (for max/min via unsigned compares).
__device__ __forceinline__ uint32_t f32_ordered(float f) {
  const uint32_t b = __float_as_uint(f);
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}
__device__ __forceinline__ float f32_from_ordered(uint32_t o) {
  return __uint_as_float((o & 0x80000000u) ? (o & 0x7FFFFFFFu) : ~o);
}

}  // namespace averis
