// Quantized NT GEMM with the rank-one mean term for gfx950.
//
// Forward and dgrad of the Averis linear ("Lighthouse" review §2.2):
//   Y  = 1 (mean_q W_q)   + X_R,q W_q
//   dX = 1 (mean_q,D W_q^T) + D_R,q W_q^T
// both as C = deq(A) deq(B)^T + 1 rho^T with A = the quantized residual
// (rows x K) and B the quantized weight copy stored N x K (K contiguous).
//
// Exactness of the operands: an E2M1 value (at most 2 significant bits) times
// an E4M3 scale (4 significant bits) has at most 6 significant bits and lies
// in [2^-10, 2688], so it is exact in fp16; the MFMA's fp16 x fp16 products
// are exact in fp32.  The tensor scales S_dec(A) S_dec(B) are applied once in
// the epilogue, so the only roundings are the fp32 accumulation and the
// epilogue.  CDNA4's scaled FP4 MFMA takes E8M0 scales per 32 elements and
// cannot apply E4M3 scales per 16; the exact operands therefore run on
// v_mfma_f32_32x32x16_f16.
//
// rho_j = S_dec(mean) S_dec(B) sum_k deq'(mean)_k deq'(B)_jk comes from a
// small GEMV kernel and is added in the GEMM epilogue as a broadcast row.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"
#include "segments.hpp"

namespace averis {

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int LDSK = BK + 8;  // fp16 per LDS row (16-byte pad against bank conflicts)

// fp16 bit pattern of an E2M1 code: magnitude index c = e m (2+1 bits);
// e > 0: 2^(e-1) (1 + m/2) -> exponent e + 14, mantissa m << 9; e = 0: m/2.
__device__ __forceinline__ uint32_t e2m1_f16_bits(uint32_t code) {
  const uint32_t c = code & 7u, e = c >> 1, m = c & 1u;
  const uint32_t mag = e ? (((e + 14u) << 10) | (m << 9)) : (m ? 0x3800u : 0u);
  return mag | ((code & 8u) << 12);
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  if (e == 0) return (float)m * 0.001953125f;
  return __uint_as_float(((e + 120u) << 23) | (m << 20));
}

// 8 codes (one dword) times a block scale -> 8 fp16 (exact)
__device__ __forceinline__ uint4 dequant8(uint32_t w, _Float16 s) {
  uint32_t out[4];
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const uint32_t lo = e2m1_f16_bits((w >> (8 * p)) & 0xFu);
    const uint32_t hi = e2m1_f16_bits((w >> (8 * p + 4)) & 0xFu);
    const _Float16 a = __builtin_bit_cast(_Float16, (uint16_t)lo) * s;
    const _Float16 b = __builtin_bit_cast(_Float16, (uint16_t)hi) * s;
    out[p] = (uint32_t)__builtin_bit_cast(uint16_t, a) |
             ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
  }
  return make_uint4(out[0], out[1], out[2], out[3]);
}

// Load one thread's share of an operand tile (row r of the tile, 32
// consecutive k from kb) and store it dequantized to LDS.
__device__ __forceinline__ void stage_rows(const uint8_t* codes, const uint8_t* scales,
                                           int64_t row, bool row_ok, int64_t k, int64_t kb,
                                           _Float16* lds_row) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int64_t kk = kb + 8 * q;
    uint32_t w = 0;
    _Float16 s = (_Float16)0.0f;
    if (row_ok && kk < k) {
      w = *reinterpret_cast<const uint32_t*>(codes + row * (k >> 1) + (kk >> 1));
      s = (_Float16)e4m3_value(scales[row * (k >> 4) + (kk >> 4)]);
    }
    *reinterpret_cast<uint4*>(lds_row + 8 * q) = dequant8(w, s);
  }
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

}  // namespace

template <bool OUT_BF16, bool HAS_MEAN>
__global__ __launch_bounds__(256) void k_gemm_nt(QOperand A, QOperand B, int64_t m, int64_t n,
                                                 int64_t k, const int64_t* offs, int nseg,
                                                 const float* __restrict__ rho, void* c,
                                                 int64_t ldc) {
  __shared__ __attribute__((aligned(16))) _Float16 As[BM * LDSK];
  __shared__ __attribute__((aligned(16))) _Float16 Bs[BN * LDSK];

  const SegRange sr = locate_chunk(offs, nseg, m, BM, blockIdx.y);
  if (sr.seg < 0) return;
  const int seg = sr.seg;
  const int64_t m0 = sr.r0, m_end = sr.r1;
  const int64_t n0 = (int64_t)blockIdx.x * BN;
  const uint8_t* bcodes = B.codes + (offs ? (int64_t)seg * n * (k >> 1) : 0);
  const uint8_t* bscales = B.scales + (offs ? (int64_t)seg * n * (k >> 4) : 0);

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w >> 1, wn = w & 1;
  const int srow = t >> 1, shalf = t & 1;

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  for (int64_t k0 = 0; k0 < k; k0 += BK) {
    stage_rows(A.codes, A.scales, m0 + srow, m0 + srow < m_end, k, k0 + 32 * shalf,
               As + srow * LDSK + 32 * shalf);
    stage_rows(bcodes, bscales, n0 + srow, n0 + srow < n, k, k0 + 32 * shalf,
               Bs + srow * LDSK + 32 * shalf);
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      half8_t af[2], bf[2];
#pragma unroll
      for (int i = 0; i < 2; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(
            As + (wm * 64 + i * 32 + (lane & 31)) * LDSK + kk + (lane >> 5) * 8);
#pragma unroll
      for (int j = 0; j < 2; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(
            Bs + (wn * 64 + j * 32 + (lane & 31)) * LDSK + kk + (lane >> 5) * 8);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(af[i], bf[j], acc[i][j], 0, 0, 0);
    }
    __syncthreads();
  }

  const float alpha = A.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
      if (col >= n) continue;
      const float r1 = HAS_MEAN ? rho[(int64_t)seg * n + col] : 0.0f;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int64_t row = m0 + wm * 64 + i * 32 + (v >> 2) * 8 + (lane >> 5) * 4 + (v & 3);
        if (row >= m_end) continue;
        const float y = acc[i][j][v] * alpha + r1;
        if (OUT_BF16)
          static_cast<uint16_t*>(c)[row * ldc + col] = f32_to_bf16_rne(y);
        else
          static_cast<float*>(c)[row * ldc + col] = y;
      }
    }
}

// rho[seg][j] = S_dec(mean_seg) S_dec(B_seg) sum_k deq'(mean_seg)_k deq'(B_seg)_jk
// one wavefront per output column j
__global__ __launch_bounds__(256) void k_rank1(QOperand M, QOperand B, int64_t n, int64_t k,
                                               bool grouped, float* __restrict__ rho) {
  const int seg = blockIdx.y;
  const int lane = threadIdx.x & 63;
  const int64_t j = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (j >= n) return;
  const int64_t nb = k >> 4;
  const uint8_t* mc = M.codes + (int64_t)seg * (k >> 1);
  const uint8_t* ms = M.scales + (int64_t)seg * nb;
  const int64_t brow = (grouped ? (int64_t)seg * n : 0) + j;
  const uint8_t* bc = B.codes + brow * (k >> 1);
  const uint8_t* bs = B.scales + brow * nb;
  float acc = 0.0f;
  for (int64_t blk = lane; blk < nb; blk += 64) {
    const uint2 wm = *reinterpret_cast<const uint2*>(mc + blk * 8);
    const uint2 wb = *reinterpret_cast<const uint2*>(bc + blk * 8);
    float s = 0.0f;
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const uint32_t cm = ((e < 8 ? wm.x : wm.y) >> (4 * (e & 7))) & 0xFu;
      const uint32_t cb = ((e < 8 ? wb.x : wb.y) >> (4 * (e & 7))) & 0xFu;
      const float vm = (float)__builtin_bit_cast(_Float16, (uint16_t)e2m1_f16_bits(cm));
      const float vb = (float)__builtin_bit_cast(_Float16, (uint16_t)e2m1_f16_bits(cb));
      s += vm * vb;   // exact: products and partial sums of a block are small dyadics
    }
    acc += s * (e4m3_value(ms[blk]) * e4m3_value(bs[blk]));
  }
  for (int d = 32; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 64);
  if (lane == 0) {
    const float sd = M.tscale[2 * seg + 1] * B.tscale[(grouped ? 2 * seg : 0) + 1];
    rho[(int64_t)seg * n + j] = acc * sd;
  }
}

size_t gemm_ws_bytes(int64_t n, int nseg) {
  return (size_t)(n * (int64_t)(nseg > 0 ? nseg : 1) * 4 + 255) & ~(size_t)255;
}

hipError_t launch_gemm(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                       int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                       int64_t ldc, float* rho_ws, hipStream_t st) {
  const int ns = offs ? nseg : 1;
  if (mean) {
    dim3 g((unsigned)((n + 3) / 4), (unsigned)ns);
    k_rank1<<<g, 256, 0, st>>>(*mean, b, n, k, offs != nullptr, rho_ws);
  }
  const int64_t tiles_m = chunk_upper_bound(m, offs ? nseg : 1, BM);
  if (tiles_m == 0 || n == 0) return hipGetLastError();
  dim3 g((unsigned)((n + BN - 1) / BN), (unsigned)tiles_m);
  if (c_bf16) {
    if (mean)
      k_gemm_nt<true, true><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho_ws, c, ldc);
    else
      k_gemm_nt<true, false><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho_ws, c, ldc);
  } else {
    if (mean)
      k_gemm_nt<false, true><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho_ws, c, ldc);
    else
      k_gemm_nt<false, false><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho_ws, c, ldc);
  }
  return hipGetLastError();
}

}  // namespace averis
