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
// rho_j = S_dec(mean) S_dec(B) sum_k deq'(mean)_k deq'(B)_jk is added in the
// GEMM epilogue as a broadcast row.  It comes from the split that made A
// (the rank-one entry points), else from the small GEMV kernel k_rank1 below,
// or, in the warp-specialized kernel, from its producer waves' dot products.
//
// Dispatch: the codes-in-LDS kernel (gemm_win.hip) wherever K % 256 == 0;
// the warp-specialized kernel (gemm_ws.hip) for the remaining K % 64 == 0;
// the simple tiled kernel k_gemm_nt below for any other K.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"
#include "launch.hpp"
#include "segments.hpp"

namespace averis {


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

// E4M3FN byte -> fp32 (exact), branch-free: normal (1 + m/8) 2^(e-7),
// subnormal m 2^-9
__device__ __forceinline__ float e4m3_value(uint32_t c) {
  const uint32_t e = (c >> 3) & 15u, m = c & 7u;
  const uint32_t normal = ((e + 120u) << 23) | (m << 20);
  const uint32_t sub = __float_as_uint((float)m * 0.001953125f);
  return __uint_as_float(e ? normal : sub);
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
    if (k0 + BK >= k) mfma_drain();   // last stage: fence in the block of the last MFMA
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
          store_out(f32_to_bf16_rne(y), static_cast<uint16_t*>(c) + row * ldc + col);
        else
          store_out(y, static_cast<float*>(c) + row * ldc + col);
      }
    }
}


size_t gemm_ws_bytes(int64_t n, int64_t, int nseg) {
  return (size_t)(n * (int64_t)(nseg > 0 ? nseg : 1) * 4 + 255) & ~(size_t)255;
}


// rho[seg][j] = S_dec(mean_seg) S_dec(B_seg) sum_k deq'(mean_seg)_k deq'(B_seg)_jk
// (the rank-one term of one output column).  Sixteen lanes per column j, four
// columns per wavefront: each lane takes 16-element blocks k = 16 (l + 16 i)
// of its column, dequantizes B and the mean exactly to fp16 and accumulates
// v_dot2_f32_f16 products in fp32; the sixteen partial sums are combined by a
// fixed butterfly.
constexpr int kRank1Cols = 16;   // columns per workgroup of 256 threads
__global__ __launch_bounds__(256) void k_rank1(QOperand M, QOperand B, int64_t n, int64_t k,
                                               bool grouped, float* __restrict__ rho) {
  const int seg = blockIdx.y;
  const int sub = threadIdx.x & 15;
  const int64_t j = (int64_t)blockIdx.x * kRank1Cols + (threadIdx.x >> 4);
  const bool live = j < n;
  const int64_t jj = live ? j : n - 1;   // keep every lane in the butterfly
  const int64_t kh = k >> 1, kb = k >> 4;
  const uint8_t* mc = M.codes + (int64_t)seg * kh;
  const uint8_t* ms = M.scales + (int64_t)seg * kb;
  const int64_t brow = (grouped ? (int64_t)seg * n : 0) + jj;
  const uint8_t* bc = B.codes + brow * kh;
  const uint8_t* bs = B.scales + brow * kb;
  float acc = 0.0f;
  // four blocks per pass, their loads issued before any arithmetic; blocks
  // past the end are clamped to the last one and their products dropped
  constexpr int U = 4;
  for (int64_t b0 = sub; b0 < kb; b0 += 16 * U) {
    uint2 wm[U], wb[U];
    uint32_t sm[U], sb[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t blk = b0 + 16 * u < kb ? b0 + 16 * u : kb - 1;
      wm[u] = *reinterpret_cast<const uint2*>(mc + 8 * blk);
      wb[u] = *reinterpret_cast<const uint2*>(bc + 8 * blk);
      sm[u] = ms[blk];
      sb[u] = bs[blk];
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const half2_t smh = scales2(sm[u]), sbh = scales2(sb[u]);
      const half2_t m0 = {smh.x, smh.x}, bb = {sbh.x, sbh.x};
      const uint4 dm[2] = {deq8(wm[u].x, m0), deq8(wm[u].y, m0)};
      const uint4 db[2] = {deq8(wb[u].x, bb), deq8(wb[u].y, bb)};
      float p = 0.0f;
#pragma unroll
      for (int e = 0; e < 2; ++e) {
        p = __builtin_amdgcn_fdot2(h2(dm[e].x), h2(db[e].x), p, false);
        p = __builtin_amdgcn_fdot2(h2(dm[e].y), h2(db[e].y), p, false);
        p = __builtin_amdgcn_fdot2(h2(dm[e].z), h2(db[e].z), p, false);
        p = __builtin_amdgcn_fdot2(h2(dm[e].w), h2(db[e].w), p, false);
      }
      acc += b0 + 16 * u < kb ? p : 0.0f;
    }
  }
  for (int d = 8; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 16);
  if (sub == 0 && live) {
    const float sd = M.tscale[2 * seg + 1] * B.tscale[(grouped ? 2 * seg : 0) + 1];
    rho[(int64_t)seg * n + j] = acc * sd;
  }
}


hipError_t launch_gemm(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                       int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                       int64_t ldc, void* ws, hipStream_t st) {
  float* rho_ws = static_cast<float*>(ws);
  if (m == 0 || n == 0) return hipGetLastError();
  const int ns = offs ? nseg : 1;
  // codes-in-LDS kernel wherever it applies (K % 256 == 0); with a mean, the
  // rank-one row from its own GEMV first
  const int fn = win_pick(m, n, k, ns, 1);
  if (fn != 0) {
    if (mean) {
      dim3 g((unsigned)((n + kRank1Cols - 1) / kRank1Cols), (unsigned)ns);
      k_rank1<<<g, 256, 0, st>>>(*mean, b, n, k, offs != nullptr, rho_ws);
    }
    return launch_gemm_win(fn, a, mean ? rho_ws : nullptr, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  }
  // warp-specialized kernel wherever it applies (K % 64 == 0, a mean row that
  // fits its LDS)
  const int v = ws_pick(m, n, k, ns, mean != nullptr);
  if (v != 0) return launch_gemm_ws(v, a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  // general path (K % 64 != 0, or a mean vector too long for LDS): the
  // rank-one row from its own GEMV, then the simple tiled kernel
  if (mean) {
    dim3 g((unsigned)((n + kRank1Cols - 1) / kRank1Cols), (unsigned)ns);
    k_rank1<<<g, 256, 0, st>>>(*mean, b, n, k, offs != nullptr, rho_ws);
  }
  const int64_t tiles_m = chunk_upper_bound(m, ns, BM);
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

// C = deq(A) deq(B)^T + 1 rho^T, rho precomputed by the split that made A
// (per segment when grouped)
hipError_t launch_gemm_rho(const QOperand& a, const float* rho, const QOperand& b, int64_t m,
                           int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                           bool c_bf16, int64_t ldc, hipStream_t st) {
  if (m == 0 || n == 0) return hipGetLastError();
  const int fn = win_pick(m, n, k, offs ? nseg : 1, 1);
  if (fn != 0) return launch_gemm_win(fn, a, rho, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  const int v = ws_pick(m, n, k, offs ? nseg : 1, false);
  if (v == 1 || v == 2)
    return launch_gemm_ws_rho(v, a, rho, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  // general path (K % 64 != 0): the simple kernel reads rho from global memory
  dim3 g((unsigned)((n + BN - 1) / BN), (unsigned)chunk_upper_bound(m, offs ? nseg : 1, BM));
  if (c_bf16)
    k_gemm_nt<true, true><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho, c, ldc);
  else
    k_gemm_nt<false, true><<<g, 256, 0, st>>>(a, b, m, n, k, offs, nseg, rho, c, ldc);
  return hipGetLastError();
}

// the same with the column statistics of the (bf16) output written for the
// split that will read it: the codes-in-LDS kernel where K % 256 == 0, else
// the warp-specialized one (K % 64 == 0); other K are rejected
hipError_t launch_gemm_rho_stats(const QOperand& a, const float* rho, const QOperand& b, int64_t m,
                                 int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                                 int64_t ldc, const ColStats& cs, hipStream_t st) {
  if (m == 0 || n == 0) return hipGetLastError();
  const int fn = win_pick(m, n, k, offs ? nseg : 1, 1);
  if (fn != 0)
    return launch_gemm_win(fn, a, rho, b, m, n, k, offs, nseg, c, true, ldc, st, 1, 0, cs);
  const int v = ws_pick(m, n, k, offs ? nseg : 1, false);
  if (v != 1 && v != 2) return hipErrorInvalidValue;
  return launch_gemm_ws_rho(v, a, rho, b, m, n, k, offs, nseg, c, true, ldc, st, cs);
}

// ---------------------------------------------------------------------------
// wgrad: dW = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X mu_D^T.  Its output
// (m x n) is short and wide next to its contraction over the tokens, so the
// product runs split-K into fp32 partials and one pass sums them in split
// order (the same bits on every run) and adds the outer product of the means.
// ---------------------------------------------------------------------------

// splits of the token axis: enough 256 x 192 tiles for one round over the
// 256 CUs, each split a multiple of 64 tokens and at least 512 long
int wgrad_splits(int64_t m, int64_t n, int64_t l) {
  if (m <= 0 || n <= 0 || l % 64 != 0) return 1;
  const int64_t tiles = ((m + 255) / 256) * ((n + 191) / 192);
  int s = 1;
  while (s < 8 && tiles * 2 * s <= 256 && l % (2 * s * 64) == 0 && l / (2 * s) >= 512) s *= 2;
  return s;
}

size_t wgrad_ws_bytes(int64_t m, int64_t n, int64_t l) {
  if (m <= 0 || n <= 0) return 0;
  return ((size_t)wgrad_splits(m, n, l) * (size_t)m * (size_t)n * 4 + 255) & ~(size_t)255;
}

__global__ __launch_bounds__(256) void k_fill_zero(float* p, int64_t quads) {
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q < quads) *reinterpret_cast<f32x4_t*>(p + 4 * q) = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
}

// out[i][j] = sum_z part[z][i][j] (in z order) + (l mu_x[i]) mu_d[j]; four
// consecutive outputs per thread (n % 16 == 0)
template <bool OUT_BF16>
__global__ __launch_bounds__(256) void k_wgrad_reduce(const float* __restrict__ part, int splits,
                                                      int64_t m, int64_t n,
                                                      const float* __restrict__ mu_x,
                                                      const float* __restrict__ mu_d, float l,
                                                      void* out, int64_t ldo) {
  const int64_t nq = n >> 2;
  const int64_t q = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (q >= m * nq) return;
  const int64_t i = q / nq, j = (q - i * nq) * 4;
  const int64_t mn = m * n;
  f32x4_t acc = *reinterpret_cast<const f32x4_t*>(part + i * n + j);
  for (int z = 1; z < splits; ++z) {
    const f32x4_t p = *reinterpret_cast<const f32x4_t*>(part + z * mn + i * n + j);
    acc += p;
  }
  const float li = l * mu_x[i];
  const f32x4_t md = *reinterpret_cast<const f32x4_t*>(mu_d + j);
  float y[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(li, md[e], acc[e]);
  if constexpr (OUT_BF16) {
    uint16_t* o = static_cast<uint16_t*>(out) + i * ldo + j;
    if ((ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 7) == 0) {
      u32x2_t v = {bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3])};
      *reinterpret_cast<u32x2_t*>(o) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = (uint16_t)bf16x2_rne(y[e], 0.0f);
    }
  } else {
    float* o = static_cast<float*>(out) + i * ldo + j;
    if ((ldo & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0) {
      f32x4_t v = {y[0], y[1], y[2], y[3]};
      *reinterpret_cast<f32x4_t*>(o) = v;
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = y[e];
    }
  }
}

hipError_t launch_wgrad(const QOperand& xt, const QOperand& dt, const float* mu_x,
                        const float* mu_d, int64_t m, int64_t n, int64_t l, void* out, bool bf16,
                        int64_t ldo, void* ws, hipStream_t st) {
  if (m == 0 || n == 0) return hipGetLastError();
  float* part = static_cast<float*>(ws);
  const int splits = wgrad_splits(m, n, l);
  hipError_t e;
  if (l == 0) {
    // no tokens: the product is zero; the reduce of one zero partial adds
    // the (zero-weighted) mean term
    e = hipSuccess;
  } else if (splits > 1) {
    const int fn = win_pick(m, n, l / splits, 1, splits);
    e = fn != 0 ? launch_gemm_win(fn, xt, nullptr, dt, m, n, l, nullptr, 1, part, false, n, st,
                                  splits, m * n)
                : launch_gemm_ws_splitk(xt, dt, m, n, l, splits, part, st);
  } else {
    e = launch_gemm(xt, nullptr, dt, m, n, l, nullptr, 1, part, false, n, nullptr, st);
  }
  if (e != hipSuccess) return e;
  const int64_t quads = m * (n >> 2);
  const dim3 g((unsigned)((quads + 255) / 256));
  if (l == 0) {
    // one partial of zeros, written by a kernel (no memset in a captured graph)
    k_fill_zero<<<g, 256, 0, st>>>(part, quads);
  }
  if (bf16)
    k_wgrad_reduce<true><<<g, 256, 0, st>>>(part, splits, m, n, mu_x, mu_d, (float)l, out, ldo);
  else
    k_wgrad_reduce<false><<<g, 256, 0, st>>>(part, splits, m, n, mu_x, mu_d, (float)l, out, ldo);
  return hipGetLastError();
}

}  // namespace averis
