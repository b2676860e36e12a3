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

#include <cstdlib>

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

// ---------------------------------------------------------------------------
// Fast path (K % 64 == 0): WG tile (64 TM) x (64 TN), 4 waves in a 2 x 2
// grid, each wave 32 TM x 32 TN outputs.  Per 64-wide K stage every thread
// loads raw codes for the next stage into registers while the waves run the
// MFMAs of the current stage from LDS; the codes are then dequantized with
// v_cvt_scalef32_pk_f16_fp4 (scale 1) and v_pk_mul_f16 by the E4M3 block
// scale (both exact) into the other LDS buffer.  One barrier per stage.
// The rank-one term is fused: the thread that stages row j of B also
// accumulates sum_k deq'(mean)_k deq'(B)_jk with v_dot2_f32_f16 on the
// values it has just dequantized, so no extra launch or pass over B.
// ---------------------------------------------------------------------------
namespace {



__device__ __forceinline__ half2_t scale_h2(uint32_t byte) {
  const _Float16 s = (_Float16)e4m3_value(byte & 0xFFu);
  half2_t r = {s, s};
  return r;
}


}  // namespace


#ifndef AVERIS_GEMM_INTERLEAVE
#define AVERIS_GEMM_INTERLEAVE 0
#endif
constexpr bool INTERLEAVE = AVERIS_GEMM_INTERLEAVE;

template <int TM, int TN, int WM, int WN, int PF, bool OUT_BF16, bool HAS_MEAN>
__global__ __launch_bounds__(64 * WM * WN, 1) void k_gemm_fast(QOperand A, QOperand B, QOperand MU,
                                                      int64_t m, int64_t n, int64_t k,
                                                      const int64_t* offs, int nseg, void* c,
                                                      int64_t ldc) {
  constexpr int NT = 64 * WM * WN;                // threads
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  // 32-element chunks per thread and stage; when a tile has fewer chunks
  // than threads, the surplus (whole) wavefronts skip them
  constexpr int CA = (2 * BM + NT - 1) / NT, CB = (2 * BN + NT - 1) / NT;
  extern __shared__ __attribute__((aligned(16))) _Float16 smem[];
  _Float16* As = smem;                          // [2][BM][LDSK]
  _Float16* Bs = As + 2 * BM * LDSK;            // [2][BN][LDSK]
  float* rho_sh = reinterpret_cast<float*>(Bs + 2 * BN * LDSK);   // [2][BN]
  _Float16* Ms = reinterpret_cast<_Float16*>(rho_sh + 2 * BN);    // [k] dequantized mean

  // Workgroups are dispatched round-robin over the 8 XCDs (linear id % 8).
  // Renumber them so each XCD walks a contiguous, row-major run of tiles:
  // the tiles an XCD runs together share A rows in its L2.
  int64_t tile_x, tile_y;
  {
    const int64_t gx = gridDim.x, total = gx * gridDim.y;
    const int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
    const int64_t even = total - total % kXcds;
    int64_t id = lin;
    if (lin < even) id = (lin % kXcds) * (even / kXcds) + lin / kXcds;
    tile_y = id / gx;
    tile_x = id - tile_y * gx;
  }
  const SegRange sr = locate_chunk(offs, nseg, m, BM, tile_y);
  if (sr.seg < 0) return;
  const int seg = sr.seg;
  const int64_t m0 = sr.r0, m_end = sr.r1;
  const int64_t n0 = tile_x * BN;
  const int64_t kh = k >> 1, kb = k >> 4;
  const uint8_t* bcodes = B.codes + (offs ? (int64_t)seg * n * kh : 0);
  const uint8_t* bscales = B.scales + (offs ? (int64_t)seg * n * kb : 0);

  const int t = threadIdx.x, lane = t & 63, w = t >> 6;
  const int wm = w / WN, wn = w % WN;

  if (HAS_MEAN) {
    // the whole dequantized mean vector (without its tensor scale) in LDS
    const uint8_t* mcodes = MU.codes + (int64_t)seg * kh;
    const uint8_t* mscales = MU.scales + (int64_t)seg * kb;
    for (int64_t q = t; q < (k >> 3); q += NT) {
      const uint32_t wq = *reinterpret_cast<const uint32_t*>(mcodes + 4 * q);
      reinterpret_cast<uint4*>(Ms)[q] = deq8(wq, scale_h2(mscales[q >> 1]));
    }
  }

  // Staging: chunk q = t + 256 i covers row q >> 1 of the tile, k-half q & 1
  // of each 64-wide stage.  Rows past the edge are clamped to the last valid
  // row: their products land only in outputs that are never stored.
  // Byte offsets are 32-bit and fixed; each stage adds a uniform k offset.
  const uint8_t* a_c = A.codes + m0 * kh;
  const uint8_t* a_s = A.scales + m0 * kb;
  const uint8_t* b_c = bcodes + n0 * kh;
  const uint8_t* b_s = bscales + n0 * kb;
  uint32_t oac[CA], oas[CA], obc[CB], obs[CB];
#pragma unroll
  for (int i = 0; i < CA; ++i) {
    const int q = t + NT * i, hf = q & 1;
    const int64_t row = (q >> 1) < (m_end - m0) ? (q >> 1) : (m_end - m0 - 1);
    oac[i] = (uint32_t)(row * kh) + 16u * hf;
    oas[i] = (uint32_t)(row * kb) + 2u * hf;
  }
#pragma unroll
  for (int i = 0; i < CB; ++i) {
    const int q = t + NT * i, hf = q & 1;
    const int64_t row = (q >> 1) < (n - n0) ? (q >> 1) : (n - n0 - 1);
    obc[i] = (uint32_t)(row * kh) + 16u * hf;
    obs[i] = (uint32_t)(row * kb) + 2u * hf;
  }

  // raw codes of K stage j live in register slot j % PF
  uint4 ra[PF][CA], rb[PF][CB];
  uint32_t sa[PF][CA], sb[PF][CB];
  float rho_acc[CB];
#pragma unroll
  for (int i = 0; i < CB; ++i) rho_acc[i] = 0.0f;

  auto gload = [&](int slot, int64_t k0) {
    const uint8_t* ac = a_c + (k0 >> 1);
    const uint8_t* as_ = a_s + (k0 >> 4);
    const uint8_t* bc = b_c + (k0 >> 1);
    const uint8_t* bs_ = b_s + (k0 >> 4);
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      if (t + NT * i >= 2 * BM) break;
      ra[slot][i] = *reinterpret_cast<const uint4*>(ac + oac[i]);
      sa[slot][i] = *reinterpret_cast<const uint16_t*>(as_ + oas[i]);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      if (t + NT * i >= 2 * BN) break;
      rb[slot][i] = *reinterpret_cast<const uint4*>(bc + obc[i]);
      sb[slot][i] = *reinterpret_cast<const uint16_t*>(bs_ + obs[i]);
    }
  };

  // dequantize the staged registers into LDS buffer `buf`; B rows also feed
  // the rank-one partial sums (Ms is written before the first barrier)
  auto stage = [&](int slot, int buf, int64_t k0) {
    _Float16* as = As + buf * BM * LDSK;
    _Float16* bs = Bs + buf * BN * LDSK;
#pragma unroll
    for (int i = 0; i < CA; ++i) {
      const int q = t + NT * i, row = q >> 1, hf = q & 1;
      if (q >= 2 * BM) break;
      const half2_t sc = scales2(sa[slot][i]);
      const half2_t s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
      uint4* dst = reinterpret_cast<uint4*>(as + row * LDSK + 32 * hf);
      dst[0] = deq8(ra[slot][i].x, s0);
      dst[1] = deq8(ra[slot][i].y, s0);
      dst[2] = deq8(ra[slot][i].z, s1);
      dst[3] = deq8(ra[slot][i].w, s1);
    }
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int q = t + NT * i, row = q >> 1, hf = q & 1;
      if (q >= 2 * BN) break;
      const half2_t sc = scales2(sb[slot][i]);
      const half2_t s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
      uint4 d[4];
      d[0] = deq8(rb[slot][i].x, s0);
      d[1] = deq8(rb[slot][i].y, s0);
      d[2] = deq8(rb[slot][i].z, s1);
      d[3] = deq8(rb[slot][i].w, s1);
      uint4* dst = reinterpret_cast<uint4*>(bs + row * LDSK + 32 * hf);
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[e] = d[e];
      if (HAS_MEAN) {
        const uint4* mv = reinterpret_cast<const uint4*>(Ms + k0 + 32 * hf);
        float a = rho_acc[i];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint4 m4 = mv[e];
          a = __builtin_amdgcn_fdot2(h2(d[e].x), h2(m4.x), a, false);
          a = __builtin_amdgcn_fdot2(h2(d[e].y), h2(m4.y), a, false);
          a = __builtin_amdgcn_fdot2(h2(d[e].z), h2(m4.z), a, false);
          a = __builtin_amdgcn_fdot2(h2(d[e].w), h2(m4.w), a, false);
        }
        rho_acc[i] = a;
      }
    }
  };

  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  // LDS fragment offsets (in fp16 elements) of this lane
  const int a_frag = (wm * 32 * TM + (lane & 31)) * LDSK + (lane >> 5) * 8;
  const int b_frag = (wn * 32 * TN + (lane & 31)) * LDSK + (lane >> 5) * 8;
  auto mfma_stage = [&](int buf) {
    const _Float16* as = As + buf * BM * LDSK + a_frag;
    const _Float16* bs = Bs + buf * BN * LDSK + b_frag;
#pragma unroll
    for (int kk = 0; kk < BK; kk += 16) {
      half8_t af[TM], bf[TN];
#pragma unroll
      for (int i = 0; i < TM; ++i)
        af[i] = *reinterpret_cast<const half8_t*>(as + i * 32 * LDSK + kk);
#pragma unroll
      for (int j = 0; j < TN; ++j)
        bf[j] = *reinterpret_cast<const half8_t*>(bs + j * 32 * LDSK + kk);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[j], af[i], acc[i][j], 0, 0, 0);
    }
  };

  // One K stage `it`: refill slot it % PF with stage it + PF, run the MFMAs
  // of LDS buffer it & 1, dequantize stage it + 1 into the other buffer.
  const int nk = (int)(k / BK);
  auto step = [&](int it, int slot, bool refill, bool next) {
    if (refill) gload(slot, (int64_t)(it + PF) * BK);
    // keep the prefetch loads ahead of everything else in the step: vmcnt
    // drains in issue order, so a load scheduled after the dequantization
    // below would make it wait for this step's loads too
    __builtin_amdgcn_sched_barrier(0);
    mfma_stage(it & 1);
    if (!next) mfma_drain();   // last stage: fence in the block of the last MFMA
    if (next) stage((slot + 1) % PF, (it + 1) & 1, (int64_t)(it + 1) * BK);
    if (INTERLEAVE && refill && next) {
      // Ask the scheduler to interleave: each MFMA leaves ~28 idle issue
      // cycles that the next stage's dequantization (VALU), its LDS writes
      // and this stage's fragment reads can fill.
      // coarse groups keep the scheduler's group solver cheap
      constexpr int NG = BK / 16;                     // one group per k-step
      constexpr int NM = TM * TN;                     // MFMAs per k-step
#pragma unroll
      for (int i = 0; i < NG; ++i) {
        __builtin_amdgcn_sched_group_barrier(0x100, TM + TN, 0);  // fragment reads
        __builtin_amdgcn_sched_group_barrier(0x008, NM / 2, 0);   // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x002, 16, 0);       // VALU
        __builtin_amdgcn_sched_group_barrier(0x008, NM / 2, 0);   // MFMAs
        __builtin_amdgcn_sched_group_barrier(0x200, 4, 0);        // LDS writes
      }
    }
    __syncthreads();
  };
#pragma unroll
  for (int p = 0; p < PF; ++p)
    if (p < nk) gload(p, (int64_t)p * BK);
  if (HAS_MEAN) __syncthreads();   // Ms visible before stage() reads it
  stage(0, 0, 0);
  __syncthreads();
  int it = 0;
  // steady state: every refill and every next stage exists
  for (; it + 2 * PF - 1 < nk; it += PF) {
#pragma unroll
    for (int u = 0; u < PF; ++u) step(it + u, u, true, true);
  }
  // tail: fewer than 2 PF - 1 stages left
#pragma unroll
  for (int u = 0; u < 2 * PF - 1; ++u) {
    const int i2 = it + u;
    if (i2 < nk) step(i2, u % PF, i2 + PF < nk, i2 + 1 < nk);
  }

  if (HAS_MEAN) {
#pragma unroll
    for (int i = 0; i < CB; ++i) {
      const int q = t + NT * i, row = q >> 1, hf = q & 1;
      if (q >= 2 * BN) break;
      rho_sh[hf * BN + row] = rho_acc[i];
    }
    __syncthreads();
    // each column's two k-half sums, times the tensor scales, in place
    const float sd = MU.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
    for (int cidx = t; cidx < BN; cidx += NT) rho_sh[cidx] = (rho_sh[cidx] + rho_sh[BN + cidx]) * sd;
    __syncthreads();
  }

  // The MFMAs take the B fragment first, so a lane's accumulators hold four
  // consecutive output columns (v & 3) of one output row: 8-byte (bf16) or
  // 16-byte (fp32) stores.
  const float alpha = A.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
  const bool full = (m0 + BM <= m_end) && (n0 + BN <= n);
  const bool vec = full && (ldc % 4 == 0) &&
                   ((reinterpret_cast<uintptr_t>(c) & (OUT_BF16 ? 7 : 15)) == 0);
  const int64_t row_base = m0 + wm * 32 * TM + (lane & 31);
  const int cl_base = wn * 32 * TN + (lane >> 5) * 4;   // tile-local column of v = 0
#pragma unroll
  for (int j = 0; j < TN; ++j) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const int cl = cl_base + j * 32 + 8 * q;
      const int64_t col = n0 + cl;
      f32x4_t r1 = {0.0f, 0.0f, 0.0f, 0.0f};
      if (HAS_MEAN) r1 = *reinterpret_cast<const f32x4_t*>(rho_sh + cl);
#pragma unroll
      for (int i = 0; i < TM; ++i) {
        const int64_t row = row_base + i * 32;
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = acc[i][j][4 * q + e] * alpha + r1[e];
        if (vec) {
          if (OUT_BF16) {
            const u32x2_t pk = {(uint32_t)f32_to_bf16_rne(y[0]) | ((uint32_t)f32_to_bf16_rne(y[1]) << 16),
                                (uint32_t)f32_to_bf16_rne(y[2]) | ((uint32_t)f32_to_bf16_rne(y[3]) << 16)};
            store_out(pk, reinterpret_cast<u32x2_t*>(static_cast<uint16_t*>(c) + row * ldc + col));
          } else {
            const f32x4_t v4 = {y[0], y[1], y[2], y[3]};
            store_out(v4, reinterpret_cast<f32x4_t*>(static_cast<float*>(c) + row * ldc + col));
          }
        } else if (row < m_end) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            if (col + e >= n) break;
            if (OUT_BF16)
              store_out(f32_to_bf16_rne(y[e]), static_cast<uint16_t*>(c) + row * ldc + col + e);
            else
              store_out(y[e], static_cast<float*>(c) + row * ldc + col + e);
          }
        }
      }
    }
  }
}

size_t gemm_ws_bytes(int64_t n, int64_t, int nseg) {
  return (size_t)(n * (int64_t)(nseg > 0 ? nseg : 1) * 4 + 255) & ~(size_t)255;
}

// dynamic LDS of k_gemm_fast
static size_t fast_lds_bytes(int tm, int tn, int64_t k, bool has_mean) {
  return (size_t)(2 * 64 * tm * LDSK + 2 * 64 * tn * LDSK) * 2 + (size_t)2 * 64 * tn * 4 +
         (has_mean ? (size_t)k * 2 : 0);
}

// 160 KB of LDS per workgroup, less room for the kernel's static LDS (segment lookup)
constexpr size_t kLdsLimit = 160 * 1024 - 512;

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

template <int TM, int TN, int PF, bool OB, bool HM, int WM = 2, int WN = 2>
static hipError_t launch_fast(const QOperand& a, const QOperand& mu, const QOperand& b, int64_t m,
                              int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                              int64_t ldc, hipStream_t st) {
  constexpr int BM = 32 * TM * WM, BN = 32 * TN * WN;
  const size_t lds = fast_lds_bytes(BM / 64, BN / 64, k, HM);
  {
    const hipError_t e = lds_attr_once<&k_gemm_fast<TM, TN, WM, WN, PF, OB, HM>>((int)kLdsLimit);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles_m = chunk_upper_bound(m, offs ? nseg : 1, BM);
  dim3 g((unsigned)((n + BN - 1) / BN), (unsigned)tiles_m);
  k_gemm_fast<TM, TN, WM, WN, PF, OB, HM><<<g, 64 * WM * WN, lds, st>>>(a, b, mu, m, n, k, offs, nseg, c, ldc);
  return hipGetLastError();
}

template <int TM, int TN, int PF>
static hipError_t launch_fast_any(const QOperand& a, const QOperand* mean, const QOperand& b,
                                  int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
                                  void* c, bool c_bf16, int64_t ldc, hipStream_t st) {
  const QOperand mu = mean ? *mean : QOperand{nullptr, nullptr, nullptr};
  if (c_bf16)
    return mean ? launch_fast<TM, TN, PF, true, true>(a, mu, b, m, n, k, offs, nseg, c, ldc, st)
                : launch_fast<TM, TN, PF, true, false>(a, mu, b, m, n, k, offs, nseg, c, ldc, st);
  return mean ? launch_fast<TM, TN, PF, false, true>(a, mu, b, m, n, k, offs, nseg, c, ldc, st)
              : launch_fast<TM, TN, PF, false, false>(a, mu, b, m, n, k, offs, nseg, c, ldc, st);
}

// Tile shape for the fast kernel, by estimated time: rounds of workgroups
// over the 256 CUs times the work of one round, with an efficiency factor per
// variant (the 8-wave variants run two waves per SIMD and overlap one wave's
// dequantization with the other's MFMAs; larger tiles dequantize fewer
// operand values per MFMA).  Returns 0 if the fast kernel does not apply.
//   1: 256x256, 4 waves   2: 256x128, 4 waves   3: 128x128, 4 waves (2 per CU)
//   4: 256x256, 8 waves   5: 256x128, 8 waves   6: 256x192, 8 waves
static int pick_tile(int64_t m, int64_t n, int64_t k, int nseg_eff, bool has_mean) {
  if (k % BK != 0) return 0;
  struct Cand { int id, bm, bn, per_cu; double eff; };
  const Cand cands[6] = {{6, 256, 192, 1, 1.05}, {5, 256, 128, 1, 1.0}, {4, 256, 256, 1, 0.95},
                         {3, 128, 128, 2, 0.9},  {2, 256, 128, 1, 0.85}, {1, 256, 256, 1, 0.8}};
  int best = 0;
  double best_cost = 0;
  for (const Cand& cd : cands) {
    if (fast_lds_bytes(cd.bm / 64, cd.bn / 64, k, has_mean) * cd.per_cu > kLdsLimit) continue;
    const int64_t tiles = chunk_upper_bound(m, nseg_eff, cd.bm) * ((n + cd.bn - 1) / cd.bn);
    const int64_t slots = 256 * cd.per_cu;
    const double rounds = (double)((tiles + slots - 1) / slots);
    const double cost = rounds * cd.bm * cd.bn * cd.per_cu / cd.eff;
    if (best == 0 || cost < best_cost) {
      best = cd.id;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_gemm(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                       int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                       int64_t ldc, void* ws, hipStream_t st) {
  float* rho_ws = static_cast<float*>(ws);
  if (m == 0 || n == 0) return hipGetLastError();
  // warp-specialized kernel (default); AVERIS_GEMM_KERNEL = 1 selects the
  // lock-step kernel below, AVERIS_GEMM_WS_TILE = 1..4 forces a variant,
  // AVERIS_GEMM_BQ = 1 keeps B as codes in LDS
  static const int kernel_sel = [] {
    const char* e = std::getenv("AVERIS_GEMM_KERNEL");
    return e ? std::atoi(e) : 0;
  }();
  if (kernel_sel == 0) {
    int v = ws_pick(m, n, k, offs ? nseg : 1, mean != nullptr);
    static const int forced_ws = [] {
      const char* e = std::getenv("AVERIS_GEMM_WS_TILE");
      return e ? std::atoi(e) : 0;
    }();
    static const int bq = [] {
      const char* e = std::getenv("AVERIS_GEMM_BQ");
      return e ? std::atoi(e) : 0;
    }();
    // B kept as codes in LDS (variants 3, 4) has no rank-one path
    if (v != 0 && bq == 1 && !mean) v += 2;
    if (v != 0 && forced_ws >= 1 && forced_ws <= 4 && !(mean && forced_ws > 2)) v = forced_ws;
    if (v != 0) return launch_gemm_ws(v, a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  }
  int choice = pick_tile(m, n, k, offs ? nseg : 1, mean != nullptr);
  // tuning override: AVERIS_GEMM_TILE = 1..6 (see pick_tile)
  static const int forced = [] {
    const char* e = std::getenv("AVERIS_GEMM_TILE");
    return e ? std::atoi(e) : 0;
  }();
  if (choice != 0 && forced >= 1 && forced <= 6) {
    static const int dims[7][2] = {{0, 0}, {4, 4}, {4, 2}, {2, 2}, {4, 4}, {4, 2}, {4, 3}};
    if (fast_lds_bytes(dims[forced][0], dims[forced][1], k, mean != nullptr) <= kLdsLimit)
      choice = forced;
  }
  static const int pf = [] {
    const char* e = std::getenv("AVERIS_GEMM_PF");
    return e ? std::atoi(e) : 2;
  }();
  const QOperand mu = mean ? *mean : QOperand{nullptr, nullptr, nullptr};
#define AVERIS_FAST(TM_, TN_)                                                               \
  switch (pf) {                                                                            \
    case 1: return launch_fast_any<TM_, TN_, 1>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st); \
    case 3: return launch_fast_any<TM_, TN_, 3>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st); \
    default: return launch_fast_any<TM_, TN_, 2>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st); \
  }
#define AVERIS_FAST8(TM_, TN_)                                                              \
  if (c_bf16)                                                                              \
    return mean ? launch_fast<TM_, TN_, 2, true, true, 4, 2>(a, mu, b, m, n, k, offs, nseg, c, ldc, st) \
                : launch_fast<TM_, TN_, 2, true, false, 4, 2>(a, mu, b, m, n, k, offs, nseg, c, ldc, st); \
  return mean ? launch_fast<TM_, TN_, 2, false, true, 4, 2>(a, mu, b, m, n, k, offs, nseg, c, ldc, st) \
              : launch_fast<TM_, TN_, 2, false, false, 4, 2>(a, mu, b, m, n, k, offs, nseg, c, ldc, st);
  switch (choice) {
    case 1: AVERIS_FAST(4, 4)
    case 2: AVERIS_FAST(4, 2)
    case 3: AVERIS_FAST(2, 2)
    case 4: AVERIS_FAST8(2, 4)
    case 5: AVERIS_FAST8(2, 2)
    case 6: AVERIS_FAST8(2, 3)
    default: break;
  }
#undef AVERIS_FAST
#undef AVERIS_FAST8
  // general path (K % 64 != 0, or a mean vector too long for LDS)
  const int ns = offs ? nseg : 1;
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
    e = launch_gemm_ws_splitk(xt, dt, m, n, l, splits, part, st);
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
