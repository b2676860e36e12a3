// Warp-specialized quantized NT GEMM for gfx950 (K % 64 == 0).
//
// Computes the Averis products of the "Lighthouse" review §2.2 (forward
// Y = 1 (mean_q W_q) + X_R,q W_q and dgrad dX = 1 (mean_q,D W_q^T) +
// D_R,q W_q^T) as C = deq(A) deq(B)^T + 1 rho^T with
// rho_j = S_dec(mean) S_dec(B) sum_k deq'(mean)_k deq'(B)_jk.
//
// A workgroup of eight wavefronts owns a (64 TM) x (64 TN) output tile and
// splits the work by role, so that each SIMD runs one wavefront of each:
//   consumers (waves 0..3, a 2 x 2 grid): each owns a (32 TM) x (32 TN)
//     sub-tile, reads fp16 operand fragments from LDS and issues
//     v_mfma_f32_32x32x16_f16 back to back (fp32 accumulation);
//   producers (waves 4..7): load the next stages' 4-bit codes and E4M3
//     scales into a register ring and dequantize them exactly to fp16
//     (v_cvt_scalef32_pk_f16_fp4, v_pk_mul_f16 by the scale that
//     v_cvt_scalef32_pk_f16_fp8 decodes exactly) into the other LDS buffer.
// One barrier per 64-wide K stage hands the two LDS buffers over.  When all
// waves do both jobs in lock step, the MFMA phase and the dequantization
// phase of a stage follow each other on every SIMD; with split roles the
// dequantization of stage s + 1 runs on the same SIMDs during the MFMAs of
// stage s.
//
// The rank-one term rho (one value per output column) is summed by the
// producers while they dequantize B: each B chunk is dotted (v_dot2_f32_f16)
// with the matching 32 values of the mean row, which the producers dequantize
// into LDS once per tile; the two k-halves of a row are added across
// neighbouring lanes and the result is staged in LDS for the epilogue.  Every
// row tile of a column sums in the same order, so all of them add the same
// rho.  The MFMA takes the B fragment first, so a lane's accumulators hold
// four consecutive output columns of one output row: 8-byte (bf16) or
// 16-byte (fp32) stores.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"
#include "launch.hpp"
#include "segments.hpp"

namespace averis {
namespace {

constexpr int kWsBK = 64;
constexpr int kWsLdsK = kWsBK + 8;   // fp16 per LDS row (16-byte pad against bank conflicts)
constexpr int kProducers = 256;      // producer threads (waves 4..7)

template <int V>
struct WsIC {
  static constexpr int value = V;
};

template <int I, int N, typename F>
__device__ __forceinline__ void ws_unroll(F&& f) {
  if constexpr (I < N) {
    f(WsIC<I>{});
    ws_unroll<I + 1, N>(f);
  }
}

}  // namespace

// RG (with HAS_MEAN): the rank-one row comes precomputed (rho_g, one float
// per column of B) instead of being summed by the producers from the mean row
template <int TM, int TN, int PF, bool OUT_BF16, bool HAS_MEAN, bool SG, bool RG = false>
__global__ __launch_bounds__(512, 1) void k_gemm_ws(QOperand A, QOperand B, QOperand M, int64_t m,
                                                    int64_t n, int64_t k, const int64_t* offs,
                                                    int nseg, void* c, int64_t ldc, int64_t kld,
                                                    int64_t c_split, const float* rho_g,
                                                    ColStats cs) {
  constexpr int BM = 64 * TM, BN = 64 * TN;
  // 32-element chunks dequantized per stage: A rows and B rows
  constexpr int NCH = 2 * (BM + BN);
  constexpr int CP = (NCH + kProducers - 1) / kProducers;  // chunks per producer thread
  constexpr int IA = 2 * BM / kProducers;                // chunk rounds that hold A rows
  static_assert((2 * BM) % kProducers == 0 && (2 * BN) % 64 == 0, "whole-wave chunk rounds");
  static_assert(!RG || HAS_MEAN, "a precomputed rank-one row is a mean term");
  constexpr bool DOTS = HAS_MEAN && !RG;   // the producers sum the rank-one row
  constexpr int CPB = CP - IA;   // chunk rounds that hold B rows
  extern __shared__ __attribute__((aligned(16))) _Float16 smem_ws[];
  _Float16* As = smem_ws;                                // [2][BM][LDSK]
  _Float16* Bs = As + 2 * BM * kWsLdsK;                  // [2][BN][LDSK]
  float* rho_sh = reinterpret_cast<float*>(Bs + 2 * BN * kWsLdsK);   // [BN]
  // HAS_MEAN: the segment's mean row, dequantized to fp16 once ([k])
  _Float16* mean_sh = reinterpret_cast<_Float16*>(rho_sh + BN);

  int64_t tile_x, tile_y;
  xcd_tile(tile_x, tile_y);
  const SegRange sr = locate_chunk(offs, nseg, m, BM, tile_y);
  if (sr.seg < 0) return;
  const int seg = sr.seg;
  const int64_t m0 = sr.r0, m_end = sr.r1;
  const int64_t n0 = tile_x * BN;
  // split-K (gridDim.z > 1): split z contracts k = kld / gridDim.z columns
  // starting at z k of operands whose rows hold kld columns, and writes its
  // partial product to c + z c_split
  const int64_t kh = kld >> 1, kb = kld >> 4;
  const int64_t kz = (int64_t)blockIdx.z * k;
  c = static_cast<char*>(c) + (int64_t)blockIdx.z * c_split * (OUT_BF16 ? 2 : 4);
  const uint8_t* bcodes = B.codes + (offs ? (int64_t)seg * n * kh : 0) + (kz >> 1);
  const uint8_t* bscales = B.scales + (offs ? (int64_t)seg * n * kb : 0) + (kz >> 4);

  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const bool producer = wave >= 4;
  const int nk = (int)(k / kWsBK);

  // bf16 output of a full tile goes out through LDS: the consumers write the
  // finished tile into the (then free) stage buffers and all eight waves
  // store it in 16-byte pieces, eight lanes to a 128-byte output line (a
  // direct store writes 16 bytes into each of 32 lines, and the L2's write
  // request rate, not its bandwidth, bounds the epilogue)
  constexpr int kStLd = 2 * BN + 16;   // staged row, bytes (16-byte aligned, staggered banks)
  constexpr size_t kStageRoom = (size_t)2 * (BM + BN) * kWsLdsK * 2;
  constexpr bool kCanStage = OUT_BF16 && (size_t)BM * kStLd <= kStageRoom;
  constexpr bool stage_out = kCanStage;   // every tile of a bf16 output
  // pieces that lie wholly inside the output, with 16-byte aligned rows, go
  // out as one store; the others (edge tiles, odd strides) element by element
  const bool st_vec = (ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(c) & 15) == 0);
  const int rows_here = (int)(m_end - m0 < BM ? m_end - m0 : BM);
  const int cols_here = (int)(n - n0 < BN ? n - n0 : BN);
  unsigned char* stg = reinterpret_cast<unsigned char*>(smem_ws);
  auto store_staged = [&]() __attribute__((always_inline)) {
    constexpr int CPR = 2 * BN / 16;   // 16-byte pieces per tile row
    uint16_t* cb = static_cast<uint16_t*>(c) + m0 * ldc + n0;
#pragma unroll
    for (int it = 0; it < BM * CPR / 512; ++it) {
      const int cidx = t + 512 * it;
      const int r = cidx / CPR, cc = cidx - r * CPR;
      if (r >= rows_here) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * kStLd + cc * 16);
      uint16_t* dst = cb + (int64_t)r * ldc + cc * 8;
      if (st_vec && cc * 8 + 8 <= cols_here) {
        store_out(v, reinterpret_cast<u32x4_t*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (cc * 8 + e < cols_here) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
  };
  static_assert((BM * (2 * BN / 16)) % 512 == 0, "whole store rounds");
  // column statistics of the staged bf16 tile, as stored (cs.psum set): per
  // column of the tile the fp64 sum, max, min and smallest nonzero magnitude
  // of its rows_here values -> the chunk's partials [tile_y][col] of the split
  // that will read this output.  Thread (p, g) takes column pair p and rows
  // g, g + G, ...; the G row groups meet in the stage room past the tile.
  auto col_stats = [&]() __attribute__((always_inline)) {
    constexpr int P = BN / 2, G = 512 / P;
    static_assert((size_t)BM * kStLd + (size_t)G * BN * 16 + (size_t)G * P * 4 <= kStageRoom,
                  "room for the row groups' partials");
    double* gs = reinterpret_cast<double*>(stg + BM * kStLd);   // [G][BN]
    float* gmx = reinterpret_cast<float*>(gs + G * BN);         // [G][BN]
    float* gmn = gmx + G * BN;                                  // [G][BN]
    uint32_t* gmz = reinterpret_cast<uint32_t*>(gmn + G * BN);  // [G][P] packed 16-bit minima
    typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
    typedef short i16x2 __attribute__((ext_vector_type(2)));
    // bf16 bits -> 16-bit integers in the order of the values (a negative
    // value's magnitude bits flipped), so one packed integer max or min
    // covers both columns of a pair; the map is its own inverse
    auto ordered = [](uint32_t w) __attribute__((always_inline)) {
      const i16x2 x = __builtin_bit_cast(i16x2, w);
      return x ^ ((x >> 15) & i16x2{0x7FFF, 0x7FFF});
    };
    const int p = t % P, g = t / P;
    if (g < G) {
      double s0 = 0.0, s1 = 0.0;
      i16x2 mx = {-32768, -32768}, mn = {32767, 32767};
      // smallest nonzero |bf16| as (|bits| - 1) per half: a zero wraps to
      // 0xFFFF and never wins the minimum
      u16x2 mz = {0xFFFFu, 0xFFFFu};
      auto add_row = [&](uint32_t w) __attribute__((always_inline)) {
        const i16x2 o = ordered(w);
        mx = __builtin_elementwise_max(mx, o);
        mn = __builtin_elementwise_min(mn, o);
        mz = __builtin_elementwise_min(mz, __builtin_bit_cast(u16x2, w & 0x7FFF7FFFu) - u16x2{1, 1});
      };
      // full rounds of U rows (their reads issued together, at constant
      // offsets from one pointer), then the remaining rows one by one
      constexpr int U = 4;
      const unsigned char* q = stg + g * kStLd + 4 * p;
      int r = g;
      for (; r + (U - 1) * G < rows_here; r += U * G, q += U * G * kStLd) {
        uint32_t w[U];
#pragma unroll
        for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint32_t*>(q + u * G * kStLd);
#pragma unroll
        for (int u = 0; u < U; ++u) {
          s0 += (double)__uint_as_float(w[u] << 16);
          s1 += (double)__uint_as_float(w[u] & 0xFFFF0000u);
          add_row(w[u]);
        }
      }
      for (; r < rows_here; r += G, q += G * kStLd) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(q);
        s0 += (double)__uint_as_float(w << 16);
        s1 += (double)__uint_as_float(w & 0xFFFF0000u);
        add_row(w);
      }
      const uint32_t bx = __builtin_bit_cast(uint32_t, ordered(__builtin_bit_cast(uint32_t, mx)));
      const uint32_t bn = __builtin_bit_cast(uint32_t, ordered(__builtin_bit_cast(uint32_t, mn)));
      // a thread without rows keeps -inf / +inf
      const bool any = g < rows_here;
      gs[g * BN + 2 * p] = s0;
      gs[g * BN + 2 * p + 1] = s1;
      gmx[g * BN + 2 * p] = any ? __uint_as_float(bx << 16) : -__builtin_inff();
      gmx[g * BN + 2 * p + 1] = any ? __uint_as_float(bx & 0xFFFF0000u) : -__builtin_inff();
      gmn[g * BN + 2 * p] = any ? __uint_as_float(bn << 16) : __builtin_inff();
      gmn[g * BN + 2 * p + 1] = any ? __uint_as_float(bn & 0xFFFF0000u) : __builtin_inff();
      gmz[g * P + p] = __builtin_bit_cast(uint32_t, mz);
    }
    __syncthreads();
    if (t < BN && n0 + t < n) {
      double s = 0.0;
      float x = -__builtin_inff(), y = __builtin_inff();
      uint32_t z = 0xFFFFu;
      for (int gg = 0; gg < G; ++gg) {
        s += gs[gg * BN + t];
        x = __builtin_fmaxf(x, gmx[gg * BN + t]);
        y = __builtin_fminf(y, gmn[gg * BN + t]);
        const uint32_t q = (gmz[gg * P + (t >> 1)] >> (16 * (t & 1))) & 0xFFFFu;
        z = q < z ? q : z;
      }
      const int64_t o = tile_y * n + n0 + t;
      cs.psum[o] = s;
      cs.pmax[o] = x;
      cs.pmin[o] = y;
      cs.pmnz[o] = z == 0xFFFFu ? __builtin_inff() : __uint_as_float((z + 1u) << 16);
    }
  };

  if (producer) {
    // ------------------------------------------------------------------ producers
    const int pt = t - 512 + kProducers;
    // chunk q = pt + 256 i: A row q >> 1 (rounds i < IA) or B row
    // (q - 2 BM) >> 1, k-half q & 1 of each stage.  Rows past the edge are
    // clamped to the last valid row: their products only reach outputs that
    // are never stored.  Byte offsets are 32-bit; each stage adds a uniform
    // k offset.
    const uint8_t* a_c = A.codes + m0 * kh + (kz >> 1);
    const uint8_t* a_s = A.scales + m0 * kb + (kz >> 4);
    const uint8_t* b_c = bcodes + n0 * kh;
    const uint8_t* b_s = bscales + n0 * kb;
    // W2 (with SG): one load instruction covers 64 contiguous code bytes of a
    // row -- two stages, four lanes to a row -- where the per-stage mapping
    // covers 32 (two lanes to a row); a second load takes the wave's other 16
    // rows with the two stages swapped, so each lane still holds one chunk
    // per stage, of row lo or row hi, picked per lane when it is dequantized.
    // The loads touch half as many cache lines per byte.  Used with three
    // column fragments per consumer wave (48 MFMAs per stage); with two, the
    // stage is too short for the producers' extra selects (measured slower).
    constexpr bool W2 = SG && TN == 3;
    const int w2_p = pt & 3;                      // 16-byte piece of the 64-byte window
    const bool w2_sel = (w2_p >> 1) != 0;         // row lo holds the window's second stage
    uint32_t oc_lo[CP], oc_hi[CP], os_lo[CP], os_hi[CP];
    int lrow_lo[CP], lrow_hi[CP];
    if constexpr (W2) {
#pragma unroll
      for (int i = 0; i < CP; ++i) {
        const bool is_a = i < IA;
        const int base = (is_a ? 128 * i : 128 * (i - IA)) + 32 * ((pt >> 6) & 3);
        const int64_t lim = is_a ? (m_end - m0) : (n - n0);
        // the four lanes of group g take rows 2g (lo) and 2g + 1 (hi): the
        // eight lanes of a 128-byte LDS write cycle then write four
        // consecutive rows, in distinct banks (rows 16 apart share banks)
        const int rl = base + 2 * ((pt & 63) >> 2), rh = rl + 1;
        const int64_t rowl = rl < lim ? rl : lim - 1, rowh = rh < lim ? rh : lim - 1;
        lrow_lo[i] = rl;
        lrow_hi[i] = rh;
        oc_lo[i] = (uint32_t)(rowl * kh) + 16u * (uint32_t)w2_p;
        oc_hi[i] = (uint32_t)(rowh * kh) + 16u * (uint32_t)((w2_p + 2) & 3);
        os_lo[i] = (uint32_t)(rowl * kb);
        os_hi[i] = (uint32_t)(rowh * kb);
      }
    }
    uint32_t oc[CP], os[CP];
    int lrow[CP];
#pragma unroll
    for (int i = 0; i < CP; ++i) {
      const int q = pt + kProducers * i, hf = q & 1;
      const bool is_a = i < IA;
      const int r = is_a ? (q >> 1) : ((q - 2 * BM) >> 1);
      const int64_t lim = is_a ? (m_end - m0) : (n - n0);
      const int64_t row = r < lim ? r : lim - 1;
      lrow[i] = r;
      oc[i] = (uint32_t)(row * kh) + 16u * hf;
      os[i] = (uint32_t)(row * kb) + (SG ? 0u : 2u * hf);
    }
    // SG (K % 256 == 0): a chunk's scale bytes come 16 at a time -- its row's
    // four stages of one 256-wide group -- into a two-group ring, instead of
    // two bytes per stage (the loads, not their bytes, are what costs)
    const uint32_t ssh = 16u * (uint32_t)(pt & 1);   // the chunk's k-half picks 2 of 4 bytes
    uint4 rc[PF][CP];
    uint32_t rs[PF][CP];
    uint4 rsg[2][CP];
    uint4 rsg_hi[2][CP];   // W2: the scale groups of row hi

    // sw: the stage index mod 8, a compile-time constant wherever these run
    // (the loop below advances 8 stages per iteration when SG).
    // Every lane issues every load of the ring, also in the chunk round that
    // only part of the waves dequantize (their rows are clamped) and past the
    // last stage (see ld_stage): the compiler counts outstanding loads
    // exactly only through straight-line code, and a load under a branch makes
    // it wait for all of them (vmcnt(0)) at the next use, which drains the ring.
    auto gload = [&](int slot, int st, auto sw_c) __attribute__((always_inline)) {
      constexpr int sw = decltype(sw_c)::value;
      if constexpr (W2) {
        // st even: stages st and st + 1 into ring slots slot and slot + 1
#pragma unroll
        for (int i = 0; i < CP; ++i) {
          const uint8_t* cb = (i < IA ? a_c : b_c) + 32 * st;
          rc[slot][i] = *reinterpret_cast<const uint4*>(cb + oc_lo[i]);
          rc[slot + 1][i] = *reinterpret_cast<const uint4*>(cb + oc_hi[i]);
          if constexpr ((sw & 3) == 0) {
            const uint8_t* sb = (i < IA ? a_s : b_s) + 4 * st;
            rsg[(sw >> 2) & 1][i] = *reinterpret_cast<const uint4*>(sb + os_lo[i]);
            rsg_hi[(sw >> 2) & 1][i] = *reinterpret_cast<const uint4*>(sb + os_hi[i]);
          }
        }
        return;
      }
#pragma unroll
      for (int i = 0; i < CP; ++i) {
        const uint8_t* cb = (i < IA ? a_c : b_c) + 32 * st;
        rc[slot][i] = *reinterpret_cast<const uint4*>(cb + oc[i]);
        if constexpr (SG) {
          if constexpr ((sw & 3) == 0) {
            const uint8_t* sb = (i < IA ? a_s : b_s) + 4 * st;
            rsg[(sw >> 2) & 1][i] = *reinterpret_cast<const uint4*>(sb + os[i]);
          }
        } else {
          const uint8_t* sb = (i < IA ? a_s : b_s) + 4 * st;
          rs[slot][i] = *reinterpret_cast<const uint16_t*>(sb + os[i]);
        }
      }
    };
    // HAS_MEAN: rank-one partial sums of the chunk rows that hold B, in
    // stage order (so every row tile of a column adds the same bits)
    float racc[CPB > 0 ? CPB : 1];
    float racc_hi[CPB > 0 ? CPB : 1];   // W2: a lane's chunks alternate between rows lo and hi
#pragma unroll
    for (int i = 0; i < (CPB > 0 ? CPB : 1); ++i) racc[i] = racc_hi[i] = 0.0f;
    auto dequant = [&](int slot, int buf, int st, auto sw_c) __attribute__((always_inline)) {
      constexpr int sw = decltype(sw_c)::value;
#pragma unroll
      for (int i = 0; i < CP; ++i) {
        const int q = pt + kProducers * i, hf = q & 1;
        if (q >= NCH) break;
        uint32_t sbytes;
        uint4 cw;
        int drow;
        if constexpr (W2) {
          // the window's chunks sit in ring slots se (from row lo) and se + 1
          // (row hi); x picks the one that holds this stage for this lane
          constexpr int se = sw & 2;
          const bool x = w2_sel != ((sw & 1) != 0);
          const uint4 glo = rsg[(sw >> 2) & 1][i], ghi = rsg_hi[(sw >> 2) & 1][i];
          const uint32_t wlo = (sw & 3) == 0 ? glo.x : (sw & 3) == 1 ? glo.y : (sw & 3) == 2 ? glo.z : glo.w;
          const uint32_t whi = (sw & 3) == 0 ? ghi.x : (sw & 3) == 1 ? ghi.y : (sw & 3) == 2 ? ghi.z : ghi.w;
          sbytes = (x ? whi : wlo) >> ssh;
          cw = x ? rc[se + 1][i] : rc[se][i];
          drow = x ? lrow_hi[i] : lrow_lo[i];
        } else {
          if constexpr (SG) {
            const uint4 g = rsg[(sw >> 2) & 1][i];
            const uint32_t wd = (sw & 3) == 0 ? g.x : (sw & 3) == 1 ? g.y : (sw & 3) == 2 ? g.z : g.w;
            sbytes = wd >> ssh;
          } else {
            sbytes = rs[slot][i];
          }
          cw = rc[slot][i];
          drow = lrow[i];
        }
        const half2_t sc = scales2(sbytes);
        const half2_t s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
        uint4 d[4];
        d[0] = deq8(cw.x, s0);
        d[1] = deq8(cw.y, s0);
        d[2] = deq8(cw.z, s1);
        d[3] = deq8(cw.w, s1);
        _Float16* base = i < IA ? As + buf * BM * kWsLdsK : Bs + buf * BN * kWsLdsK;
        uint4* dst = reinterpret_cast<uint4*>(base + drow * kWsLdsK + 32 * hf);
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[e] = d[e];
        if constexpr (DOTS) {
          if (i >= IA) {
            // the products of two exact fp16 values (<= 5 significant bits
            // each) are exact; fp32 accumulation
            // four independent chains (one per 8 elements), then their sum
            const uint4* mv = reinterpret_cast<const uint4*>(mean_sh + st * kWsBK + 32 * hf);
            float r[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint4 mm = mv[e];
              r[e] = __builtin_amdgcn_fdot2(h2(d[e].x), h2(mm.x), 0.0f, false);
              r[e] = __builtin_amdgcn_fdot2(h2(d[e].y), h2(mm.y), r[e], false);
              r[e] = __builtin_amdgcn_fdot2(h2(d[e].z), h2(mm.z), r[e], false);
              r[e] = __builtin_amdgcn_fdot2(h2(d[e].w), h2(mm.w), r[e], false);
            }
            const float rsum = (r[0] + r[1]) + (r[2] + r[3]);
            if constexpr (W2) {
              const bool xh = drow != lrow_lo[i];
              racc[i - IA] += xh ? 0.0f : rsum;
              racc_hi[i - IA] += xh ? rsum : 0.0f;
            } else {
              racc[i - IA] += rsum;
            }
          }
        }
      }
    };

    // stage j's codes live in ring slot j % PF, PF stages ahead of their
    // dequantization; buffer j & 1 of LDS receives stage j.  With SG the
    // group ring's slot (j >> 2) & 1 is refilled when stage j = 4g is loaded,
    // after stage 4g - 5 (the last user of that slot) was dequantized.
    static_assert(!SG || PF == 4, "scale groups assume a 4-stage ring");
    constexpr int UNR = SG ? 8 : PF;   // stages per loop iteration
    // the mean row (HAS_MEAN) is loaded first: the in-order load counter
    // then lets its dequantization start before the stages' loads land
    constexpr int kMeanPer = 4;   // 32-element chunks of the mean row per thread, at most
    uint4 mw[kMeanPer];
    uint32_t msc[kMeanPer];
    const int nmc = DOTS ? (int)(k >> 5) : 0;
    if constexpr (DOTS) {
      const uint8_t* mc = M.codes + (int64_t)seg * kh;
      const uint8_t* ms = M.scales + (int64_t)seg * kb;
#pragma unroll
      for (int u = 0; u < kMeanPer; ++u) {
        const int cidx = pt + kProducers * u;
        if (cidx < nmc) {
          mw[u] = *reinterpret_cast<const uint4*>(mc + 16 * cidx);
          msc[u] = *reinterpret_cast<const uint16_t*>(ms + 2 * cidx);
        }
      }
    }
    // a load for a stage past the end fetches an in-bounds stage instead
    // (never dequantized): the last stage, or the last 256-wide scale group
    // with SG (nk % 4 == 0 there, so nk - 4 >= 0 is a group's first stage)
    auto ld_stage = [&](int st) __attribute__((always_inline)) {
      return st < nk ? st : (SG ? nk - 4 : nk - 1);
    };
    // RG: every lane loads a value of the rank-one row ahead of the ring (an
    // in-bounds column for lanes past the tile), so that waiting for it does
    // not wait for the ring's loads
    float rho_v = 0.0f;
    if constexpr (RG) {
      const int64_t cj = n0 + (pt < BN ? pt : BN - 1);
      rho_v = rho_g[(offs ? (int64_t)seg * n : 0) + (cj < n ? cj : n - 1)];
    }
    if constexpr (W2) {
      // windows 0 and 1 (stages 0..3) fill the ring (nk >= 4 with SG)
      gload(0, 0, WsIC<0>{});
      gload(2, 2, WsIC<2>{});
    } else {
      ws_unroll<0, PF>([&](auto p_c) __attribute__((always_inline)) {
        constexpr int p = decltype(p_c)::value;
        gload(p, ld_stage(p), WsIC<p>{});
      });
    }
    if constexpr (RG) {
      // published by the stage-0 barrier below; lanes past the tile store
      // the last column's value again (no branch around the load's use)
      const int pc = pt < BN ? pt : BN - 1;
      rho_sh[pc] = n0 + pc < n ? rho_v : 0.0f;
    } else if constexpr (HAS_MEAN) {
#pragma unroll
      for (int u = 0; u < kMeanPer; ++u) {
        const int cidx = pt + kProducers * u;
        if (cidx < nmc) {
          const half2_t sc = scales2(msc[u]);
          const half2_t s0 = {sc.x, sc.x}, s1 = {sc.y, sc.y};
          uint4* dst = reinterpret_cast<uint4*>(mean_sh + 32 * cidx);
          dst[0] = deq8(mw[u].x, s0);
          dst[1] = deq8(mw[u].y, s0);
          dst[2] = deq8(mw[u].z, s1);
          dst[3] = deq8(mw[u].w, s1);
        }
      }
      __syncthreads();   // mean row published (the consumers wait here too)
    }
    dequant(0, 0, 0, WsIC<0>{});
    if constexpr (!W2) gload(0, ld_stage(PF), WsIC<PF % 8>{});
    __syncthreads();
    // iteration it: dequantize stage it + 1 (slot (it + 1) % PF) into buffer
    // (it + 1) & 1, refill that slot with stage it + 1 + PF
    int it = 0;
    for (; it + UNR <= nk; it += UNR) {
      ws_unroll<0, UNR>([&](auto u_c) __attribute__((always_inline)) {
        constexpr int u = decltype(u_c)::value;
        constexpr int su = (u + 1) % PF;
        const int i2 = it + u;
        if (i2 + 1 < nk) dequant(su, (i2 + 1) & 1, i2 + 1, WsIC<(u + 1) % 8>{});
        if constexpr (W2) {
          // after an odd stage both slots of the window three stages on
          // are free: stages i2 + 4 and i2 + 5
          if constexpr (((u + 1) & 1) == 1) gload((u + 4) % PF, ld_stage(i2 + 4), WsIC<(u + 4) % 8>{});
        } else {
          gload(su, ld_stage(i2 + 1 + PF), WsIC<(u + 1 + PF) % 8>{});
        }
        __syncthreads();
      });
    }
    ws_unroll<0, UNR>([&](auto u_c) __attribute__((always_inline)) {
      constexpr int u = decltype(u_c)::value;
      constexpr int su = (u + 1) % PF;
      const int i2 = it + u;
      if (i2 < nk) {
        if (i2 + 1 < nk) dequant(su, (i2 + 1) & 1, i2 + 1, WsIC<(u + 1) % 8>{});
        if constexpr (W2) {
          if constexpr (((u + 1) & 1) == 1) gload((u + 4) % PF, ld_stage(i2 + 4), WsIC<(u + 4) % 8>{});
        } else {
          gload(su, ld_stage(i2 + 1 + PF), WsIC<(u + 1 + PF) % 8>{});
        }
        __syncthreads();
      }
    });
    if constexpr (DOTS) {
      // the two k-halves of a row sit in neighbouring lanes
      const float rs_scale = M.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
#pragma unroll
      for (int i = IA; i < CP; ++i) {
        if (pt + kProducers * i >= NCH) break;   // whole waves
        if constexpr (W2) {
          // rows lo and hi were each summed by the four lanes of a row group
          float vl = racc[i - IA], vh = racc_hi[i - IA];
          vl += __shfl_xor(vl, 1, 64);
          vh += __shfl_xor(vh, 1, 64);
          vl += __shfl_xor(vl, 2, 64);
          vh += __shfl_xor(vh, 2, 64);
          if ((pt & 3) == 0) {
            rho_sh[lrow_lo[i]] = vl * rs_scale;
            rho_sh[lrow_hi[i]] = vh * rs_scale;
          }
        } else {
          const float v = racc[i - IA] + __shfl_xor(racc[i - IA], 1, 64);
          if ((pt & 1) == 0) rho_sh[lrow[i]] = v * rs_scale;
        }
      }
      __syncthreads();   // rank-one terms published for the epilogue
    }
    if constexpr (stage_out) {
      __syncthreads();   // the consumers have staged the tile
      store_staged();
      if (cs.psum) col_stats();   // uniform
    }
    return;
  }

  // -------------------------------------------------------------------- consumers
  const int wm = wave >> 1, wn = wave & 1;
  f32x16_t acc[TM][TN];
#pragma unroll
  for (int i = 0; i < TM; ++i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;
  const int a_frag = (wm * 32 * TM + (lane & 31)) * kWsLdsK + (lane >> 5) * 8;
  const int b_frag = (wn * 32 * TN + (lane & 31)) * kWsLdsK + (lane >> 5) * 8;
  // fragments of k-step kk of the stage in buffer b; the reads for k-step
  // kk + 1 are issued before the MFMAs of k-step kk, so the MFMAs hide the
  // LDS latency (the first k-step of a stage waits for the barrier)
  half8_t af[2][TM], bf[2][TN];
  auto read_frags = [&](int slot, int b, int kk) __attribute__((always_inline)) {
    const _Float16* as = As + b * BM * kWsLdsK + a_frag + kk;
#pragma unroll
    for (int i = 0; i < TM; ++i)
      af[slot][i] = *reinterpret_cast<const half8_t*>(as + i * 32 * kWsLdsK);
    const _Float16* bs = Bs + b * BN * kWsLdsK + b_frag + kk;
#pragma unroll
    for (int j = 0; j < TN; ++j)
      bf[slot][j] = *reinterpret_cast<const half8_t*>(bs + j * 32 * kWsLdsK);
  };
  if constexpr (DOTS) __syncthreads();   // the producers' mean row
  __syncthreads();   // stage 0 in buffer 0
  read_frags(0, 0, 0);
  // a consumer meets the stage barrier as soon as its last fragment reads of
  // the stage have landed, before the last k-step's MFMAs, and reads the next
  // stage's first fragments while those MFMAs run
  for (int it = 0; it < nk; ++it) {
    const int b = it & 1;
#pragma unroll
    for (int s4 = 0; s4 < 4; ++s4) {
      const int cur = s4 & 1;
      if (s4 < 3) {
        read_frags(cur ^ 1, b, 16 * (s4 + 1));
      } else {
        __syncthreads();   // buffer b read out; stage it + 1 in buffer b ^ 1
        if (it + 1 < nk) read_frags(0, b ^ 1, 0);
      }
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(bf[cur][j], af[cur][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
    if (it + 1 == nk) mfma_drain();   // fence in the block of the last MFMA
  }

  if constexpr (DOTS) __syncthreads();   // the producers' rank-one terms
  const float alpha = A.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
  if constexpr (stage_out) {
    const int srow = wm * 32 * TM + (lane & 31);
    const int scol = wn * 32 * TN + (lane >> 5) * 4;
    // a lane's four columns of a (j, q) group are the same in every row
    // fragment i: their rank-one values are read once for all of them
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = scol + j * 32 + 8 * q;
        f32x4_t r1 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (HAS_MEAN) r1 = *reinterpret_cast<const f32x4_t*>(rho_sh + cl);
#pragma unroll
        for (int i = 0; i < TM; ++i) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(acc[i][j][4 * q + e], alpha, r1[e]);
          const u32x2_t pk = {bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3])};
          *reinterpret_cast<u32x2_t*>(stg + (srow + 32 * i) * kStLd + 2 * cl) = pk;
        }
      }
    }
    __syncthreads();   // tile staged (the producers store too)
    store_staged();
    if (cs.psum) col_stats();   // uniform
  } else {
  const bool full = (m0 + BM <= m_end) && (n0 + BN <= n);
  const bool vec = full && (ldc % 4 == 0) &&
                   ((reinterpret_cast<uintptr_t>(c) & (OUT_BF16 ? 7 : 15)) == 0);
  const int64_t row_base = m0 + wm * 32 * TM + (lane & 31);
  const int cl_base = wn * 32 * TN + (lane >> 5) * 4;   // tile-local column of v = 0
  // row blocks outermost: the eight partial writes that fill one 128-byte
  // output line follow each other closely, so the line is whole in L2 before
  // it can be evicted (written back in pieces, it costs HBM bandwidth twice)
#pragma unroll
  for (int i = 0; i < TM; ++i) {
    const int64_t row = row_base + i * 32;
#pragma unroll
    for (int j = 0; j < TN; ++j) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = cl_base + j * 32 + 8 * q;
        const int64_t col = n0 + cl;
        f32x4_t r1 = {0.0f, 0.0f, 0.0f, 0.0f};
        if (HAS_MEAN) r1 = *reinterpret_cast<const f32x4_t*>(rho_sh + cl);
        float y[4];
#pragma unroll
        for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(acc[i][j][4 * q + e], alpha, r1[e]);
        if (vec) {
          if (OUT_BF16) {
            const u32x2_t pk = {bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3])};
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
              store_out((uint16_t)bf16x2_rne(y[e], 0.0f), static_cast<uint16_t*>(c) + row * ldc + col + e);
            else
              store_out(y[e], static_cast<float*>(c) + row * ldc + col + e);
          }
        }
      }
    }
  }
  }
}

namespace {

size_t ws_lds_bytes(int tm, int tn) {
  return (size_t)2 * 64 * (tm + tn) * kWsLdsK * 2 + (size_t)64 * tn * 4;
}

constexpr size_t kWsLdsLimit = 160 * 1024 - 512;

// SG: K % 256 == 0, scale bytes loaded a 256-wide group at a time
template <int TM, int TN, bool OB, bool HM, bool SG, bool RG = false>
hipError_t launch_ws(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m, int64_t n,
                     int64_t k, const int64_t* offs, int nseg, void* c, int64_t ldc,
                     hipStream_t st, int splits = 1, int64_t c_split = 0,
                     const float* rho = nullptr,
                     const ColStats& cs = ColStats{nullptr, nullptr, nullptr, nullptr}) {
  constexpr int PF = SG ? 4 : 2, BM = 64 * TM, BN = 64 * TN;
  const size_t lds = ws_lds_bytes(TM, TN) + (HM && !RG ? (size_t)k * 2 : 0);
  {
    const hipError_t e = lds_attr_once<&k_gemm_ws<TM, TN, PF, OB, HM, SG, RG>>((int)kWsLdsLimit);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles_m = chunk_upper_bound(m, offs ? nseg : 1, BM);
  dim3 grid((unsigned)((n + BN - 1) / BN), (unsigned)tiles_m, (unsigned)splits);
  const QOperand mu = mean ? *mean : QOperand{nullptr, nullptr, nullptr};
  k_gemm_ws<TM, TN, PF, OB, HM, SG, RG><<<grid, 512, lds, st>>>(a, b, mu, m, n, k / splits, offs,
                                                                nseg, c, ldc, k, c_split, rho, cs);
  return hipGetLastError();
}

template <int TM, int TN, bool SG>
hipError_t launch_ws_sg(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                        int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                        int64_t ldc, hipStream_t st) {
  if (c_bf16)
    return mean ? launch_ws<TM, TN, true, true, SG>(a, mean, b, m, n, k, offs, nseg, c, ldc, st)
                : launch_ws<TM, TN, true, false, SG>(a, mean, b, m, n, k, offs, nseg, c, ldc, st);
  return mean ? launch_ws<TM, TN, false, true, SG>(a, mean, b, m, n, k, offs, nseg, c, ldc, st)
              : launch_ws<TM, TN, false, false, SG>(a, mean, b, m, n, k, offs, nseg, c, ldc, st);
}

template <int TM, int TN>
hipError_t launch_ws_any(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                         int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                         int64_t ldc, hipStream_t st) {
  if (k % 256 == 0)
    return launch_ws_sg<TM, TN, true>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
  return launch_ws_sg<TM, TN, false>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
}

}  // namespace

// Variants (workgroup tile): 1: 256 x 192, 2: 256 x 128.  The tile is
// chosen by rounds of workgroups over the 256 CUs (one resident workgroup
// per CU) times the tile's work.  Returns 0 when the kernel does not apply.
int ws_pick(int64_t m, int64_t n, int64_t k, int nseg_eff, bool has_mean) {
  if (k % kWsBK != 0) return 0;
  struct Cand { int id, tm, tn; double eff; };
  const Cand cands[2] = {{1, 4, 3, 1.0}, {2, 4, 2, 0.95}};
  int best = 0;
  double best_cost = 0;
  for (const Cand& cd : cands) {
    // with a mean, its dequantized row (k fp16 values, k <= 32768) shares the LDS
    if (has_mean && k > 4 * kProducers * 32) continue;
    if (ws_lds_bytes(cd.tm, cd.tn) + (has_mean ? (size_t)k * 2 : 0) > kWsLdsLimit) continue;
    const int64_t bm = 64 * cd.tm, bn = 64 * cd.tn;
    const int64_t tiles = chunk_upper_bound(m, nseg_eff, bm) * ((n + bn - 1) / bn);
    const double rounds = (double)((tiles + 255) / 256);
    const double cost = rounds * bm * bn / cd.eff;
    if (best == 0 || cost < best_cost) {
      best = cd.id;
      best_cost = cost;
    }
  }
  return best;
}

// Split-K product for short, wide outputs (the wgrad product): fp32
// partials part[z] = deq(A[:, z k/S ..]) deq(B[:, z k/S ..])^T, each m x n
// with row stride n; k / splits a multiple of 64.  256 x 192 tiles.
hipError_t launch_gemm_ws_splitk(const QOperand& a, const QOperand& b, int64_t m, int64_t n,
                                 int64_t k, int splits, float* part, hipStream_t st) {
  if (splits < 1 || k % splits != 0 || (k / splits) % kWsBK != 0) return hipErrorInvalidValue;
  if ((k / splits) % 256 == 0)
    return launch_ws<4, 3, false, false, true>(a, nullptr, b, m, n, k, nullptr, 1, part, n,
                                                      st, splits, m * n);
  return launch_ws<4, 3, false, false, false>(a, nullptr, b, m, n, k, nullptr, 1, part, n,
                                                     st, splits, m * n);
}

// rank-one row precomputed: 256 x 192 (variant 1) or 256 x 128 (variant 2)
// tiles; with cs set (bf16 output only) the epilogue also writes the column
// statistics of the output
template <int TM, int TN>
hipError_t launch_ws_rho(const QOperand& a, const float* rho, const QOperand& b, int64_t m,
                         int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                         int64_t ldc, hipStream_t st, const ColStats& cs) {
  static_assert(64 * TM == kGemmRows, "the statistics' chunks are the row tiles");
  if (cs.psum && !c_bf16) return hipErrorInvalidValue;
  if (k % 256 == 0) {
    if (c_bf16)
      return launch_ws<TM, TN, true, true, true, true>(a, nullptr, b, m, n, k, offs, nseg, c,
                                                       ldc, st, 1, 0, rho, cs);
    return launch_ws<TM, TN, false, true, true, true>(a, nullptr, b, m, n, k, offs, nseg, c,
                                                      ldc, st, 1, 0, rho);
  }
  if (c_bf16)
    return launch_ws<TM, TN, true, true, false, true>(a, nullptr, b, m, n, k, offs, nseg, c,
                                                      ldc, st, 1, 0, rho, cs);
  return launch_ws<TM, TN, false, true, false, true>(a, nullptr, b, m, n, k, offs, nseg, c,
                                                     ldc, st, 1, 0, rho);
}

hipError_t launch_gemm_ws_rho(int variant, const QOperand& a, const float* rho, const QOperand& b,
                              int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
                              void* c, bool c_bf16, int64_t ldc, hipStream_t st,
                              const ColStats& cs) {
  if (variant == 1)
    return launch_ws_rho<4, 3>(a, rho, b, m, n, k, offs, nseg, c, c_bf16, ldc, st, cs);
  if (variant == 2)
    return launch_ws_rho<4, 2>(a, rho, b, m, n, k, offs, nseg, c, c_bf16, ldc, st, cs);
  return hipErrorInvalidValue;
}

hipError_t launch_gemm_ws(int variant, const QOperand& a, const QOperand* mean, const QOperand& b,
                          int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                          bool c_bf16, int64_t ldc, hipStream_t st) {
  switch (variant) {
    case 1: return launch_ws_any<4, 3>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
    case 2: return launch_ws_any<4, 2>(a, mean, b, m, n, k, offs, nseg, c, c_bf16, ldc, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace averis
