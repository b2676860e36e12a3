// Quantized NT GEMM for gfx950 with the 4-bit operands staged in LDS as codes
// (K % 256 == 0).
//
// Computes the Averis products of the "Lighthouse" review §2.2 (forward
// Y = 1 (mean_q W_q) + X_R,q W_q and dgrad dX = 1 (mean_q,D W_q^T) +
// D_R,q W_q^T) as C = alpha deq(A) deq(B)^T + 1 rho^T, rho the rank-one row
// the split of A computed (or none), alpha = S_dec(A) S_dec(B).
//
// One workgroup of four wavefronts per CU (one per SIMD, 512 registers each),
// a 2 x 2 wave grid over a 256 x (64 FN) output tile; each wave owns a
// 128 x (32 FN) sub-tile: 4 x FN accumulators of v_mfma_f32_32x32x16_f16 in
// the accumulation registers.
//
// Data movement.  The codes and scale bytes go from global memory to LDS by
// direct-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes land at
// M0 + 16 lane), a window of four 64-wide K stages at a time: per operand row
// the window's 128 code bytes (eight lanes to a row, eight rows to a load:
// few cache lines per load, which is what the address unit's time goes by)
// and its 16 scale bytes (one lane to a row).  Within a row the eight 16-byte
// pieces are stored in the order piece ^ (row mod 8), so the fragment reads
// below hit eight distinct bank groups.  Two window slots: the loads of window
// w + 2 go into window w's slot after the one barrier per window (every wave
// has read window w out by then), spread over three stages at one load per
// eight MFMAs, so they never queue up in front of the MFMAs.
//
// Dequantization.  v_mfma_f32_32x32x16_f16 takes 8 consecutive k of a row per
// lane (k 8 (lane >> 5) .. + 7 of the k-step).  The contraction does not care
// which k a k-step covers as long as A and B agree, so k-step js of lane half
// h takes the stage's elements 32 h + 8 js .. + 7: one 16-byte LDS read per
// fragment row gives a lane its codes for all four k-steps of a stage, and
// its two scale blocks are 2 h and 2 h + 1.  Each wave dequantizes its own
// fragments exactly to fp16 (v_cvt_scalef32_pk_f16_fp4 with scale 1 gives
// the code values; v_pk_mul_f16 by the E4M3 scale decoded exactly by
// v_cvt_scalef32_pk_f16_fp8; an E2M1 value times an E4M3 scale has at most 6
// significant bits and lies in [2^-10, 2688]) one k-step ahead of the MFMAs
// that use them: four VALU instructions per MFMA, interleaved with the MFMAs
// by sched_group_barrier.  The products are exact in fp32; the only roundings
// are the fp32 accumulation (k-steps in order, the same on every run) and the
// epilogue.
//
// Epilogue: y = fma(acc, alpha, rho_j).  bf16 output is staged in the freed
// LDS and stored in 16-byte pieces, eight lanes to a 128-byte line, with
// streaming (nontemporal) stores; with
// column statistics requested the staged tile's per-column fp64 sum, max,
// min and smallest nonzero magnitude go out too.  fp32 output (split-K
// partials) is stored directly, 16 bytes per lane, with plain stores: the
// reduce that follows reads the partials back while they are still cached.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "gemm_common.hpp"
#include "launch.hpp"
#include "segments.hpp"

namespace averis {
namespace {

typedef __attribute__((address_space(3))) void lds_void;

template <int V>
struct WIC {
  static constexpr int value = V;
};

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt in bits 3:0 and 15:14; expcnt and
// lgkmcnt at their maxima, i.e. not waited for)
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

constexpr int kWinBM = 256;        // output rows per tile
constexpr int kWinThreads = 256;   // four waves

constexpr size_t win_ring_bytes(int fn) {
  return (size_t)(kWinBM + 64 * fn) * (2 * 128 + 2 * 16);
}
constexpr size_t win_stage_row(int fn) { return (size_t)2 * 64 * fn + 16; }
// staged tile + the statistics' row-group partials
constexpr size_t win_epi_bytes(int fn) {
  return (size_t)kWinBM * win_stage_row(fn) +
         (size_t)(kWinThreads / (32 * fn) > 0 ? kWinThreads / (32 * fn) : 1) * 64 * fn * 16 +
         (size_t)(kWinThreads / (32 * fn) > 0 ? kWinThreads / (32 * fn) : 1) * 32 * fn * 4;
}
// the rank-one row (64 fn floats) lives past the ring: it is loaded with the
// first window and read in the epilogue
constexpr size_t win_lds_bytes(int fn) {
  return (win_ring_bytes(fn) > win_epi_bytes(fn) ? win_ring_bytes(fn) : win_epi_bytes(fn)) +
         (size_t)64 * fn * 4;
}

}  // namespace

template <int FN, bool OUT_BF16, bool RHO, bool STATS>
__global__ __launch_bounds__(kWinThreads, 1) void k_gemm_win(
    QOperand A, QOperand B, int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
    void* c, int64_t ldc, int64_t kld, int64_t c_split, const float* rho_g, ColStats cs) {
  constexpr int BM = kWinBM, BN = 64 * FN, ROWS = BM + BN;
  constexpr int WSLOT = ROWS * 128;   // a window's codes: four stages, 128 bytes per row
  constexpr int SSLOT = ROWS * 16;    // its scale bytes: 16 per row
  constexpr int NCI = ROWS / 8;       // code loads per window, eight rows each
  constexpr int NSI = ROWS / 64;      // scale loads per window, 64 rows each
  constexpr int CPW = NCI / 4;        // code loads per wave
  constexpr int SPW = (NSI + 3) / 4;  // scale loads per wave, at most
  constexpr int NF = 4 + FN;          // fragments a wave dequantizes: 4 of A, FN of B
  static_assert(NCI % 4 == 0 && BM % 32 == 0, "whole code loads per wave");
  static_assert(!STATS || OUT_BF16, "statistics of a bf16 output");
  extern __shared__ __attribute__((aligned(16))) unsigned char smem_win[];
  unsigned char* ring = smem_win;                  // [2][WSLOT]
  unsigned char* sring = smem_win + 2 * WSLOT;     // [2][SSLOT]

  int64_t tile_x, tile_y;
  xcd_tile(tile_x, tile_y);
  const SegRange sr = locate_chunk(offs, nseg, m, BM, tile_y);
  if (sr.seg < 0) return;
  const int seg = sr.seg;
  const int64_t m0 = sr.r0, m_end = sr.r1;
  const int64_t n0 = tile_x * BN;
  // split-K (gridDim.z > 1): split z contracts the k columns from z k of
  // operands whose rows hold kld columns, into c + z c_split
  const int64_t kh = kld >> 1, kb = kld >> 4;
  const int64_t kz = (int64_t)blockIdx.z * k;
  c = static_cast<char*>(c) + (int64_t)blockIdx.z * c_split * (OUT_BF16 ? 2 : 4);
  const int64_t boff = offs ? (int64_t)seg * n : 0;
  const int t = threadIdx.x, lane = t & 63;
  const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
  const int wm = wave >> 1, wn = wave & 1;
  const int nw = (int)(k >> 8);
  const int rows_here = (int)(m_end - m0 < BM ? m_end - m0 : BM);
  const int cols_here = (int)(n - n0 < BN ? n - n0 : BN);

  const uint8_t* a_c = A.codes + m0 * kh + (kz >> 1);
  const uint8_t* b_c = B.codes + (boff + n0) * kh + (kz >> 1);
  const uint8_t* a_s = A.scales + m0 * kb + (kz >> 4);
  const uint8_t* b_s = B.scales + (boff + n0) * kb + (kz >> 4);

  // code load j of a window: rows 8 j .. 8 j + 7 of the tile's A rows then B
  // rows; lane l -> row 8 j + (l >> 3), LDS piece l & 7 <- the row's 16-byte
  // piece (l & 7) ^ (l >> 3) of the window (piece 2 s + h: stage s, k-half
  // h).  Rows past the edge are clamped to the last valid one: their products
  // only reach outputs that are never stored.
  const int lr = lane >> 3;
  const uint32_t piece_off = 16u * (uint32_t)((lane & 7) ^ lr);
  uint32_t cofs[CPW];
#pragma unroll
  for (int q = 0; q < CPW; ++q) {
    const int j = wave + 4 * q;
    const bool isa = 8 * j < BM;
    const int r = (isa ? 8 * j : 8 * j - BM) + lr;
    const int lim = isa ? rows_here : cols_here;
    const int rr = r < lim ? r : lim - 1;
    cofs[q] = (uint32_t)(rr * kh) + piece_off;
  }
  // scale load i: rows 64 i .. 64 i + 63, one lane (16 bytes) per row
  uint32_t sofs[SPW];
#pragma unroll
  for (int q = 0; q < SPW; ++q) {
    const int i = wave + 4 * q;
    const bool isa = 64 * i < BM;
    const int r = (isa ? 64 * i : 64 * i - BM) + lane;
    const int lim = isa ? rows_here : cols_here;
    const int rr = r < lim ? r : lim - 1;
    sofs[q] = (uint32_t)(rr * kb);
  }
  // a window's loads in three parts (scale loads and the first code loads,
  // then the other code loads in two); a window past the end loads the last
  // one again (never read), so every wave issues the same loads
  constexpr int P0 = (CPW + SPW) / 3 > SPW ? (CPW + SPW) / 3 - SPW : 0;
  constexpr int P1 = P0 + (CPW - P0) / 2;
  // fewest loads any wave issues for one window
  constexpr int LOADS_MIN = CPW + NSI / 4;
  auto dma_part = [&](int w, int slot, auto hc) __attribute__((always_inline)) {
    constexpr int hf = decltype(hc)::value;
    const int wl = w < nw ? w : nw - 1;
    if constexpr (hf == 0) {
#pragma unroll
      for (int q = 0; q < SPW; ++q) {
        const int i = wave + 4 * q;
        if (NSI % 4 == 0 || i < NSI) {
          // 64 i < BM exactly when q < BM / 256 (wave < 4, BM % 256 == 0)
          const uint8_t* base = (q < BM / 256 ? a_s : b_s) + 16 * wl;
          __builtin_amdgcn_global_load_lds((const void*)(base + sofs[q]),
                                           (lds_void*)(sring + slot * SSLOT + i * 1024), 16, 0, 0);
        }
      }
    }
    constexpr int q0 = hf == 0 ? 0 : hf == 1 ? P0 : P1;
    constexpr int q1 = hf == 0 ? P0 : hf == 1 ? P1 : CPW;
#pragma unroll
    for (int q = q0; q < q1; ++q) {
      const int j = wave + 4 * q;
      // 8 j < BM exactly when q < BM / 32 (wave < 4, BM / 8 a multiple of 4)
      const uint8_t* base = (q < BM / 32 ? a_c : b_c) + 128 * wl;
      __builtin_amdgcn_global_load_lds((const void*)(base + cofs[q]),
                                       (lds_void*)(ring + slot * WSLOT + j * 1024), 16, 0, 0);
    }
  };

  // the rank-one row goes to LDS by a direct-to-LDS load (4 bytes a lane,
  // column n0 + t; columns past n repeat the last one, never stored), issued
  // before the first window's loads, so the prologue's counted wait covers it
  // and its latency hides under them
  constexpr size_t kRhoOff = win_lds_bytes(FN) - (size_t)BN * 4;
  float* rho_sh = reinterpret_cast<float*>(smem_win + kRhoOff);
  if constexpr (RHO) {
    if (64 * wave < BN) {   // uniform per wave
      const int64_t cj = n0 + 64 * wave + lane;
      __builtin_amdgcn_global_load_lds((const void*)(rho_g + boff + (cj < n ? cj : n - 1)),
                                       (lds_void*)(smem_win + kRhoOff + 256 * wave), 4, 0, 0);
    }
  }

  u32x4_t cw[2][NF];     // a stage's codes per fragment, two stages
  u32x4_t sraw[NF];      // a window's scale bytes per fragment row (read once)
  uint32_t sg[NF][2];    // the lane's 8 of them: stage s's pair in word s & 1 of sg[f][s >> 1]
  half2_t fs[2][NF];     // a stage's two scales per fragment, fp16
  half8_t dq[2][NF];     // dequantized fragments of a k-step, two k-steps
  f32x16_t acc[4][FN];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < FN; ++j)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.0f;

  const int lrow = lane & 31, lh = lane >> 5;
  // stage s of the window in slot `slot` -> cw[p]: row R's piece 2 s + h is
  // stored at 16 ((2 s + h) ^ (R & 7)), and R & 7 = lane & 7 for every
  // fragment (fragment rows start at multiples of 32)
  auto read_stage = [&](int slot, auto sc, auto pc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value, p = decltype(pc)::value;
    const unsigned char* sl = ring + slot * WSLOT + lrow * 128 + 16 * ((2 * s + lh) ^ (lane & 7));
#pragma unroll
    for (int i = 0; i < 4; ++i)
      cw[p][i] = *reinterpret_cast<const u32x4_t*>(sl + (wm * 128 + 32 * i) * 128);
#pragma unroll
    for (int j = 0; j < FN; ++j)
      cw[p][4 + j] = *reinterpret_cast<const u32x4_t*>(sl + (BM + wn * 32 * FN + 32 * j) * 128);
  };
  // a window's scale bytes: one 16-byte read per fragment row (16
  // consecutive rows of 16 bytes per eight lanes: no bank conflicts) ...
  auto read_scales = [&](int slot) __attribute__((always_inline)) {
    const unsigned char* ss = sring + slot * SSLOT + lrow * 16;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const int row0 = f < 4 ? wm * 128 + 32 * f : BM + wn * 32 * FN + 32 * (f - 4);
      sraw[f] = *reinterpret_cast<const u32x4_t*>(ss + row0 * 16);
    }
  };
  // ... of which the lane keeps its half's two bytes per stage
  auto pick_scales = [&]() __attribute__((always_inline)) {
    const uint32_t sel = lh ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      sg[f][0] = __builtin_amdgcn_perm(sraw[f].y, sraw[f].x, sel);
      sg[f][1] = __builtin_amdgcn_perm(sraw[f].w, sraw[f].z, sel);
    }
  };
  // stage s's scales -> fs[p] (v_cvt_scalef32_pk_f16_fp8 decodes every finite
  // E4M3 byte exactly, subnormals included), a k-step ahead of their use
  auto prep_scales = [&](auto pc, auto sc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, s = decltype(sc)::value;
#pragma unroll
    for (int f = 0; f < NF; ++f)
      fs[p][f] = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(sg[f][s >> 1], 1.0f, (s & 1) != 0);
  };
  // k-step js of code buffer p -> dq[q]
  auto deq = [&](auto pc, auto jc, auto qc) __attribute__((always_inline)) {
    constexpr int p = decltype(pc)::value, js = decltype(jc)::value, q = decltype(qc)::value;
#pragma unroll
    for (int f = 0; f < NF; ++f) {
      const uint32_t w = cw[p][f][js];
      const _Float16 sh = (js >> 1) ? fs[p][f].y : fs[p][f].x;
      const half2_t s = {sh, sh};
      const half2_t h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s;
      const half2_t h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s;
      const half2_t h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s;
      const half2_t h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s;
      dq[q][f] = half8_t{h0.x, h0.y, h1.x, h1.y, h2.x, h2.y, h3.x, h3.y};
    }
  };
  // the MFMA takes the B fragment first, so a lane's accumulators hold four
  // consecutive output columns of one output row
  auto mfmas = [&](auto qc) __attribute__((always_inline)) {
    constexpr int q = decltype(qc)::value;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(dq[q][4 + j], dq[q][i], acc[i][j], 0, 0, 0);
  };
  // a workgroup barrier without a memory fence (a fence would wait for every
  // load in flight): the waits before it are explicit, and the empty asm
  // statements keep the compiler from moving memory accesses across it
  auto barrier = []() __attribute__((always_inline)) {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
  };
  // per MFMA: NV VALU instructions, an LDS read (DS) and, with DM, a load
  // every eight MFMAs
  auto interleave = [](auto nvc, auto dsc, auto dmc) __attribute__((always_inline)) {
    constexpr int NV = decltype(nvc)::value;
    constexpr bool DS = decltype(dsc)::value != 0, DM = decltype(dmc)::value != 0;
#pragma unroll
    for (int i = 0; i < 4 * FN; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      if constexpr (DM) {
        if (i % 8 == 0) __builtin_amdgcn_sched_group_barrier(0x010, 1, 0);
      }
      if constexpr (DS) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      if constexpr (DS || DM) __builtin_amdgcn_sched_group_barrier(0x004, 2, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, NV, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  // prologue: windows 0 and 1 in flight, wait for window 0
  dma_part(0, 0, WIC<0>{});
  dma_part(0, 0, WIC<1>{});
  dma_part(0, 0, WIC<2>{});
  dma_part(1, 1, WIC<0>{});
  dma_part(1, 1, WIC<1>{});
  dma_part(1, 1, WIC<2>{});
  wait_vmcnt<LOADS_MIN>();
  barrier();
  read_stage(0, WIC<0>{}, WIC<0>{});
  read_scales(0);
  pick_scales();
  prep_scales(WIC<0>{}, WIC<0>{});
  deq(WIC<0>{}, WIC<0>{}, WIC<0>{});

  // stage s of window w (slot w & 1); on entry its codes are in cw[s & 1],
  // its scales in fs[s & 1] and its k-step 0 in dq[0].  k-step 0; at s == 3:
  // window w + 1 landed -> barrier (every wave done with window w's slot);
  // then this stage's part of a window's loads (s == 3: part 0 of window
  // w + 2 into slot w & 1; s == 0, 1: parts 1, 2 of window w + 1) and the
  // reads of the next stage under k-step 1; k-steps 2, 3, with the next
  // stage's scales and k-step 0 dequantized under them.
  auto stage = [&](int w, auto sc) __attribute__((always_inline)) {
    constexpr int s = decltype(sc)::value, p = s & 1;
    constexpr WIC<p> pc{};
    deq(pc, WIC<1>{}, WIC<1>{});
    mfmas(WIC<0>{});
    interleave(WIC<4>{}, WIC<0>{}, WIC<0>{});
    if constexpr (s == 3) {
      wait_vmcnt<0>();
      barrier();
    }
    __builtin_amdgcn_sched_barrier(0);
    if constexpr (s == 3) dma_part(w + 2, w & 1, WIC<0>{});
    if constexpr (s == 0) dma_part(w + 1, (w + 1) & 1, WIC<1>{});
    if constexpr (s == 1) dma_part(w + 1, (w + 1) & 1, WIC<2>{});
    if constexpr (s < 3) {
      read_stage(w & 1, WIC<s + 1>{}, WIC<p ^ 1>{});
    } else {
      read_stage((w + 1) & 1, WIC<0>{}, WIC<p ^ 1>{});
      read_scales((w + 1) & 1);
    }
    constexpr int DM = s != 2 ? 1 : 0;
    deq(pc, WIC<2>{}, WIC<0>{});
    mfmas(WIC<1>{});
    interleave(WIC<4>{}, WIC<1>{}, WIC<DM>{});
    if constexpr (s == 3) pick_scales();
    prep_scales(WIC<p ^ 1>{}, WIC<(s + 1) & 3>{});
    deq(pc, WIC<3>{}, WIC<1>{});
    mfmas(WIC<0>{});
    interleave(WIC<5>{}, WIC<0>{}, WIC<DM>{});
    deq(WIC<p ^ 1>{}, WIC<0>{}, WIC<0>{});
    mfmas(WIC<1>{});
    interleave(WIC<6>{}, WIC<0>{}, WIC<DM>{});
  };
  // every window the same four stages.  The last stage reads and dequantizes
  // a stage past the end (a copy of the last window, never multiplied), and
  // window 0's stages 0, 1 issue window 1's parts 1, 2 again (same bytes
  // into the same slot, before anything reads it)
  for (int w = 0; w < nw; ++w) {
    stage(w, WIC<0>{});
    stage(w, WIC<1>{});
    stage(w, WIC<2>{});
    stage(w, WIC<3>{});
  }
  // the accumulator copies the compiler hoists onto the loop's exit path
  // come before this fence; it pads those itself (s_nop ahead of the first)
  mfma_drain();

  // ------------------------------------------------------------------ epilogue
  wait_vmcnt<0>();
  __syncthreads();   // every load landed; every wave done with the ring
  const float alpha = A.tscale[2 * seg + 1] * B.tscale[(offs ? 2 * seg : 0) + 1];
  constexpr int kStLd = (int)win_stage_row(FN);
  unsigned char* stg = smem_win;
  const int srow = wm * 128 + lrow;
  const int scol = wn * 32 * FN + lh * 4;
  if constexpr (OUT_BF16) {
    // a lane's four columns of a (j, q) group are the same in every row
    // fragment i: their rank-one values are read once for all of them, the
    // four groups of a fragment column j together (one wait for the four
    // LDS reads, not one per group)
#pragma unroll
    for (int j = 0; j < FN; ++j) {
      f32x4_t r1[4];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        r1[q] = f32x4_t{0.0f, 0.0f, 0.0f, 0.0f};
        if constexpr (RHO) r1[q] = *reinterpret_cast<const f32x4_t*>(rho_sh + scol + j * 32 + 8 * q);
      }
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int cl = scol + j * 32 + 8 * q;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(acc[i][j][4 * q + e], alpha, r1[q][e]);
          const u32x2_t pk = {bf16x2_rne(y[0], y[1]), bf16x2_rne(y[2], y[3])};
          *reinterpret_cast<u32x2_t*>(stg + (srow + 32 * i) * kStLd + 2 * cl) = pk;
        }
      }
    }
    __syncthreads();   // tile staged
    constexpr int CPR = 2 * BN / 16;   // 16-byte pieces per tile row
    static_assert((BM * CPR) % kWinThreads == 0, "whole store rounds");
    uint16_t* cb = static_cast<uint16_t*>(c) + m0 * ldc + n0;
    const bool st_vec = (ldc % 8 == 0) && ((reinterpret_cast<uintptr_t>(c) & 15) == 0);
#pragma unroll 4
    for (int it = 0; it < BM * CPR / kWinThreads; ++it) {
      const int cidx = t + kWinThreads * it;
      const int r = cidx / CPR, cc = cidx - r * CPR;
      if (r >= rows_here) continue;
      const u32x4_t v = *reinterpret_cast<const u32x4_t*>(stg + r * kStLd + cc * 16);
      uint16_t* dst = cb + (int64_t)r * ldc + cc * 8;
      if (st_vec && cc * 8 + 8 <= cols_here) {
        store_stream(v, reinterpret_cast<u32x4_t*>(dst));
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e)
          if (cc * 8 + e < cols_here) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
      }
    }
    if constexpr (STATS) {
      // column statistics of the staged tile, as stored: per column the fp64
      // sum, max, min and smallest nonzero magnitude of its rows_here values
      // -> the chunk's partials [tile_y][col].  Thread (pp, g) takes column
      // pair pp and rows g, g + G, ...; the G row groups meet in LDS past the
      // staged tile.
      constexpr int P = BN / 2, G = kWinThreads / P;
      static_assert(G >= 1, "a row group per column pair");
      double* gs = reinterpret_cast<double*>(smem_win + (size_t)BM * kStLd);   // [G][BN]
      float* gmx = reinterpret_cast<float*>(gs + G * BN);          // [G][BN]
      float* gmn = gmx + G * BN;                                   // [G][BN]
      uint32_t* gmz = reinterpret_cast<uint32_t*>(gmn + G * BN);   // [G][P]
      typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
      typedef short i16x2 __attribute__((ext_vector_type(2)));
      // bf16 bits -> 16-bit integers in the order of the values (a negative
      // value's magnitude bits flipped): one packed integer max or min covers
      // both columns of a pair; the map is its own inverse
      auto ordered = [](uint32_t w) __attribute__((always_inline)) {
        const i16x2 x = __builtin_bit_cast(i16x2, w);
        return x ^ ((x >> 15) & i16x2{0x7FFF, 0x7FFF});
      };
      const int pp = t % P, g = t / P;
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
        constexpr int U = 4;   // rows whose reads are in flight together
        const unsigned char* qp = stg + g * kStLd + 4 * pp;
        int r = g;
        for (; r + (U - 1) * G < rows_here; r += U * G, qp += U * G * kStLd) {
          uint32_t w[U];
#pragma unroll
          for (int u = 0; u < U; ++u) w[u] = *reinterpret_cast<const uint32_t*>(qp + u * G * kStLd);
#pragma unroll
          for (int u = 0; u < U; ++u) {
            s0 += (double)__uint_as_float(w[u] << 16);
            s1 += (double)__uint_as_float(w[u] & 0xFFFF0000u);
            add_row(w[u]);
          }
        }
        for (; r < rows_here; r += G, qp += G * kStLd) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(qp);
          s0 += (double)__uint_as_float(w << 16);
          s1 += (double)__uint_as_float(w & 0xFFFF0000u);
          add_row(w);
        }
        const uint32_t bx = __builtin_bit_cast(uint32_t, ordered(__builtin_bit_cast(uint32_t, mx)));
        const uint32_t bn = __builtin_bit_cast(uint32_t, ordered(__builtin_bit_cast(uint32_t, mn)));
        // a row group without rows keeps -inf / +inf
        const bool any = g < rows_here;
        gs[g * BN + 2 * pp] = s0;
        gs[g * BN + 2 * pp + 1] = s1;
        gmx[g * BN + 2 * pp] = any ? __uint_as_float(bx << 16) : -__builtin_inff();
        gmx[g * BN + 2 * pp + 1] = any ? __uint_as_float(bx & 0xFFFF0000u) : -__builtin_inff();
        gmn[g * BN + 2 * pp] = any ? __uint_as_float(bn << 16) : __builtin_inff();
        gmn[g * BN + 2 * pp + 1] = any ? __uint_as_float(bn & 0xFFFF0000u) : __builtin_inff();
        gmz[g * P + pp] = __builtin_bit_cast(uint32_t, mz);
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
    }
  } else {
    const bool vec = (m0 + BM <= m_end) && (n0 + BN <= n) && (ldc % 4 == 0) &&
                     ((reinterpret_cast<uintptr_t>(c) & 15) == 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t row = m0 + srow + 32 * i;
#pragma unroll
      for (int j = 0; j < FN; ++j) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cl = scol + j * 32 + 8 * q;
          const int64_t col = n0 + cl;
          f32x4_t r1 = {0.0f, 0.0f, 0.0f, 0.0f};
          if constexpr (RHO) r1 = *reinterpret_cast<const f32x4_t*>(rho_sh + cl);
          float y[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) y[e] = __builtin_fmaf(acc[i][j][4 * q + e], alpha, r1[e]);
          float* dst = static_cast<float*>(c) + row * ldc + col;
          if (vec) {
            store_out(f32x4_t{y[0], y[1], y[2], y[3]}, reinterpret_cast<f32x4_t*>(dst));
          } else if (row < m_end) {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (col + e < n) dst[e] = y[e];
          }
        }
      }
    }
  }
}

namespace {

template <int FN, bool OB, bool RHO, bool STATS>
hipError_t launch_win_t(const QOperand& a, const QOperand& b, int64_t m, int64_t n, int64_t k,
                        const int64_t* offs, int nseg, void* c, int64_t ldc, hipStream_t st,
                        int splits, int64_t c_split, const float* rho, const ColStats& cs) {
  constexpr size_t lds = win_lds_bytes(FN);
  static_assert(lds + 64 <= 160 * 1024, "fits one CU's LDS");
  {
    const hipError_t e = lds_attr_once<&k_gemm_win<FN, OB, RHO, STATS>>((int)lds);
    if (e != hipSuccess) return e;
  }
  const int64_t tiles_m = chunk_upper_bound(m, offs ? nseg : 1, kWinBM);
  dim3 grid((unsigned)((n + 64 * FN - 1) / (64 * FN)), (unsigned)tiles_m, (unsigned)splits);
  k_gemm_win<FN, OB, RHO, STATS><<<grid, kWinThreads, lds, st>>>(
      a, b, m, n, k / splits, offs, nseg, c, ldc, k, c_split, rho, cs);
  return hipGetLastError();
}

template <int FN>
hipError_t launch_win_fn(const QOperand& a, const QOperand& b, int64_t m, int64_t n, int64_t k,
                         const int64_t* offs, int nseg, void* c, bool c_bf16, int64_t ldc,
                         hipStream_t st, int splits, int64_t c_split, const float* rho,
                         const ColStats& cs) {
  if (cs.psum) {
    if (!c_bf16 || !rho) return hipErrorInvalidValue;
    return launch_win_t<FN, true, true, true>(a, b, m, n, k, offs, nseg, c, ldc, st, splits,
                                              c_split, rho, cs);
  }
  if (c_bf16) {
    if (rho)
      return launch_win_t<FN, true, true, false>(a, b, m, n, k, offs, nseg, c, ldc, st, splits,
                                                 c_split, rho, cs);
    return launch_win_t<FN, true, false, false>(a, b, m, n, k, offs, nseg, c, ldc, st, splits,
                                                c_split, rho, cs);
  }
  if (rho)
    return launch_win_t<FN, false, true, false>(a, b, m, n, k, offs, nseg, c, ldc, st, splits,
                                                c_split, rho, cs);
  return launch_win_t<FN, false, false, false>(a, b, m, n, k, offs, nseg, c, ldc, st, splits,
                                               c_split, rho, cs);
}

}  // namespace

// Tile width: 64 FN columns, FN in {4, 3, 2}, picked by rounds of
// workgroups over the 256 CUs times the tile's width (one resident workgroup
// per CU); ties go to the wider tile.  0 when the kernel does not apply
// (K per split not a multiple of 256).
int win_pick(int64_t m, int64_t n, int64_t k_split, int nseg_eff, int splits) {
  if (k_split <= 0 || k_split % 256 != 0) return 0;
  int best = 0;
  int64_t best_cost = 0;
  for (int fn = 4; fn >= 2; --fn) {
    const int64_t bn = 64 * fn;
    const int64_t tiles = chunk_upper_bound(m, nseg_eff, kWinBM) * ((n + bn - 1) / bn) * splits;
    const int64_t cost = ((tiles + 255) / 256) * bn;
    if (best == 0 || cost < best_cost) {
      best = fn;
      best_cost = cost;
    }
  }
  return best;
}

hipError_t launch_gemm_win(int fn, const QOperand& a, const float* rho, const QOperand& b,
                           int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
                           void* c, bool c_bf16, int64_t ldc, hipStream_t st, int splits,
                           int64_t c_split, const ColStats& cs) {
  if (splits < 1 || k % splits != 0 || (k / splits) % 256 != 0) return hipErrorInvalidValue;
  switch (fn) {
    case 4: return launch_win_fn<4>(a, b, m, n, k, offs, nseg, c, c_bf16, ldc, st, splits, c_split, rho, cs);
    case 3: return launch_win_fn<3>(a, b, m, n, k, offs, nseg, c, c_bf16, ldc, st, splits, c_split, rho, cs);
    case 2: return launch_win_fn<2>(a, b, m, n, k, offs, nseg, c, c_bf16, ldc, st, splits, c_split, rho, cs);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace averis
