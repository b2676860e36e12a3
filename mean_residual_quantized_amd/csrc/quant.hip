// Split-quant and plain quant kernels for gfx950.
//
// Averis split ("Lighthouse" review §2.1-§2.2; gist.science summary §2):
//   mu_j = (1/l) sum_i a_ij over a segment's rows, X_R = X - 1 mu^T, and
//   Q4(X_R), Q4(mu) quantized separately (NVFP4-style, 16-blocks along cols).
//
// Three launches per call:
//   stats     one pass over A: per row-chunk partial column sums (fp64), max
//             and min (split), or per-chunk max |a| (plain)
//   finalize  (split) per column: mu = fp32(fp64(sum) / l), and the column's
//             max |fp32(a - mu)| = max(fp32(max - mu), fp32(mu - min)) (fp32
//             subtraction is monotone), reduced per column tile
//   quant     per 16-block: residual, block amax, E4M3 scale, Philox SR or RN,
//             packed nibbles; extra workgroups quantize the mean vectors
// Partial sums are exact in fp64 when a column's values span a narrow enough
// range (checked per column from its largest and smallest nonzero magnitude);
// a column that fails the check is summed again exactly (its chunks' partials
// that are exact on their own, and the rows of the others, in a 320-bit
// integer, rounded once), so the mean never depends on the order.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "device_common.hpp"
#include "exact_sum.hpp"
#include "gemm_common.hpp"
#include "launch.hpp"
#include "segments.hpp"

namespace averis {

// ---------------------------------------------------------------------------
// element loads: 8 consecutive columns as fp32
// ---------------------------------------------------------------------------
template <typename T>
struct Load8;

template <>
struct Load8<uint16_t> {  // bf16
  static __device__ __forceinline__ void run(const uint16_t* p, float* v) {
    const uint4 w = *reinterpret_cast<const uint4*>(p);
    v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
    v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
    v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
    v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
  }
};

template <>
struct Load8<float> {
  static __device__ __forceinline__ void run(const float* p, float* v) {
    const float4 a = *reinterpret_cast<const float4*>(p);
    const float4 b = *reinterpret_cast<const float4*>(p + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  }
};

// 8 consecutive elements kept as loaded (bf16: one 16-byte word) and
// unpacked to fp32 where they are used, so many rows fit in flight
template <typename T>
struct Raw8;

template <>
struct Raw8<uint16_t> {
  uint4 w;
  __device__ __forceinline__ void load(const uint16_t* p) { w = *reinterpret_cast<const uint4*>(p); }
  __device__ __forceinline__ float get(int k) const {
    const uint32_t x = k < 2 ? w.x : k < 4 ? w.y : k < 6 ? w.z : w.w;
    return (k & 1) ? bf16_hi(x) : bf16_lo(x);
  }
};

template <>
struct Raw8<float> {
  float4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = *reinterpret_cast<const float4*>(p);
    b = *reinterpret_cast<const float4*>(p + 4);
  }
  __device__ __forceinline__ float get(int k) const {
    const float4& h = k < 4 ? a : b;
    const int kk = k & 3;
    return kk == 0 ? h.x : kk == 1 ? h.y : kk == 2 ? h.z : h.w;
  }
};

__device__ __forceinline__ float block_max(float v, float* red) {
  // max over the 256 threads of a block
  for (int d = 32; d > 0; d >>= 1) v = __builtin_fmaxf(v, __shfl_xor(v, d, 64));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  v = __builtin_fmaxf(__builtin_fmaxf(red[0], red[1]), __builtin_fmaxf(red[2], red[3]));
  __syncthreads();
  return v;
}

// ---------------------------------------------------------------------------
// stats over one chunk of kStatsRows rows: a block covers 128 columns (16
// column-octets x 16 row lanes, 8 rows per thread; the plain pass's maxima are
// kept per kPlainStatsCols-column block).  Every row load of a thread is issued before
// its arithmetic.  A chunk that ends before kStatsRows rows (the last one of
// a segment) clamps its loads to the segment's last row and masks them; a
// full chunk takes the same code without the masks.
// ---------------------------------------------------------------------------
template <bool SPLIT>
struct StatsShape {
  static constexpr int TX = 16;                      // threads across the columns
  static constexpr int TY = 256 / TX;                // row lanes
  static constexpr int CW = TX * 8;                  // columns per block
  static constexpr int U = (int)(kStatsRows / TY);   // rows per thread
  static_assert(SPLIT || CW == kPlainStatsCols, "the plain pass's maxima blocks");
};

// SSQ (with SPLIT): also the column sums of squares, for the mean-energy
// ratio (each square is exact in fp64, one fma per element)
template <typename T, bool SPLIT, bool SSQ = false>
__global__ __launch_bounds__(256) void k_stats(const T* __restrict__ a, int64_t rows, int64_t cols,
                                               int64_t lda, const int64_t* offs, int nseg,
                                               double* __restrict__ psum,
                                               float* __restrict__ pmax,
                                               float* __restrict__ pmin,
                                               float* __restrict__ pmnz,
                                               float* __restrict__ pamax,
                                               double* __restrict__ psq = nullptr) {
  using SH = StatsShape<SPLIT>;
  constexpr int TX = SH::TX, TY = SH::TY, CW = SH::CW, U = SH::U;
  const SegRange sr = locate_chunk(offs, nseg, rows, kStatsRows, blockIdx.y);
  const int tx = threadIdx.x % TX, ty = threadIdx.x / TX;
  const int64_t c = (int64_t)blockIdx.x * CW + tx * 8;
  const bool active = sr.seg >= 0 && c < cols;

  double s[8], sq[8];
  float mx[8], mn[8], mz[8];
  float am = 0.0f;
  // bf16: the smallest nonzero magnitude per column as packed 16-bit
  // (|bits| - 1), where a zero wraps to 0xFFFF and never wins the minimum
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 mzp[4];
#pragma unroll
  for (int w = 0; w < 4; ++w) mzp[w] = u16x2{0xFFFFu, 0xFFFFu};
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    s[k] = 0.0;
    sq[k] = 0.0;
    mx[k] = -__builtin_inff();
    mn[k] = __builtin_inff();
    mz[k] = __builtin_inff();
  }
  // the chunk's rows of this thread: loads first, then the arithmetic; MASK:
  // rows past the segment end (clamped to its last row, so the loads stay
  // legal) are left out of the sums -- a repeated real value is harmless for
  // the max, min and smallest magnitude
  auto accumulate = [&](auto maskc) __attribute__((always_inline)) {
    constexpr bool MASK = decltype(maskc)::value;
    const int64_t rlast = sr.r1 - 1;
    Raw8<T> v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t r = sr.r0 + ty + TY * u;
      v[u].load(a + (MASK && r > rlast ? rlast : r) * lda + c);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const bool ok = !MASK || sr.r0 + ty + TY * u <= rlast;
#pragma unroll
      for (int k = 0; k < 8; ++k) {
        const float x = v[u].get(k);
        if (SPLIT) {
          if (MASK) {
            s[k] += ok ? (double)x : 0.0;
          } else {
            s[k] += (double)x;
          }
          if constexpr (SSQ) {
            const double xd = ok ? (double)x : 0.0;
            sq[k] = __builtin_fma(xd, xd, sq[k]);
          }
          mx[k] = __builtin_fmaxf(mx[k], x);
          mn[k] = __builtin_fminf(mn[k], x);
          if constexpr (sizeof(T) != 2) {
            // smallest nonzero magnitude: sets the grid every value lies on
            const float ax = __builtin_fabsf(x);
            mz[k] = __builtin_fminf(mz[k], ax > 0.0f ? ax : __builtin_inff());
          }
        } else {
          am = __builtin_fmaxf(am, __builtin_fabsf(x));
        }
      }
      if constexpr (SPLIT && sizeof(T) == 2) {
        const uint32_t wd[4] = {v[u].w.x, v[u].w.y, v[u].w.z, v[u].w.w};
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const u16x2 m = __builtin_bit_cast(u16x2, wd[w] & 0x7FFF7FFFu) - u16x2{1, 1};
          mzp[w] = __builtin_elementwise_min(mzp[w], m);
        }
      }
    }
  };
  if (active) {
    if (sr.r1 - sr.r0 == kStatsRows)
      accumulate(std::integral_constant<bool, false>{});
    else
      accumulate(std::integral_constant<bool, true>{});
  }
  if constexpr (SPLIT && sizeof(T) == 2) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t m = mzp[w][h];
        mz[2 * w + h] = m == 0xFFFFu ? __builtin_inff() : __uint_as_float((m + 1u) << 16);
      }
    }
  }
  if constexpr (SPLIT) {
    // 32 KB of LDS: the smallest nonzero magnitudes go through the max buffer
    // in a second round
    __shared__ double ls[TY][CW];
    __shared__ float lmx[TY][CW], lmn[TY][CW];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      ls[ty][tx * 8 + k] = s[k];
      lmx[ty][tx * 8 + k] = mx[k];
      lmn[ty][tx * 8 + k] = mn[k];
    }
    __syncthreads();
    // the row lanes of column j: two threads per column, halves then combined
    const int j = threadIdx.x % CW, hf = threadIdx.x / CW;
    static_assert(2 * CW == 256, "two threads per column");
    const int64_t col = (int64_t)blockIdx.x * CW + j;
    const bool live = sr.seg >= 0 && col < cols;
    const int64_t o = (int64_t)blockIdx.y * cols + col;
    double t = 0.0;
    float m1 = -__builtin_inff(), m0 = __builtin_inff();
    if (hf == 0) {
#pragma unroll
      for (int q = 0; q < TY; ++q) {
        t += ls[q][j];
        m1 = __builtin_fmaxf(m1, lmx[q][j]);
        m0 = __builtin_fminf(m0, lmn[q][j]);
      }
      if (live) {
        psum[o] = t;
        pmax[o] = m1;
        pmin[o] = m0;
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      lmx[ty][tx * 8 + k] = mz[k];
      if constexpr (SSQ) ls[ty][tx * 8 + k] = sq[k];
    }
    __syncthreads();
    if (live && hf == 1) {
      float mzz = __builtin_inff();
#pragma unroll
      for (int q = 0; q < TY; ++q) mzz = __builtin_fminf(mzz, lmx[q][j]);
      pmnz[o] = mzz;
    }
    if constexpr (SSQ) {
      if (live && hf == 0) {
        double t2 = 0.0;
#pragma unroll
        for (int q = 0; q < TY; ++q) t2 += ls[q][j];
        psq[o] = t2;
      }
    }
  } else {
    __shared__ float red[4];
    am = block_max(am, red);
    if (threadIdx.x == 0) pamax[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = am;
  }
}

// ---------------------------------------------------------------------------
// The correctly rounded sum of column j of one segment whose fp64 running sum
// is not certified (certificate below), by one wavefront (all 64 lanes, in
// wave-uniform control flow).  The chunks' fp64 partial sums that are exact
// by their own certificate (a chunk spans far fewer rows and usually a far
// narrower range of values) are added exactly, the rows of the other chunks
// one by one, into a signed 64-bit integer in units of the grid every value
// of the column lies on (2^gexp, from its smallest nonzero magnitude) when the
// column's sum stays below 2^62 of them, else into a 320-bit integer in units
// of 2^-149 (exact_sum.hpp); either is rounded once to the nearest double.
// Chunk c of the segment goes to lane c mod 64; the lanes' accumulators are
// then added by a butterfly of shuffles (exact, so the order is free) and
// every lane gets the result.
// Kept out of line: the finalize passes call it only for a column that fails
// the certificate.
// ---------------------------------------------------------------------------

// Certificate of an fp64 sum of n values of one column: every value is a
// multiple of g = 2^(ez - 1 - P) (ez: binary exponent of the smallest nonzero
// |a|, mnz; P = 7 for bf16 input, 23 for fp32) and every partial sum is at
// most n max|a|, so when that is at most 2^52 g every fp64 addition was exact,
// in any order.  No nonzero value: the sum is 0.
__device__ __forceinline__ bool sum_certified(double n, double amax, float mnz, bool bf16) {
  if (!(mnz < __builtin_inff())) return true;
  int ez;
  (void)__builtin_frexp((double)mnz, &ez);
  return n * amax <= __builtin_ldexp(1.0, 52 + ez - 1 - (bf16 ? 7 : 23));
}

__device__ __noinline__ double exact_column_sum(const void* a, bool bf16, int64_t lda,
                                                int64_t cols, int64_t seg_r0, int64_t seg_r1,
                                                int64_t c0, int64_t c1, int64_t ch, int64_t j,
                                                const double* __restrict__ psum,
                                                const float* __restrict__ pmax,
                                                const float* __restrict__ pmin,
                                                const float* __restrict__ pmnz) {
  const int lane = threadIdx.x & 63;
  // The column's largest and smallest nonzero magnitude over its chunks: when
  // its values, all on the grid 2^gexp of the smallest, sum to below 2^62
  // grid units, a signed 64-bit integer holds the exact sum (in any order)
  // and one rounding gives the correctly rounded double; else the 320-bit sum.
  {
    float am = 0.0f, mz = __builtin_inff();
    for (int64_t c = c0 + lane; c < c1; c += 64) {
      const int64_t o = c * cols + j;
      am = __builtin_fmaxf(am, __builtin_fmaxf(__builtin_fabsf(pmax[o]), __builtin_fabsf(pmin[o])));
      mz = __builtin_fminf(mz, pmnz[o]);
    }
    for (int d = 32; d > 0; d >>= 1) {
      am = __builtin_fmaxf(am, __shfl_xor(am, d, 64));
      mz = __builtin_fminf(mz, __shfl_xor(mz, d, 64));
    }
    if (!(mz < __builtin_inff())) return 0.0;   // no nonzero value
    const int gexp = value_grid_exp(mz, bf16 ? 7 : 23);
    if (grid_sum_fits((double)(seg_r1 - seg_r0), (double)am, gexp)) {   // uniform
      int64_t n = 0;
      for (int64_t c = c0 + lane; c < c1; c += 64) {
        const int64_t r0 = seg_r0 + (c - c0) * ch;
        const int64_t r1 = r0 + ch < seg_r1 ? r0 + ch : seg_r1;
        const int64_t o = c * cols + j;
        const double cam = __builtin_fmax(__builtin_fabs((double)pmax[o]), __builtin_fabs((double)pmin[o]));
        if (sum_certified((double)(r1 - r0), cam, pmnz[o], bf16)) {
          n += grid_int64(psum[o], gexp);   // an exact sum of values on the grid
        } else {
          for (int64_t r = r0; r < r1; ++r) {
            const float v = bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(a)[r * lda + j] << 16)
                                 : static_cast<const float*>(a)[r * lda + j];
            n += grid_int64((double)v, gexp);
          }
        }
      }
      for (int d = 32; d > 0; d >>= 1) {
        const uint32_t lo = __shfl_xor((uint32_t)(uint64_t)n, d, 64);
        const uint32_t hi = __shfl_xor((uint32_t)((uint64_t)n >> 32), d, 64);
        n += (int64_t)(((uint64_t)hi << 32) | lo);
      }
      return grid_int64_to_double(n, gexp);
    }
  }
  uint32_t acc[kWideWords];
#pragma unroll
  for (int i = 0; i < kWideWords; ++i) acc[i] = 0u;
  for (int64_t c = c0 + lane; c < c1; c += 64) {
    const int64_t r0 = seg_r0 + (c - c0) * ch;
    const int64_t r1 = r0 + ch < seg_r1 ? r0 + ch : seg_r1;
    const int64_t o = c * cols + j;
    const double am = __builtin_fmax(__builtin_fabs((double)pmax[o]), __builtin_fabs((double)pmin[o]));
    if (sum_certified((double)(r1 - r0), am, pmnz[o], bf16)) {
      wide_add_f64(acc, psum[o]);
    } else {
      for (int64_t r = r0; r < r1; ++r) {
        const float v = bf16 ? __uint_as_float((uint32_t)static_cast<const uint16_t*>(a)[r * lda + j] << 16)
                             : static_cast<const float*>(a)[r * lda + j];
        wide_add_f32(acc, v);
      }
    }
  }
  // butterfly over the wavefront: every lane ends with the total
  for (int d = 32; d > 0; d >>= 1) {
    uint32_t other[kWideWords];
#pragma unroll
    for (int i = 0; i < kWideWords; ++i) other[i] = __shfl_xor(acc[i], d, 64);
    wide_add(acc, other);
  }
  return wide_to_double(acc);
}

// ---------------------------------------------------------------------------
// finalize (split): block = kFinCols (16) columns x 16 chunk lanes, per
// segment, over the partials of chunks of `ch` rows (the statistics pass's
// kStatsRows, or the row tiles of a GEMM that wrote the statistics of its
// output); each lane keeps all its partial loads in flight.  The fp64 partial
// sums are exact, so the order of the reduction is free.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_finalize(const void* a, bool a_bf16, int64_t lda,
                                                  int64_t rows, int64_t cols, const int64_t* offs,
                                                  int nseg, const double* __restrict__ psum,
                                                  const float* __restrict__ pmax,
                                                  const float* __restrict__ pmin,
                                                  const float* __restrict__ pmnz,
                                                  float* __restrict__ mu,
                                                  float* __restrict__ mean_out,
                                                  float* __restrict__ tmax_r,
                                                  float* __restrict__ tmax_mu,
                                                  const double* __restrict__ psq,
                                                  double* __restrict__ tssq,
                                                  double* __restrict__ tmu2, int64_t ch) {
  constexpr int NC = (int)kFinCols, NQ = 256 / NC;
  const int seg = blockIdx.y;
  const SegRange sr = describe_segment(offs, nseg, rows, ch, seg);
  const int jl = threadIdx.x % NC, q = threadIdx.x / NC;
  const int64_t j = (int64_t)blockIdx.x * NC + jl;
  double s = 0.0, s2 = 0.0;
  float m1 = -__builtin_inff(), m0 = __builtin_inff(), mz = __builtin_inff();
  if (j < cols && sr.c1 > sr.c0) {
    constexpr int U = 8;   // up to 128 chunks in one round of loads
    const int64_t clast = sr.c1 - 1;
    for (int64_t ck = sr.c0 + q; ck < sr.c1; ck += NQ * U) {
      double ps[U], pq[U];
      float px[U], pn[U], pz[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int64_t cc = ck + NQ * u < clast ? ck + NQ * u : clast;
        ps[u] = psum[cc * cols + j];
        pq[u] = psq ? psq[cc * cols + j] : 0.0;
        px[u] = pmax[cc * cols + j];
        pn[u] = pmin[cc * cols + j];
        pz[u] = pmnz[cc * cols + j];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const bool ok = ck + NQ * u <= clast;
        s += ok ? ps[u] : 0.0;
        s2 += ok ? pq[u] : 0.0;
        m1 = __builtin_fmaxf(m1, px[u]);   // a clamped chunk repeats a real one
        m0 = __builtin_fminf(m0, pn[u]);
        mz = __builtin_fminf(mz, pz[u]);
      }
    }
  }
  __shared__ double ls[NQ][NC], lq[NQ][NC];
  __shared__ float lx[NQ][NC], ln[NQ][NC], lz[NQ][NC];
  __shared__ uint32_t need_mask;   // bit c: column c of the tile failed the certificate
  __shared__ double exact_s[NC];
  ls[q][jl] = s;
  lq[q][jl] = s2;
  lx[q][jl] = m1;
  ln[q][jl] = m0;
  lz[q][jl] = mz;
  __syncthreads();
  float rmax = 0.0f, amu = 0.0f;
  double t = 0.0, t2 = 0.0, mu2 = 0.0;
  float x1 = -__builtin_inff(), x0 = __builtin_inff();
  const int64_t l = sr.seg_r1 - sr.seg_r0;
  bool fail = false;
  if (q == 0) {
    float z = __builtin_inff();
#pragma unroll
    for (int p = 0; p < NQ; ++p) {
      t += ls[p][jl];
      t2 += lq[p][jl];
      x1 = __builtin_fmaxf(x1, lx[p][jl]);
      x0 = __builtin_fminf(x0, ln[p][jl]);
      z = __builtin_fminf(z, lz[p][jl]);
    }
    // Certificate: every value of the column is a multiple of g = 2^(ez-1-P)
    // (ez: binary exponent of the smallest nonzero |a|; P = 7 for bf16 input,
    // 23 for fp32), and every partial sum is at most l * max|a|.  When that
    // bound is <= 2^52 g, every fp64 addition above was exact, in any order.
    if (j < cols && l > 0) {
      const double amx = __builtin_fmax(__builtin_fabs((double)x1), __builtin_fabs((double)x0));
      fail = !sum_certified((double)l, amx, z, a_bf16);
    }
  }
  // the q == 0 lanes are lanes 0 .. NC-1 of wave 0
  if (threadIdx.x < 64) {
    const uint64_t bal = __ballot(fail);
    if (threadIdx.x == 0) need_mask = (uint32_t)bal;
  }
  __syncthreads();
  const uint32_t mask = need_mask;   // uniform
  // the failing columns' exact sums, the k-th of them by wave k mod 4
  {
    const int wv = threadIdx.x >> 6;
    int k = 0;
    for (uint32_t mrest = mask; mrest != 0; mrest &= mrest - 1, ++k) {
      if ((k & 3) != wv) continue;   // wave-uniform
      const int cidx = __builtin_ctz(mrest);
      const double v = exact_column_sum(a, a_bf16, lda, cols, sr.seg_r0, sr.seg_r1, sr.c0, sr.c1,
                                        ch, (int64_t)blockIdx.x * NC + cidx, psum, pmax, pmin,
                                        pmnz);
      if ((threadIdx.x & 63) == 0) exact_s[cidx] = v;
    }
  }
  if (mask) __syncthreads();
  if (q == 0 && j < cols) {
    if ((mask >> jl) & 1u) t = exact_s[jl];
    float m = 0.0f;
    if (l > 0) {
      const double md = t / (double)l;
      m = (float)md;
      rmax = __builtin_fmaxf(x1 - m, m - x0);
      mu2 = md * md;
    }
    mu[(int64_t)seg * cols + j] = m;
    if (mean_out) mean_out[(int64_t)seg * cols + j] = m;
    amu = __builtin_fabsf(m);
  }
  // the column maxima of this tile: lanes 0 .. NC-1 of wave 0 hold them
  if (threadIdx.x < 64) {
    for (int d = NC / 2; d > 0; d >>= 1) {
      rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, d, 64));
      amu = __builtin_fmaxf(amu, __shfl_xor(amu, d, 64));
    }
    if (threadIdx.x == 0) {
      tmax_r[(int64_t)seg * gridDim.x + blockIdx.x] = rmax;
      tmax_mu[(int64_t)seg * gridDim.x + blockIdx.x] = amu;
    }
    if (psq) {
      // the tile's sums for the mean-energy ratio (columns past the end
      // hold zeros), in a fixed butterfly order
      for (int d = NC / 2; d > 0; d >>= 1) {
        t2 += __shfl_xor(t2, d, 64);
        mu2 += __shfl_xor(mu2, d, 64);
      }
      if (threadIdx.x == 0) {
        tssq[(int64_t)seg * gridDim.x + blockIdx.x] = t2;
        tmu2[(int64_t)seg * gridDim.x + blockIdx.x] = mu2;
      }
    }
  }
}

// ---------------------------------------------------------------------------
// finalize for many short segments (grouped experts, a few chunks each):
// wave w of the block takes segment 4 blockIdx.y + w and lane l column
// 64 blockIdx.x + l, so each lane sums its column over its segment's chunks
// by itself (kSegFinU chunks' partials in flight) and only the tile maxima
// need the wave.  Same outputs as k_finalize, per 64-column tile.
// ---------------------------------------------------------------------------
constexpr int kSegFinU = 16;
__global__ __launch_bounds__(256) void k_finalize_seg(const void* a, bool a_bf16, int64_t lda,
                                                      int64_t rows, int64_t cols,
                                                      const int64_t* offs, int nseg,
                                                      const double* __restrict__ psum,
                                                      const float* __restrict__ pmax,
                                                      const float* __restrict__ pmin,
                                                      const float* __restrict__ pmnz,
                                                      float* __restrict__ mu,
                                                      float* __restrict__ mean_out,
                                                      float* __restrict__ tmax_r,
                                                      float* __restrict__ tmax_mu,
                                                      const double* __restrict__ psq,
                                                      double* __restrict__ tssq,
                                                      double* __restrict__ tmu2, int64_t ch) {
  __shared__ SegRange srs[4];
  __shared__ uint64_t fail_mask[4];
  __shared__ double exact_s[4][64];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int seg_w = (int)blockIdx.y * 4 + wave;
  if (seg_w < nseg) {   // wave-uniform
    seg_scan(offs, nseg, rows, ch, seg_w, 1, &srs[wave]);
  } else if (lane == 0) {
    SegRange none;
    none.seg = -1;
    none.r0 = none.r1 = none.seg_r0 = none.seg_r1 = 0;
    none.c0 = none.c1 = 0;
    srs[wave] = none;
  }
  __syncthreads();
  const SegRange sr = srs[wave];
  const int64_t j = (int64_t)blockIdx.x * 64 + lane;
  const bool live = sr.seg >= 0 && j < cols;
  double t = 0.0, t2 = 0.0;
  float x1 = -__builtin_inff(), x0 = __builtin_inff(), z = __builtin_inff();
  if (live && sr.c1 > sr.c0) {
    const int64_t clast = sr.c1 - 1;
    for (int64_t c = sr.c0; c < sr.c1; c += kSegFinU) {
      double ps[kSegFinU], pq[kSegFinU];
      float px[kSegFinU], pn[kSegFinU], pz[kSegFinU];
#pragma unroll
      for (int u = 0; u < kSegFinU; ++u) {
        const int64_t cc = c + u < clast ? c + u : clast;
        ps[u] = psum[cc * cols + j];
        pq[u] = psq ? psq[cc * cols + j] : 0.0;
        px[u] = pmax[cc * cols + j];
        pn[u] = pmin[cc * cols + j];
        pz[u] = pmnz[cc * cols + j];
      }
#pragma unroll
      for (int u = 0; u < kSegFinU; ++u) {
        const bool ok = c + u <= clast;
        t += ok ? ps[u] : 0.0;
        t2 += ok ? pq[u] : 0.0;
        x1 = __builtin_fmaxf(x1, px[u]);   // a clamped chunk repeats a real one
        x0 = __builtin_fminf(x0, pn[u]);
        z = __builtin_fminf(z, pz[u]);
      }
    }
  }
  const int64_t l = sr.seg_r1 - sr.seg_r0;
  bool fail = false;
  if (live && l > 0) {
    // the certificate of k_finalize: every fp64 addition above was exact
    const double amx = __builtin_fmax(__builtin_fabs((double)x1), __builtin_fabs((double)x0));
    fail = !sum_certified((double)l, amx, z, a_bf16);
  }
  const uint64_t bal = __ballot(fail);
  if (lane == 0) fail_mask[wave] = bal;
  __syncthreads();
  // each wave its own segment's failing columns
  for (uint64_t mrest = fail_mask[wave]; mrest != 0; mrest &= mrest - 1) {   // wave-uniform
    const int cidx = __builtin_ctzll(mrest);
    const double v = exact_column_sum(a, a_bf16, lda, cols, sr.seg_r0, sr.seg_r1, sr.c0, sr.c1,
                                      ch, (int64_t)blockIdx.x * 64 + cidx, psum, pmax, pmin,
                                      pmnz);
    if (lane == 0) exact_s[wave][cidx] = v;
  }
  if ((fail_mask[0] | fail_mask[1] | fail_mask[2] | fail_mask[3]) != 0) __syncthreads();
  float rmax = 0.0f, amu = 0.0f;
  double mu2 = 0.0;
  if (live) {
    if (fail) t = exact_s[wave][lane];
    float m = 0.0f;
    if (l > 0) {
      const double md = t / (double)l;
      m = (float)md;
      rmax = __builtin_fmaxf(x1 - m, m - x0);
      mu2 = md * md;
    }
    mu[(int64_t)sr.seg * cols + j] = m;
    if (mean_out) mean_out[(int64_t)sr.seg * cols + j] = m;
    amu = __builtin_fabsf(m);
  }
  // the tile's maxima (and ratio sums) over the wave's 64 columns
  for (int d = 32; d > 0; d >>= 1) {
    rmax = __builtin_fmaxf(rmax, __shfl_xor(rmax, d, 64));
    amu = __builtin_fmaxf(amu, __shfl_xor(amu, d, 64));
  }
  if (sr.seg >= 0 && lane == 0) {
    tmax_r[(int64_t)sr.seg * gridDim.x + blockIdx.x] = rmax;
    tmax_mu[(int64_t)sr.seg * gridDim.x + blockIdx.x] = amu;
  }
  if (psq) {
    for (int d = 32; d > 0; d >>= 1) {
      t2 += __shfl_xor(t2, d, 64);
      mu2 += __shfl_xor(mu2, d, 64);
    }
    if (sr.seg >= 0 && lane == 0) {
      tssq[(int64_t)sr.seg * gridDim.x + blockIdx.x] = t2;
      tmu2[(int64_t)sr.seg * gridDim.x + blockIdx.x] = mu2;
    }
  }
}

// ---------------------------------------------------------------------------
// v_cvt_scalef32_sr_pk_fp4_f32 (scale 1) into byte P of acc, keeping its other
// bytes.  Written as an instruction with a read-write destination: the
// compiler's builtin for it does not keep the destination's other bytes.
// ---------------------------------------------------------------------------
typedef float f32x2v __attribute__((ext_vector_type(2)));
template <int P>
__device__ __forceinline__ void sr_fp4_byte(uint32_t& acc, f32x2v v, uint32_t seed) {
  if constexpr (P == 0)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0" : "+v"(acc) : "v"(v), "v"(seed));
  else if constexpr (P == 1)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,0]" : "+v"(acc) : "v"(v), "v"(seed));
  else if constexpr (P == 2)
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,0,1]" : "+v"(acc) : "v"(v), "v"(seed));
  else
    asm("v_cvt_scalef32_sr_pk_fp4_f32 %0, %1, %2, 1.0 op_sel:[0,0,1,1]" : "+v"(acc) : "v"(v), "v"(seed));
}

// ---------------------------------------------------------------------------
// encode 16 values held in registers with the block's e_b (RN or SR, draws
// idx0 .. idx0 + 15); 8 code bytes, element k in nibble k
// ---------------------------------------------------------------------------
template <bool SR>
__device__ __forceinline__ void encode_block16(const float* r, float e_b, uint64_t idx0,
                                               uint32_t k0, uint32_t k1, uint32_t stream,
                                               uint2& packed) {
  if (SR) {
    // gfx950's v_cvt_scalef32_sr_pk_fp4_f32 (scale 1) rounds element 0 up iff
    // floor(2^22 frac) + seed[31:10] >= 2^22 and element 1 with seed[30:9]
    // (frac: the fraction of the E2M1 step above the lower grid point).  With
    // the 16-bit draw u in the top bits of that window -- seed = u << 16 for
    // element 0, u << 15 for element 1 -- this is the exact SR rule: up iff
    // floor(2^22 frac) + 64 u >= 2^22.  One instruction per element (the two
    // elements' dither windows overlap): both conversions of a pair take the
    // pair, the one seeded for element 0 keeps the even element's nibble
    // (low), the one seeded for element 1 the odd element's (high); the other
    // nibble of each is masked off.
    const uint64_t g = idx0 >> 3;   // idx0 is a multiple of 16
    uint32_t even[2] = {0u, 0u}, odd[2] = {0u, 0u};
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const uint64_t gg = g + h;
      const u32x4 rr = philox10((uint32_t)gg, (uint32_t)(gg >> 32), stream, 0u, k0, k1);
      const uint32_t wd[4] = {rr.x, rr.y, rr.z, rr.w};
#define AVERIS_SR_PAIR(P)                                                        \
  {                                                                              \
    const f32x2v e = {r[8 * h + 2 * (P)] * e_b, r[8 * h + 2 * (P) + 1] * e_b};   \
    sr_fp4_byte<P>(even[h], e, wd[P] << 16);                                     \
    sr_fp4_byte<P>(odd[h], e, (wd[P] & 0xFFFF0000u) >> 1);                       \
  }
      AVERIS_SR_PAIR(0)
      AVERIS_SR_PAIR(1)
      AVERIS_SR_PAIR(2)
      AVERIS_SR_PAIR(3)
#undef AVERIS_SR_PAIR
    }
    packed.x = (even[0] & 0x0F0F0F0Fu) | (odd[0] & 0xF0F0F0F0u);
    packed.y = (even[1] & 0x0F0F0F0Fu) | (odd[1] & 0xF0F0F0F0u);
  } else {
    // RN: gfx950's v_cvt_scalef32_pk_fp4_f32 with scale 1 rounds to the
    // nearest E2M1 value, ties to the even code, saturates at 6 and keeps the
    // sign of zero, two elements per instruction
    float v[16];
#pragma unroll
    for (int k = 0; k < 16; ++k) v[k] = r[k] * e_b;
    uint32_t lo = 0, hi = 0;
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[0], v[1], 1.0f, 0);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[2], v[3], 1.0f, 1);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[4], v[5], 1.0f, 2);
    lo = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(lo, v[6], v[7], 1.0f, 3);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[8], v[9], 1.0f, 0);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[10], v[11], 1.0f, 1);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[12], v[13], 1.0f, 2);
    hi = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(hi, v[14], v[15], 1.0f, 3);
    packed.x = lo;
    packed.y = hi;
  }
}

// a value the optimizer cannot see through (kept in a register pair as is)
__device__ __forceinline__ uint64_t opaque_u64(uint64_t v) {
  asm volatile("" : "+v"(v));
  return v;
}

// quantize one 16-block held in registers: its scale from its own largest
// magnitude, then its codes
template <bool SR>
__device__ __forceinline__ void quant_block16_regs(const float* r, float s_enc, uint64_t idx0,
                                                   uint32_t k0, uint32_t k1, uint32_t stream,
                                                   uint2& packed, uint32_t& sc) {
  float amax_b = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(r[k]));
  float e_b;
  block_scale(amax_b, s_enc, sc, e_b);
  encode_block16<SR>(r, e_b, idx0, k0, k1, stream, packed);
}

// the same with the element factor from the workgroup's table of s_enc /
// decode(code) (fill_eb_table): the same bits without a division per block
template <bool SR>
__device__ __forceinline__ void quant_block16_tab(const float* r, float s_enc, const float* eb_tab,
                                                  uint64_t idx0, uint32_t k0, uint32_t k1,
                                                  uint32_t stream, uint8_t* codes, uint8_t* scale) {
  float amax_b = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) amax_b = __builtin_fmaxf(amax_b, __builtin_fabsf(r[k]));
  const uint32_t sc = block_scale_code(amax_b, s_enc);
  uint2 packed;
  encode_block16<SR>(r, eb_tab[sc], idx0, k0, k1, stream, packed);
  *reinterpret_cast<uint2*>(codes) = packed;
  *scale = (uint8_t)sc;
}

template <bool SR>
__device__ __forceinline__ void quant_block16(const float* r, float s_enc, uint64_t idx0,
                                              uint32_t k0, uint32_t k1, uint32_t stream,
                                              uint8_t* codes, uint8_t* scale) {
  uint2 packed;
  uint32_t sc;
  quant_block16_regs<SR>(r, s_enc, idx0, k0, k1, stream, packed, sc);
  *reinterpret_cast<uint2*>(codes) = packed;
  *scale = (uint8_t)sc;
}

// sum of n doubles in a fixed order (thread i takes i, i + 256, ...; then a
// fixed tree over the threads); thread 0 gets the total
__device__ __forceinline__ double block_sum_f64(const double* p, int64_t n) {
  __shared__ double red[256];
  double v = 0.0;
  for (int64_t i = threadIdx.x; i < n; i += 256) v += p[i];
  red[threadIdx.x] = v;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if ((int)threadIdx.x < st) red[threadIdx.x] += red[threadIdx.x + st];
    __syncthreads();
  }
  const double t = red[0];
  __syncthreads();
  return t;
}

// max over a segment's per-tile partial maxima (all threads get it)
__device__ __forceinline__ float reduce_partials(const float* p, int64_t n) {
  __shared__ float red[4];
  float m = 0.0f;
  for (int64_t i = threadIdx.x; i < n; i += 256) m = __builtin_fmaxf(m, p[i]);
  return block_max(m, red);
}

// The rank-one operands of a split as the quant kernel takes them: up to
// kMaxRank1 B operands, operand i's workgroups ending at gend[i]
struct Rank1Set {
  QOperand b[kMaxRank1];
  int64_t n[kMaxRank1];
  float* rho[kMaxRank1];
  int64_t gend[kMaxRank1];
  int count;
};

// ---------------------------------------------------------------------------
// quant: block = 64 column-blocks (1024 columns) x 4 row lanes over a chunk
// of kQuantRows rows; blockIdx.y >= nchunk_ub quantizes segment means.
// ---------------------------------------------------------------------------
template <typename T, bool SPLIT, bool SR>
__global__ __launch_bounds__(256) void k_quant(const T* __restrict__ a, int64_t rows, int64_t cols,
                                               int64_t lda, const int64_t* offs, int nseg,
                                               int64_t nchunk_ub, uint64_t seed, uint32_t stream,
                                               const float* __restrict__ mu,
                                               const float* __restrict__ tmax,  // per segment
                                               int64_t ntmax,
                                               const float* __restrict__ tmax_mu,
                                               int64_t ntmax_mu,
                                               uint8_t* __restrict__ codes,
                                               uint8_t* __restrict__ scales,
                                               float* __restrict__ tscale,
                                               uint8_t* __restrict__ mcodes,
                                               uint8_t* __restrict__ mscales,
                                               float* __restrict__ mtscale,
                                               const double* __restrict__ tssq,
                                               const double* __restrict__ tmu2,
                                               float* __restrict__ ratio,
                                               Rank1Set r1s, int64_t rho_rows, int r1_rows) {
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int64_t nb = cols >> 4;
  const int64_t b = (int64_t)blockIdx.x * 64 + tx;   // 16-block index within a row
  int64_t by = blockIdx.y;

  if (SPLIT && r1s.count > 0) {
    // leading rows of the grid: the rank-one rows of the GEMMs that take this
    // split, rho_i[s][j] = deq(Q4(mu_s)) . deq(B_i,s,j) for each B operand i
    // and segment s (B_i holds one n_i x cols matrix per segment).  Operand
    // i owns the workgroups r1s.gend[i-1] .. r1s.gend[i]-1, r1_rows (a multiple
    // of 16) rows of one segment's B_i each: a workgroup quantizes that
    // segment's mean as the mean block below does (same tensor scale, same
    // draws), dequantizes it to fp16 in LDS (exact), and each group of 16
    // lanes sums one row of B_i against it, 16 rows per pass.
    if (by < rho_rows) {
      extern __shared__ __attribute__((aligned(16))) _Float16 r1_mean[];   // [cols]
      const int64_t rbi = by * gridDim.x + blockIdx.x;
      int bi = 0;
      while (bi + 1 < r1s.count && rbi >= r1s.gend[bi]) ++bi;   // uniform
      if (rbi >= r1s.gend[bi]) return;                        // past the last operand's rows
      const QOperand B = r1s.b[bi];
      const int64_t bn = r1s.n[bi];
      float* __restrict__ rho = r1s.rho[bi];
      const int64_t groups = (bn + r1_rows - 1) / r1_rows;
      const int64_t rloc = rbi - (bi > 0 ? r1s.gend[bi - 1] : 0);
      const int rseg = (int)(rloc / groups);
      const float am = reduce_partials(tmax_mu + (int64_t)rseg * ntmax_mu, ntmax_mu);
      float s_enc, s_dec;
      tensor_scales(am, s_enc, s_dec);
      const float* mu_s = mu + (int64_t)rseg * cols;
      for (int64_t mb = threadIdx.x; mb < nb; mb += 256) {
        float r[16];
#pragma unroll
        for (int k = 0; k < 16; ++k) r[k] = mu_s[mb * 16 + k];
        uint2 packed;
        uint32_t sc;
        quant_block16_regs<SR>(r, s_enc, (uint64_t)rseg * (uint64_t)cols + (uint64_t)mb * 16, k0,
                               k1, 1u, packed, sc);
        const half2_t sv = scales2(sc);
        const half2_t s2 = {sv.x, sv.x};
        *reinterpret_cast<uint4*>(r1_mean + mb * 16) = deq8(packed.x, s2);
        *reinterpret_cast<uint4*>(r1_mean + mb * 16 + 8) = deq8(packed.y, s2);
      }
      __syncthreads();
      const int64_t rb = rloc - (int64_t)rseg * groups;   // r1_rows rows of the segment's B
      const int sub = threadIdx.x & 15;
      const float r_dec = s_dec * B.tscale[(offs ? 2 * rseg : 0) + 1];
      for (int64_t j = rb * r1_rows + (threadIdx.x >> 4); j < (rb + 1) * r1_rows; j += 16) {
        if (j - (threadIdx.x >> 4) >= bn) break;          // uniform: the pass starts past B
        const int64_t jj = j < bn ? j : bn - 1;            // every lane joins the butterfly
        const int64_t brow = (int64_t)rseg * bn + jj;
        const uint8_t* bc = B.codes + brow * (cols >> 1);
        const uint8_t* bs = B.scales + brow * nb;
        float acc = 0.0f;
        // four blocks per pass, their loads issued before any arithmetic;
        // blocks past the end are clamped to the last one and dropped
        constexpr int U = 4;
        for (int64_t b0 = sub; b0 < nb; b0 += 16 * U) {
          uint2 w[U];
          uint32_t sb[U];
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t blk = b0 + 16 * u < nb ? b0 + 16 * u : nb - 1;
            w[u] = *reinterpret_cast<const uint2*>(bc + 8 * blk);
            sb[u] = bs[blk];
          }
#pragma unroll
          for (int u = 0; u < U; ++u) {
            const int64_t blk = b0 + 16 * u < nb ? b0 + 16 * u : nb - 1;
            const half2_t sv = scales2(sb[u]);
            const half2_t s2 = {sv.x, sv.x};
            const uint4 d0 = deq8(w[u].x, s2), d1 = deq8(w[u].y, s2);
            const uint4 m0 = *reinterpret_cast<const uint4*>(r1_mean + blk * 16);
            const uint4 m1 = *reinterpret_cast<const uint4*>(r1_mean + blk * 16 + 8);
            // products of exact fp16 values (<= 6 significant bits each) are
            // exact; fp32 accumulation
            float p = 0.0f;
            p = __builtin_amdgcn_fdot2(h2(d0.x), h2(m0.x), p, false);
            p = __builtin_amdgcn_fdot2(h2(d0.y), h2(m0.y), p, false);
            p = __builtin_amdgcn_fdot2(h2(d0.z), h2(m0.z), p, false);
            p = __builtin_amdgcn_fdot2(h2(d0.w), h2(m0.w), p, false);
            p = __builtin_amdgcn_fdot2(h2(d1.x), h2(m1.x), p, false);
            p = __builtin_amdgcn_fdot2(h2(d1.y), h2(m1.y), p, false);
            p = __builtin_amdgcn_fdot2(h2(d1.z), h2(m1.z), p, false);
            p = __builtin_amdgcn_fdot2(h2(d1.w), h2(m1.w), p, false);
            acc += b0 + 16 * u < nb ? p : 0.0f;
          }
        }
        for (int d = 8; d > 0; d >>= 1) acc += __shfl_xor(acc, d, 16);
        if (sub == 0 && j < bn) rho[(int64_t)rseg * bn + j] = acc * r_dec;
      }
      return;
    }
    by -= rho_rows;
  }

  if (SPLIT && by >= nchunk_ub) {
    // mean vector of one segment: 1 x cols, SR stream 1, index seg*cols + col
    const int seg = (int)(by - nchunk_ub);
    const float am = reduce_partials(tmax_mu + (int64_t)seg * ntmax_mu, ntmax_mu);
    float s_enc, s_dec;
    tensor_scales(am, s_enc, s_dec);
    if (blockIdx.x == 0) {
      // this segment's residual tensor scale too (written even when the
      // segment is empty and no chunk exists)
      const float amr = reduce_partials(tmax + (int64_t)seg * ntmax, ntmax);
      float r_enc, r_dec;
      tensor_scales(amr, r_enc, r_dec);
      if (threadIdx.x == 0) {
        mtscale[2 * seg] = s_enc;
        mtscale[2 * seg + 1] = s_dec;
        tscale[2 * seg] = r_enc;
        tscale[2 * seg + 1] = r_dec;
      }
      if (ratio) {
        // mean-energy ratio R = sqrt(sum mu_j^2 / (sum a_ij^2 / l)) of the
        // segment, from the per-tile sums of the finalize pass
        // (every thread takes part: both helpers synchronize the block)
        const double q2 = block_sum_f64(tssq + (int64_t)seg * ntmax_mu, ntmax_mu);
        const double m2 = block_sum_f64(tmu2 + (int64_t)seg * ntmax_mu, ntmax_mu);
        const SegRange ss = describe_segment(offs, nseg, rows, kStatsRows, seg);
        if (threadIdx.x == 0) {
          const int64_t l = ss.seg_r1 - ss.seg_r0;
          ratio[seg] = (l > 0 && q2 > 0.0) ? (float)__builtin_sqrt(m2 / (q2 / (double)l)) : 0.0f;
        }
      }
    }
    if (ty == 0 && b < nb) {
      float r[16];
      const float* m = mu + (int64_t)seg * cols + b * 16;
#pragma unroll
      for (int k = 0; k < 16; ++k) r[k] = m[k];
      const uint64_t idx0 = (uint64_t)seg * (uint64_t)cols + (uint64_t)b * 16;
      quant_block16<SR>(r, s_enc, idx0, k0, k1, 1u, mcodes + (int64_t)seg * (cols >> 1) + b * 8,
                        mscales + (int64_t)seg * nb + b);
    }
    return;
  }

  if (!SPLIT && by >= nchunk_ub) {
    // plain: one block per segment publishes the segment's tensor scale
    // (also for empty segments, which have no chunk)
    if (blockIdx.x != 0) return;
    const int seg = (int)(by - nchunk_ub);
    const SegRange ss = describe_segment(offs, nseg, rows, kStatsRows, seg);
    const float am = reduce_partials(tmax + ss.c0 * ntmax, (ss.c1 - ss.c0) * ntmax);
    float s_enc, s_dec;
    tensor_scales(am, s_enc, s_dec);
    if (threadIdx.x == 0) {
      tscale[2 * seg] = s_enc;
      tscale[2 * seg + 1] = s_dec;
    }
    return;
  }
  const SegRange sr = locate_chunk(offs, nseg, rows, kQuantRows, by);
  if (sr.seg < 0) return;
  float am;
  if (SPLIT) {
    am = reduce_partials(tmax + (int64_t)sr.seg * ntmax, ntmax);
  } else {
    // plain: the segment's stats partials are its stats chunks x column tiles
    const SegRange ss = describe_segment(offs, nseg, rows, kStatsRows, sr.seg);
    am = reduce_partials(tmax + ss.c0 * ntmax, (ss.c1 - ss.c0) * ntmax);
  }
  float s_enc, s_dec;
  tensor_scales(am, s_enc, s_dec);
  __shared__ float eb_tab[128];
  fill_eb_table(s_enc, eb_tab);
  __syncthreads();
  if (b >= nb) return;
  float m[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) m[k] = 0.0f;
  if (SPLIT) {
    const float* mp = mu + (int64_t)sr.seg * cols + b * 16;
#pragma unroll
    for (int k = 0; k < 16; ++k) m[k] = mp[k];
  }
  // every row of the chunk: loads first (rows past the end clamped), then
  // quantize; the row is uniform per wavefront, so the store guard is too.
  // Row u of the thread is row0 + 4 u: its addresses and element index are
  // the first row's plus a uniform stride (no 64-bit multiply per row).
  constexpr int R = (int)(kQuantRows / 4);
  const int64_t rlast = sr.r1 - 1;
  const int64_t row0 = sr.r0 + ty;
  const T* a_row0 = a + row0 * lda + b * 16;
  const T* a_last = a + rlast * lda + b * 16;
  float v[R][16];
#pragma unroll
  for (int u = 0; u < R; ++u) {
    const T* p = row0 + 4 * u <= rlast ? a_row0 + 4 * u * lda : a_last;
    Load8<T>::run(p, v[u]);
    Load8<T>::run(p + 8, v[u] + 8);
  }
  // (kept opaque to the optimizer, which would otherwise fold the strides
  // back into one 64-bit multiply per row)
  const uint64_t idx_row0 = opaque_u64((uint64_t)row0 * (uint64_t)cols + (uint64_t)b * 16);
  uint8_t* c_row0 = codes + (int64_t)opaque_u64((uint64_t)(row0 * (cols >> 1) + b * 8));
  uint8_t* s_row0 = scales + (int64_t)opaque_u64((uint64_t)(row0 * nb + b));
#pragma unroll
  for (int u = 0; u < R; ++u) {
    if (row0 + 4 * u > rlast) break;
    if (SPLIT) {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[u][k] = v[u][k] - m[k];
    }
    quant_block16_tab<SR>(v[u], s_enc, eb_tab, idx_row0 + (uint64_t)(4 * u) * (uint64_t)cols, k0,
                          k1, stream, c_row0 + 4 * u * (cols >> 1), s_row0 + 4 * u * nb);
  }
}

// ---------------------------------------------------------------------------
// plain quant of any-orientation, batched tensors (weights)
//   logical T_b[r][c] = a[b*bstride + r*lda + c]     (transpose = 0)
//                     = a[b*bstride + c*lda + r]     (transpose = 1)
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ float load1(const T* p);
template <>
__device__ __forceinline__ float load1<uint16_t>(const uint16_t* p) {
  return __uint_as_float((uint32_t)(*p) << 16);
}
template <>
__device__ __forceinline__ float load1<float>(const float* p) { return *p; }

// amax over the stored matrix of each batch entry (stored rows x stored cols)
template <typename T>
__global__ __launch_bounds__(256) void k_amax_batched(const T* __restrict__ a, int64_t srows,
                                                      int64_t scols, int64_t lda, int64_t bstride,
                                                      float* __restrict__ part) {
  const T* base = a + (int64_t)blockIdx.y * bstride;
  const int64_t n = srows * scols;
  float m = 0.0f;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / scols, c = i - r * scols;
    m = __builtin_fmaxf(m, __builtin_fabsf(load1<T>(base + r * lda + c)));
  }
  __shared__ float red[4];
  m = block_max(m, red);
  if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// thread per (logical row r, 16-block cb); blockIdx.z = batch entry
template <typename T, bool SR>
__global__ __launch_bounds__(256) void k_quant_batched(const T* __restrict__ a, int64_t rows,
                                                       int64_t cols, int64_t lda, int64_t bstride,
                                                       int transpose, uint64_t seed,
                                                       uint32_t stream,
                                                       const float* __restrict__ part,
                                                       int64_t npart, uint8_t* __restrict__ codes,
                                                       uint8_t* __restrict__ scales,
                                                       float* __restrict__ tscale) {
  const int bt = blockIdx.z;
  const float am = reduce_partials(part + (int64_t)bt * npart, npart);
  float s_enc, s_dec;
  tensor_scales(am, s_enc, s_dec);
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) {
    tscale[2 * bt] = s_enc;
    tscale[2 * bt + 1] = s_dec;
  }
  const int64_t r = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t cb = blockIdx.y;
  if (r >= rows) return;
  const T* base = a + (int64_t)bt * bstride;
  float v[16];
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const int64_t c = cb * 16 + k;
    v[k] = transpose ? load1<T>(base + c * lda + r) : load1<T>(base + r * lda + c);
  }
  const int64_t grow = (int64_t)bt * rows + r;
  const uint64_t idx0 = (uint64_t)grow * (uint64_t)cols + (uint64_t)cb * 16;
  quant_block16<SR>(v, s_enc, idx0, (uint32_t)seed, (uint32_t)(seed >> 32), stream,
                    codes + grow * (cols >> 1) + cb * 8, scales + grow * (cols >> 4) + cb);
}

// ---------------------------------------------------------------------------
// both orientations of a weight in one pass (Lighthouse §2.2: Q4(W^T) for the
// forward product, Q4(W) for dgrad; one tensor scale, max |W|, for both)
// ---------------------------------------------------------------------------

// max |a| of each stored rows x cols matrix, 16-byte loads; workgroup x of
// matrix y covers 16-byte chunks [x*per, (x+1)*per) of the row-major order
// a thread's max |a| over the 16-byte chunks q0 + threadIdx.x, + 256, ... < q1
// of one stored rows x cols matrix (chunk q: row q / (cols / VE))
template <typename T>
__device__ __forceinline__ float amax_chunks(const T* base, int64_t cols, int64_t lda, int64_t q0,
                                             int64_t q1) {
  constexpr int VE = 16 / (int)sizeof(T);   // elements per 16-byte chunk
  constexpr int U = 4;
  const int64_t cpr = cols / VE;
  float m = 0.0f;
  for (int64_t q = q0 + threadIdx.x; q < q1; q += 256 * U) {
    uint4 w[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t qq = q + 256 * u < q1 ? q + 256 * u : q;   // repeat a real chunk
      const int64_t r = qq / cpr;
      w[u] = *reinterpret_cast<const uint4*>(base + r * lda + (qq - r * cpr) * VE);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t x[4] = {w[u].x, w[u].y, w[u].z, w[u].w};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (sizeof(T) == 2) {
          m = __builtin_fmaxf(m, __builtin_fabsf(bf16_lo(x[i])));
          m = __builtin_fmaxf(m, __builtin_fabsf(bf16_hi(x[i])));
        } else {
          m = __builtin_fmaxf(m, __builtin_fabsf(__uint_as_float(x[i])));
        }
      }
    }
  }
  return m;
}

template <typename T>
__global__ __launch_bounds__(256) void k_amax_vec(const T* __restrict__ a, int64_t rows,
                                                  int64_t cols, int64_t lda, int64_t bstride,
                                                  int64_t per, float* __restrict__ part) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int64_t total = rows * (cols / VE);
  const int64_t q0 = (int64_t)blockIdx.x * per;
  const int64_t q1 = q0 + per < total ? q0 + per : total;
  float m = amax_chunks<T>(a + (int64_t)blockIdx.y * bstride, cols, lda, q0, q1);
  __shared__ float red[4];
  m = block_max(m, red);
  if (threadIdx.x == 0) part[(int64_t)blockIdx.y * gridDim.x + blockIdx.x] = m;
}

// one 64 x 64 tile of W_b per workgroup, staged in LDS as fp32; each thread
// quantizes one 16-block along a row (-> out) and one along a column (-> out_t)
constexpr int kPairTile = 64;
constexpr int kPairLd = kPairTile + 4;   // padded LDS row (floats), 16-byte aligned

// the 64 x 64 tile at (r0, c0) of the stored rows x cols matrix W_b at base:
// global rows of out and out_t from matrix index bt; the tensor scale from
// W_b's npart amax partials at part (written by the tile at (0, 0)); every
// launch caps npart at kAmaxBlocks, four partials a thread at most
template <typename T, bool SR>
__device__ __forceinline__ void pair_tile(const T* __restrict__ base, int64_t rows, int64_t cols,
                                          int64_t lda, int bt, int64_t r0, int64_t c0,
                                          uint64_t seed, uint32_t stream,
                                          const float* __restrict__ part, int64_t npart,
                                          const QuantOut& out, const QuantOut& out_t) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NCH = kPairTile / VE;              // 16-byte chunks per tile row
  constexpr int PER = kPairTile * NCH / 256;       // chunks per thread
  static_assert(kAmaxBlocks <= 4 * 256, "amax partials: four loads a thread");
  __shared__ float tile[kPairTile][kPairLd];
  __shared__ float red[4];
  const int tid = threadIdx.x;
  uint4 wv[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + 256 * i;
    const int lr = idx / NCH, ch = idx % NCH;
    const int64_t r = r0 + lr, c = c0 + (int64_t)ch * VE;
    // (outside the matrix: a clamped load, its value replaced by zeros, so
    // that no branch stands between these loads and the partials' below)
    const bool in = r < rows && c < cols;
    const int64_t rc = r < rows ? r : rows - 1, cc = c < cols ? c : cols - VE;
    const uint4 w = *reinterpret_cast<const uint4*>(base + rc * lda + cc);
    wv[i] = in ? w : uint4{0u, 0u, 0u, 0u};
  }
  // the thread's share of the tensor's amax partials, loaded while the tile
  // is in flight; an index past the last partial (npart >= 1) reads the last
  // one again, which leaves the maximum unchanged and needs no branch
  float pq[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int64_t j = tid + 256 * u;
    pq[u] = part[j < npart ? j : npart - 1];
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + 256 * i;
    const int lr = idx / NCH, ch = idx % NCH;
    const uint4 w = wv[i];
    float* dst = &tile[lr][ch * VE];
    if (sizeof(T) == 2) {
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = bf16_lo(x[e]);
        dst[2 * e + 1] = bf16_hi(x[e]);
      }
    } else {
      dst[0] = __uint_as_float(w.x);
      dst[1] = __uint_as_float(w.y);
      dst[2] = __uint_as_float(w.z);
      dst[3] = __uint_as_float(w.w);
    }
  }
  // the tensor scale (block_max synchronizes the block, which also
  // publishes the tile)
  const float pm = __builtin_fmaxf(__builtin_fmaxf(pq[0], pq[1]), __builtin_fmaxf(pq[2], pq[3]));
  const float am = block_max(pm, red);
  float s_enc, s_dec;
  tensor_scales(am, s_enc, s_dec);
  if (r0 == 0 && c0 == 0 && tid == 0) {
    out.tscale[2 * bt] = s_enc;
    out.tscale[2 * bt + 1] = s_dec;
    out_t.tscale[2 * bt] = s_enc;
    out_t.tscale[2 * bt + 1] = s_dec;
  }
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int l = tid >> 2, q = tid & 3;
  float v[16];
  // a 16-block along row r0 + l: out row b*rows + r, columns c0 + 16q ..
  {
    const int64_t r = r0 + l, c = c0 + 16 * q;
    if (r < rows && c < cols) {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = tile[l][16 * q + k];
      const int64_t grow = (int64_t)bt * rows + r;
      quant_block16<SR>(v, s_enc, (uint64_t)grow * (uint64_t)cols + (uint64_t)c, k0, k1, stream,
                        out.codes + grow * (cols >> 1) + (c >> 1),
                        out.scales + grow * (cols >> 4) + (c >> 4));
    }
  }
  // a 16-block along column c0 + l: out_t row b*cols + c, columns r0 + 16q ..
  {
    const int64_t c = c0 + l, r = r0 + 16 * q;
    if (c < cols && r < rows) {
#pragma unroll
      for (int k = 0; k < 16; ++k) v[k] = tile[16 * q + k][l];
      const int64_t grow = (int64_t)bt * cols + c;
      quant_block16<SR>(v, s_enc, (uint64_t)grow * (uint64_t)rows + (uint64_t)r, k0, k1, stream,
                        out_t.codes + grow * (rows >> 1) + (r >> 1),
                        out_t.scales + grow * (rows >> 4) + (r >> 4));
    }
  }
}

template <typename T, bool SR>
__global__ __launch_bounds__(256) void k_pair(const T* __restrict__ a, int64_t rows, int64_t cols,
                                              int64_t lda, int64_t bstride, uint64_t seed,
                                              uint32_t stream, const float* __restrict__ part,
                                              int64_t npart, QuantOut out, QuantOut out_t) {
  const int bt = blockIdx.z;
  pair_tile<T, SR>(a + (int64_t)bt * bstride, rows, cols, lda, bt,
                   (int64_t)blockIdx.y * kPairTile, (int64_t)blockIdx.x * kPairTile, seed, stream,
                   part + (int64_t)bt * npart, npart, out, out_t);
}

// ---------------------------------------------------------------------------
// Both copies of several weights of different shapes in two launches, one
// grid over all of them for each pass, weight i owning a contiguous range of
// the workgroups (the ranges' ends in the argument block; each workgroup
// finds its weight by a uniform scan).  Per weight the same partials (a
// partition of the same maximum) and the same tile code as k_amax_vec and
// k_pair, so the bits are those of the single-weight launches.
// ---------------------------------------------------------------------------
struct PairMultiArgs {
  WeightPair w[kMaxWeights];
  int64_t per[kMaxWeights];        // amax pass: 16-byte chunks per workgroup
  int64_t nblk[kMaxWeights];       // amax pass: workgroups (= partials)
  int64_t amax_end[kMaxWeights];   // amax pass: workgroups through weight i
  int64_t tiles_x[kMaxWeights];    // pair pass: 64 x 64 tiles across the columns
  int64_t tile_end[kMaxWeights];   // pair pass: tiles through weight i
  int n;
};

__device__ __forceinline__ int find_weight(const int64_t* end, int n, int64_t bid) {
  int i = 0;
  while (i + 1 < n && bid >= end[i]) ++i;
  return i;
}

template <typename T>
__global__ __launch_bounds__(256) void k_amax_multi(PairMultiArgs args, float* __restrict__ part) {
  constexpr int VE = 16 / (int)sizeof(T);
  const int64_t bid = blockIdx.x;
  const int i = find_weight(args.amax_end, args.n, bid);
  const WeightPair& w = args.w[i];
  const int64_t blk = bid - (i > 0 ? args.amax_end[i - 1] : 0);
  const int64_t total = w.rows * (w.cols / VE);
  const int64_t q0 = blk * args.per[i];
  const int64_t q1 = q0 + args.per[i] < total ? q0 + args.per[i] : total;
  float m = amax_chunks<T>(static_cast<const T*>(w.a), w.cols, w.lda, q0, q1);
  __shared__ float red[4];
  m = block_max(m, red);
  if (threadIdx.x == 0) part[(int64_t)i * kAmaxBlocks + blk] = m;
}

template <typename T, bool SR>
__global__ __launch_bounds__(256) void k_pair_multi(PairMultiArgs args, uint32_t stream,
                                                    const float* __restrict__ part) {
  const int64_t bid = blockIdx.x;
  const int i = find_weight(args.tile_end, args.n, bid);
  const WeightPair& w = args.w[i];
  const int64_t t = bid - (i > 0 ? args.tile_end[i - 1] : 0);
  const int64_t ty = t / args.tiles_x[i], tx = t - ty * args.tiles_x[i];
  pair_tile<T, SR>(static_cast<const T*>(w.a), w.rows, w.cols, w.lda, 0, ty * kPairTile,
                   tx * kPairTile, w.seed, stream, part + (int64_t)i * kAmaxBlocks, args.nblk[i],
                   w.out, w.out_t);
}

// ---------------------------------------------------------------------------
// shared 16 x 16-tile quantization of a weight (Lighthouse §2.2 writes the
// dgrad operand as the transpose of the forward one): one E4M3 scale per
// 16 x 16 tile of W_b from the tile's largest magnitude, the codes encoded
// once (SR index: global row b*rows + r times cols plus the column) and
// written in both layouts: out = W_b (rows x cols, 16-runs along cols) and
// out_t = W_b^T (cols x rows, 16-runs along rows), each run with its tile's
// scale.  A 64 x 64 tile of W_b per workgroup, staged in LDS as fp32 as in
// k_pair; thread (t, u) = (tid >> 4, tid & 15) takes row u of 16 x 16 tile t
// (the tile's 16 runs sit in 16 neighbouring lanes, which form its maximum
// with four butterfly steps) and, after the codes pass through LDS, column u
// of the same tile for out_t.
// ---------------------------------------------------------------------------
template <typename T, bool SR>
__global__ __launch_bounds__(256) void k_pair2d(const T* __restrict__ a, int64_t rows,
                                                int64_t cols, int64_t lda, int64_t bstride,
                                                uint64_t seed, uint32_t stream,
                                                const float* __restrict__ part, int64_t npart,
                                                QuantOut out, QuantOut out_t) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NCH = kPairTile / VE;              // 16-byte chunks per tile row
  constexpr int PER = kPairTile * NCH / 256;       // chunks per thread
  static_assert(kAmaxBlocks <= 4 * 256, "amax partials: four loads a thread");
  __shared__ float tile[kPairTile][kPairLd];
  // codes of the tile transposed, one byte each: ct[column][row]
  __shared__ __attribute__((aligned(16))) uint8_t ct[kPairTile][kPairTile + 16];
  const int bt = blockIdx.z;
  const int64_t r0 = (int64_t)blockIdx.y * kPairTile, c0 = (int64_t)blockIdx.x * kPairTile;
  const T* base = a + (int64_t)bt * bstride;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + 256 * i;
    const int lr = idx / NCH, ch = idx % NCH;
    const int64_t r = r0 + lr, c = c0 + (int64_t)ch * VE;
    uint4 w = {0u, 0u, 0u, 0u};
    if (r < rows && c < cols) w = *reinterpret_cast<const uint4*>(base + r * lda + c);
    float* dst = &tile[lr][ch * VE];
    if (sizeof(T) == 2) {
      const uint32_t x[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        dst[2 * e] = bf16_lo(x[e]);
        dst[2 * e + 1] = bf16_hi(x[e]);
      }
    } else {
      dst[0] = __uint_as_float(w.x);
      dst[1] = __uint_as_float(w.y);
      dst[2] = __uint_as_float(w.z);
      dst[3] = __uint_as_float(w.w);
    }
  }
  // the tensor scale (reduce_partials synchronizes the block, which also
  // publishes the tile)
  const float am = reduce_partials(part + (int64_t)bt * npart, npart);
  float s_enc, s_dec;
  tensor_scales(am, s_enc, s_dec);
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    out.tscale[2 * bt] = s_enc;
    out.tscale[2 * bt + 1] = s_dec;
    out_t.tscale[2 * bt] = s_enc;
    out_t.tscale[2 * bt + 1] = s_dec;
  }
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int t16 = tid >> 4, u = tid & 15;
  const int lr0 = 16 * (t16 >> 2), lc0 = 16 * (t16 & 3);   // the 16 x 16 tile's corner
  // rows % 16 == cols % 16 == 0: a 16 x 16 tile lies wholly inside or outside
  const bool inside = r0 + lr0 < rows && c0 + lc0 < cols;
  float v[16];
  float m = 0.0f;
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    v[k] = tile[lr0 + u][lc0 + k];
    m = __builtin_fmaxf(m, __builtin_fabsf(v[k]));
  }
  // the tile's largest magnitude: its 16 rows are lanes 16 g .. 16 g + 15
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
  uint32_t sc;
  float e_b;
  block_scale(m, s_enc, sc, e_b);
  const int64_t grow = (int64_t)bt * rows + r0 + lr0 + u;
  const int64_t c = c0 + lc0;
  uint2 packed;
  encode_block16<SR>(v, e_b, (uint64_t)grow * (uint64_t)cols + (uint64_t)c, k0, k1, stream, packed);
  if (inside) {
    *reinterpret_cast<uint2*>(out.codes + grow * (cols >> 1) + (c >> 1)) = packed;
    out.scales[grow * (cols >> 4) + (c >> 4)] = (uint8_t)sc;
  }
  // the run's codes into column-major LDS, then column u of the tile out
#pragma unroll
  for (int k = 0; k < 16; ++k) {
    const uint32_t wd = k < 8 ? packed.x : packed.y;
    ct[lc0 + k][lr0 + u] = (uint8_t)((wd >> (4 * (k & 7))) & 0xFu);
  }
  __syncthreads();
  const uint4 col = *reinterpret_cast<const uint4*>(&ct[lc0 + u][lr0]);
  const uint32_t cb[4] = {col.x, col.y, col.z, col.w};   // byte k = code of row lr0 + k
  uint32_t pk[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 16; ++k) pk[k >> 3] |= ((cb[k >> 2] >> (8 * (k & 3))) & 0xFu) << (4 * (k & 7));
  if (inside) {
    const int64_t growt = (int64_t)bt * cols + c0 + lc0 + u;
    const int64_t r = r0 + lr0;
    *reinterpret_cast<uint2*>(out_t.codes + growt * (rows >> 1) + (r >> 1)) = uint2{pk[0], pk[1]};
    out_t.scales[growt * (rows >> 4) + (r >> 4)] = (uint8_t)sc;
  }
}

// ---------------------------------------------------------------------------
// transposed residual of the wgrad product: Q4((a - 1 mu)^T), cols x rows,
// 16-blocks along the rows (tokens).  A workgroup stages a 128-token x
// 64-column tile of the input in LDS as loaded (full 128-byte row reads of
// bf16 input; 18 KB, so eight workgroups fit a CU) and each thread
// quantizes one token block of two neighbouring columns, forming the
// residual fp32(a - mu) as it reads the tile.  Each output row gets 64
// contiguous code bytes per workgroup.  The tensor scale is the residual's,
// read from the split's output (the same set of values).
// ---------------------------------------------------------------------------
constexpr int kRtRows = 128;
constexpr int kRtCols = 64;

template <typename T, bool SR>
__global__ __launch_bounds__(256) void k_quant_rt(const T* __restrict__ a, int64_t rows,
                                                  int64_t cols, int64_t lda,
                                                  const float* __restrict__ mu,
                                                  const float* __restrict__ tsc, uint64_t seed,
                                                  uint32_t stream, QuantOut out) {
  constexpr int VE = 16 / (int)sizeof(T);
  constexpr int NCH = kRtCols / VE;              // 16-byte chunks per tile row
  constexpr int PER = kRtRows * NCH / 256;       // chunks per thread
  constexpr int LD = kRtCols + VE;               // padded LDS row (elements, 16-byte aligned)
  __shared__ __attribute__((aligned(16))) T tile[kRtRows][LD];
  const int64_t c0 = (int64_t)blockIdx.x * kRtCols, r0 = (int64_t)blockIdx.y * kRtRows;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + 256 * i;
    const int lr = idx / NCH, ch = idx % NCH;
    const int64_t r = r0 + lr, c = c0 + (int64_t)ch * VE;
    // cols % 16 == 0, so a chunk lies wholly inside or outside the tensor
    if (r < rows && c < cols)
      *reinterpret_cast<uint4*>(&tile[lr][ch * VE]) = *reinterpret_cast<const uint4*>(a + r * lda + c);
  }
  __syncthreads();
  const float s_enc = tsc[0];
  if (blockIdx.x == 0 && blockIdx.y == 0 && tid == 0) {
    out.tscale[0] = tsc[0];
    out.tscale[1] = tsc[1];
  }
  const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
  const int cp = tid & 31, q = tid >> 5;     // column pair, token block of the tile
  const int64_t c = c0 + 2 * cp, r = r0 + 16 * q;
  const bool live = c < cols && r < rows;    // cols % 16, rows % 16 == 0: whole pairs, blocks
  float v0[16], v1[16];
  if (live) {
    const float m0 = mu[c], m1 = mu[c + 1];
#pragma unroll
    for (int k = 0; k < 16; ++k) {
      if constexpr (sizeof(T) == 2) {
        const uint32_t w = *reinterpret_cast<const uint32_t*>(&tile[16 * q + k][2 * cp]);
        v0[k] = bf16_lo(w) - m0;
        v1[k] = bf16_hi(w) - m1;
      } else {
        const float2 w = *reinterpret_cast<const float2*>(&tile[16 * q + k][2 * cp]);
        v0[k] = w.x - m0;
        v1[k] = w.y - m1;
      }
    }
  }
  __syncthreads();   // the tile is read: its memory stages the output
  // codes [64 columns][64 bytes + 16 pad] (16-byte aligned rows), then
  // scales [64 columns][8 bytes]
  constexpr int kCodeLd = 80;
  uint8_t* cst = reinterpret_cast<uint8_t*>(&tile[0][0]);
  uint8_t* sst = cst + kRtCols * kCodeLd;
  static_assert(kRtCols * (kCodeLd + 8) <= (int)sizeof(tile), "output staging fits the tile");
  static_assert(kCodeLd % 16 == 0, "16-byte aligned staged code rows");
  if (live) {
    quant_block16<SR>(v0, s_enc, (uint64_t)c * (uint64_t)rows + (uint64_t)r, k0, k1, stream,
                      cst + (2 * cp) * kCodeLd + 8 * q, sst + (2 * cp) * 8 + q);
    quant_block16<SR>(v1, s_enc, (uint64_t)(c + 1) * (uint64_t)rows + (uint64_t)r, k0, k1, stream,
                      cst + (2 * cp + 1) * kCodeLd + 8 * q, sst + (2 * cp + 1) * 8 + q);
  }
  __syncthreads();
  // each column's 64 code bytes of this tile go out in 16-byte pieces (four
  // lanes to a column) when the rows keep them 16-byte aligned, else in
  // 8-byte pieces; pieces past the last token are skipped
  {
    const int col = tid >> 2, pc = tid & 3;
    const int64_t gc = c0 + col, t0 = r0 + 32 * pc;   // first token of the piece
    if (gc < cols && t0 < rows) {
      uint8_t* dst = out.codes + gc * (rows >> 1) + (t0 >> 1);
      const uint8_t* src = cst + col * kCodeLd + 16 * pc;
      if ((rows & 31) == 0) {
        *reinterpret_cast<uint4*>(dst) = *reinterpret_cast<const uint4*>(src);
      } else {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
        if (t0 + 16 < rows)
          *reinterpret_cast<uint2*>(dst + 8) = *reinterpret_cast<const uint2*>(src + 8);
      }
    }
  }
  if (tid < kRtCols) {
    const int64_t gc = c0 + tid;
    if (gc < cols && r0 < rows) {
      uint8_t* dst = out.scales + gc * (rows >> 4) + (r0 >> 4);
      const uint8_t* src = sst + tid * 8;
      if ((rows & 127) == 0) {
        *reinterpret_cast<uint2*>(dst) = *reinterpret_cast<const uint2*>(src);
      } else {
        for (int b = 0; b < 8 && r0 + 16 * b < rows; ++b) dst[b] = src[b];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// host launchers
// ---------------------------------------------------------------------------
// finalize (split, over chunks of ch rows) and quant passes
template <typename T>
static hipError_t run_finalize_quant(const T* a, int64_t rows, int64_t cols, int64_t lda,
                                     const int64_t* offs, int nseg, bool split, bool sr,
                                     uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                     const QuantOut* mean, float* mean_f32, const SplitWs& ws,
                                     hipStream_t st, float* ratio, const Rank1Out* r1,
                                     int64_t ch) {
  const int64_t nchq = chunk_upper_bound(rows, nseg, kQuantRows);
  const int64_t ct_s = (cols + kPlainStatsCols - 1) / kPlainStatsCols;
  // finalize: many short segments (on average at most 16 chunks) take the
  // per-segment-wave kernel in 64-column tiles, else 16-column tiles with
  // the chunks spread over the lanes
  const bool fin_seg = nseg > 1 && chunk_upper_bound(rows, nseg, ch) <= 16 * (int64_t)nseg;
  const int64_t fin_cols = fin_seg ? 64 : kFinCols;
  const int64_t ct_f = (cols + fin_cols - 1) / fin_cols;   // <= the workspace's tiles
  const int64_t ct_q = ((cols >> 4) + 63) / 64;
  int64_t ntmax;
  const float* tmax;
  if (split) {
    if (fin_seg) {
      dim3 g((unsigned)ct_f, (unsigned)((nseg + 3) / 4));
      k_finalize_seg<<<g, 256, 0, st>>>(a, sizeof(T) == 2, lda, rows, cols, offs, nseg, ws.psum,
                                        ws.pmax, ws.pmin, ws.pmnz, ws.mu, mean_f32, ws.tmax_r,
                                        ws.tmax_mu, ratio ? ws.psq : nullptr, ws.tssq, ws.tmu2,
                                        ch);
    } else {
      dim3 g((unsigned)ct_f, (unsigned)nseg);
      k_finalize<<<g, 256, 0, st>>>(a, sizeof(T) == 2, lda, rows, cols, offs, nseg, ws.psum,
                                    ws.pmax, ws.pmin, ws.pmnz, ws.mu, mean_f32, ws.tmax_r,
                                    ws.tmax_mu, ratio ? ws.psq : nullptr, ws.tssq, ws.tmu2, ch);
    }
    tmax = ws.tmax_r;
    ntmax = ct_f;
  } else {
    // the quant blocks reduce the stats partials (chunks x column tiles) directly
    tmax = ws.pamax;
    ntmax = ct_s;
  }
  // rank-one workgroups take the leading grid rows: r1_rows rows of one
  // segment's B each, 16 while that gives at most 512 workgroups, else up to
  // 128 (many experts' weights: the mean's quantization and staging, which
  // every such workgroup repeats, spread over more rows)
  Rank1Set rs{};
  auto r1_wgs = [&](int rows_per) {
    int64_t g = 0;
    for (int i = 0; i < (r1 ? r1->count : 0); ++i) g += (r1->n[i] + rows_per - 1) / rows_per * nseg;
    return g;
  };
  int r1_rows = 16;
  while (r1 && r1_rows < 128 && r1_wgs(r1_rows) > 512) r1_rows *= 2;
  int64_t gend = 0;
  for (int i = 0; i < (r1 ? r1->count : 0); ++i) {
    rs.b[i] = r1->b[i];
    rs.n[i] = r1->n[i];
    rs.rho[i] = r1->rho[i];
    gend += (r1->n[i] + r1_rows - 1) / r1_rows * nseg;
    rs.gend[i] = gend;
  }
  rs.count = r1 ? r1->count : 0;
  const int64_t rho_rows = (gend + ct_q - 1) / ct_q;
  const size_t lds_r1 = rs.count ? (size_t)cols * 2 : 0;
  dim3 gq((unsigned)ct_q, (unsigned)(rho_rows + nchq + nseg));
  // the staged mean of the rank-one workgroups (at most 64 KB)
#define AVERIS_QUANT_LAUNCH(SPL, SRB)                                                        \
  if (lds_r1) {                                                                             \
    const hipError_t e = lds_attr_once<&k_quant<T, SPL, SRB>>(64 * 1024);                   \
    if (e != hipSuccess) return e;                                                          \
  }                                                                                         \
  k_quant<T, SPL, SRB><<<gq, 256, lds_r1, st>>>(                                            \
      a, rows, cols, lda, offs, nseg, nchq, seed, stream_id, ws.mu, tmax, ntmax, ws.tmax_mu, \
      ct_f, out.codes, out.scales, out.tscale, mean ? mean->codes : nullptr,                \
      mean ? mean->scales : nullptr, mean ? mean->tscale : nullptr, ws.tssq, ws.tmu2, ratio, \
      rs, rho_rows, r1_rows)
  if (split) {
    if (sr) { AVERIS_QUANT_LAUNCH(true, true); } else { AVERIS_QUANT_LAUNCH(true, false); }
  } else {
    if (sr) { AVERIS_QUANT_LAUNCH(false, true); } else { AVERIS_QUANT_LAUNCH(false, false); }
  }
#undef AVERIS_QUANT_LAUNCH
  return hipGetLastError();
}

template <typename T>
static hipError_t run_split_or_plain(const void* a_, int64_t rows, int64_t cols, int64_t lda,
                                     const int64_t* offs, int nseg, bool split, bool sr,
                                     uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                     const QuantOut* mean, float* mean_f32, const SplitWs& ws,
                                     hipStream_t st, float* ratio, const Rank1Out* r1) {
  const T* a = static_cast<const T*>(a_);
  const int64_t nchs = chunk_upper_bound(rows, nseg, kStatsRows);
  // column blocks of the stats kernel (the plain one's also index its maxima)
  const int64_t cw = split ? StatsShape<true>::CW : StatsShape<false>::CW;
  const int64_t ct_s = (cols + cw - 1) / cw;
  if (nchs > 0) {
    dim3 g((unsigned)ct_s, (unsigned)nchs);
    if (split && ratio)
      k_stats<T, true, true><<<g, 256, 0, st>>>(a, rows, cols, lda, offs, nseg, ws.psum, ws.pmax,
                                                ws.pmin, ws.pmnz, nullptr, ws.psq);
    else if (split)
      k_stats<T, true><<<g, 256, 0, st>>>(a, rows, cols, lda, offs, nseg, ws.psum, ws.pmax,
                                          ws.pmin, ws.pmnz, nullptr);
    else
      k_stats<T, false><<<g, 256, 0, st>>>(a, rows, cols, lda, offs, nseg, nullptr, nullptr,
                                           nullptr, nullptr, ws.pamax);
  }
  return run_finalize_quant<T>(a, rows, cols, lda, offs, nseg, split, sr, seed, stream_id, out,
                               mean, mean_f32, ws, st, ratio, r1, kStatsRows);
}

hipError_t launch_split_from_stats(const void* a, bool bf16, int64_t rows, int64_t cols,
                                   int64_t lda, const int64_t* offs, int nseg, int64_t ch, bool sr,
                                   uint64_t seed, const QuantOut& out, const QuantOut& mean,
                                   float* mean_f32, const SplitWs& ws, hipStream_t st,
                                   const Rank1Out* r1) {
  if (bf16)
    return run_finalize_quant<uint16_t>(static_cast<const uint16_t*>(a), rows, cols, lda, offs,
                                        nseg, true, sr, seed, 0u, out, &mean, mean_f32, ws, st,
                                        nullptr, r1, ch);
  return run_finalize_quant<float>(static_cast<const float*>(a), rows, cols, lda, offs, nseg,
                                   true, sr, seed, 0u, out, &mean, mean_f32, ws, st, nullptr, r1,
                                   ch);
}

hipError_t launch_split_or_plain(const void* a, bool bf16, int64_t rows, int64_t cols,
                                 int64_t lda, const int64_t* offs, int nseg, bool split, bool sr,
                                 uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                 const QuantOut* mean, float* mean_f32, const SplitWs& ws,
                                 hipStream_t st, float* ratio, const Rank1Out* r1) {
  if (bf16)
    return run_split_or_plain<uint16_t>(a, rows, cols, lda, offs, nseg, split, sr, seed,
                                        stream_id, out, mean, mean_f32, ws, st, ratio, r1);
  return run_split_or_plain<float>(a, rows, cols, lda, offs, nseg, split, sr, seed, stream_id,
                                   out, mean, mean_f32, ws, st, ratio, r1);
}

template <typename T>
static hipError_t run_batched(const void* a_, int batch, int64_t rows, int64_t cols, int64_t lda,
                              int64_t bstride, int transpose, bool sr, uint64_t seed,
                              uint32_t stream_id, const QuantOut& out, float* part,
                              hipStream_t st) {
  const T* a = static_cast<const T*>(a_);
  const int64_t srows = transpose ? cols : rows, scols = transpose ? rows : cols;
  const int64_t n = srows * scols;
  int64_t nblk = (n + 256 * 8 - 1) / (256 * 8);
  if (nblk > kAmaxBlocks) nblk = kAmaxBlocks;
  if (nblk < 1) nblk = 1;
  k_amax_batched<T><<<dim3((unsigned)nblk, (unsigned)batch), 256, 0, st>>>(a, srows, scols, lda,
                                                                           bstride, part);
  if (rows > 0) {
    dim3 g((unsigned)((rows + 255) / 256), (unsigned)(cols >> 4), (unsigned)batch);
    if (sr)
      k_quant_batched<T, true><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, transpose, seed,
                                                  stream_id, part, nblk, out.codes, out.scales,
                                                  out.tscale);
    else
      k_quant_batched<T, false><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, transpose, seed,
                                                   stream_id, part, nblk, out.codes, out.scales,
                                                   out.tscale);
  }
  return hipGetLastError();
}

hipError_t launch_quant_batched(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                                int64_t lda, int64_t bstride, int transpose, bool sr,
                                uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                float* part, hipStream_t st) {
  if (bf16)
    return run_batched<uint16_t>(a, batch, rows, cols, lda, bstride, transpose, sr, seed,
                                 stream_id, out, part, st);
  return run_batched<float>(a, batch, rows, cols, lda, bstride, transpose, sr, seed, stream_id,
                            out, part, st);
}

template <typename T>
static hipError_t run_pair(const void* a_, int batch, int64_t rows, int64_t cols, int64_t lda,
                           int64_t bstride, bool sr, uint64_t seed, uint32_t stream_id,
                           const QuantOut& out, const QuantOut& out_t, float* part,
                           hipStream_t st) {
  const T* a = static_cast<const T*>(a_);
  constexpr int64_t VE = 16 / (int64_t)sizeof(T);
  const int64_t total = rows * (cols / VE);
  int64_t nblk = (total + 256 * 4 - 1) / (256 * 4);
  if (nblk > kAmaxBlocks) nblk = kAmaxBlocks;
  if (nblk < 1) nblk = 1;
  const int64_t per = (total + nblk - 1) / nblk;
  k_amax_vec<T><<<dim3((unsigned)nblk, (unsigned)batch), 256, 0, st>>>(a, rows, cols, lda, bstride,
                                                                       per, part);
  const dim3 g((unsigned)((cols + kPairTile - 1) / kPairTile),
               (unsigned)((rows + kPairTile - 1) / kPairTile), (unsigned)batch);
  if (sr)
    k_pair<T, true><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, seed, stream_id, part, nblk,
                                       out, out_t);
  else
    k_pair<T, false><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, seed, stream_id, part, nblk,
                                        out, out_t);
  return hipGetLastError();
}

template <typename T>
static hipError_t run_pair2d(const void* a_, int batch, int64_t rows, int64_t cols, int64_t lda,
                             int64_t bstride, bool sr, uint64_t seed, uint32_t stream_id,
                             const QuantOut& out, const QuantOut& out_t, float* part,
                             hipStream_t st) {
  const T* a = static_cast<const T*>(a_);
  constexpr int64_t VE = 16 / (int64_t)sizeof(T);
  const int64_t total = rows * (cols / VE);
  int64_t nblk = (total + 256 * 4 - 1) / (256 * 4);
  if (nblk > kAmaxBlocks) nblk = kAmaxBlocks;
  if (nblk < 1) nblk = 1;
  const int64_t per = (total + nblk - 1) / nblk;
  k_amax_vec<T><<<dim3((unsigned)nblk, (unsigned)batch), 256, 0, st>>>(a, rows, cols, lda, bstride,
                                                                       per, part);
  const dim3 g((unsigned)((cols + kPairTile - 1) / kPairTile),
               (unsigned)((rows + kPairTile - 1) / kPairTile), (unsigned)batch);
  if (sr)
    k_pair2d<T, true><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, seed, stream_id, part, nblk,
                                         out, out_t);
  else
    k_pair2d<T, false><<<g, 256, 0, st>>>(a, rows, cols, lda, bstride, seed, stream_id, part, nblk,
                                          out, out_t);
  return hipGetLastError();
}

hipError_t launch_quant_pair2d(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                               int64_t lda, int64_t bstride, bool sr, uint64_t seed,
                               uint32_t stream_id, const QuantOut& out, const QuantOut& out_t,
                               float* part, hipStream_t st) {
  if (bf16)
    return run_pair2d<uint16_t>(a, batch, rows, cols, lda, bstride, sr, seed, stream_id, out,
                                out_t, part, st);
  return run_pair2d<float>(a, batch, rows, cols, lda, bstride, sr, seed, stream_id, out, out_t,
                           part, st);
}

hipError_t launch_quant_pair(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                             int64_t lda, int64_t bstride, bool sr, uint64_t seed,
                             uint32_t stream_id, const QuantOut& out, const QuantOut& out_t,
                             float* part, hipStream_t st) {
  if (bf16)
    return run_pair<uint16_t>(a, batch, rows, cols, lda, bstride, sr, seed, stream_id, out, out_t,
                              part, st);
  return run_pair<float>(a, batch, rows, cols, lda, bstride, sr, seed, stream_id, out, out_t, part,
                         st);
}

template <typename T>
static hipError_t run_pair_multi(int n, const WeightPair* w, bool sr, uint32_t stream_id,
                                 float* part, hipStream_t st) {
  constexpr int64_t VE = 16 / (int64_t)sizeof(T);
  PairMultiArgs args{};
  args.n = n;
  int64_t amax_wgs = 0, tiles = 0;
  for (int i = 0; i < n; ++i) {
    args.w[i] = w[i];
    // the single-weight launch's partition of the amax pass
    const int64_t total = w[i].rows * (w[i].cols / VE);
    int64_t nblk = (total + 256 * 4 - 1) / (256 * 4);
    if (nblk > kAmaxBlocks) nblk = kAmaxBlocks;
    if (nblk < 1) nblk = 1;
    args.per[i] = (total + nblk - 1) / nblk;
    args.nblk[i] = nblk;
    amax_wgs += nblk;
    args.amax_end[i] = amax_wgs;
    args.tiles_x[i] = (w[i].cols + kPairTile - 1) / kPairTile;
    tiles += args.tiles_x[i] * ((w[i].rows + kPairTile - 1) / kPairTile);
    args.tile_end[i] = tiles;
  }
  k_amax_multi<T><<<(unsigned)amax_wgs, 256, 0, st>>>(args, part);
  if (sr)
    k_pair_multi<T, true><<<(unsigned)tiles, 256, 0, st>>>(args, stream_id, part);
  else
    k_pair_multi<T, false><<<(unsigned)tiles, 256, 0, st>>>(args, stream_id, part);
  return hipGetLastError();
}

hipError_t launch_quant_pair_multi(int n, const WeightPair* w, bool bf16, bool sr,
                                   uint32_t stream_id, float* part, hipStream_t st) {
  if (bf16) return run_pair_multi<uint16_t>(n, w, sr, stream_id, part, st);
  return run_pair_multi<float>(n, w, sr, stream_id, part, st);
}

template <typename T>
static hipError_t run_rt(const void* a_, int64_t rows, int64_t cols, int64_t lda, const float* mu,
                         const float* tsc, bool sr, uint64_t seed, uint32_t stream_id,
                         const QuantOut& out, hipStream_t st) {
  const T* a = static_cast<const T*>(a_);
  // at least one workgroup: block (0, 0) also publishes the tensor scale
  // when there are no tokens
  const int64_t gy = (rows + kRtRows - 1) / kRtRows;
  const dim3 g((unsigned)((cols + kRtCols - 1) / kRtCols), (unsigned)(gy > 0 ? gy : 1));
  if (sr)
    k_quant_rt<T, true><<<g, 256, 0, st>>>(a, rows, cols, lda, mu, tsc, seed, stream_id, out);
  else
    k_quant_rt<T, false><<<g, 256, 0, st>>>(a, rows, cols, lda, mu, tsc, seed, stream_id, out);
  return hipGetLastError();
}

hipError_t launch_quant_rt(const void* a, bool bf16, int64_t rows, int64_t cols, int64_t lda,
                           const float* mu, const float* tscale_in, bool sr, uint64_t seed,
                           uint32_t stream_id, const QuantOut& out, hipStream_t st) {
  if (bf16) return run_rt<uint16_t>(a, rows, cols, lda, mu, tscale_in, sr, seed, stream_id, out, st);
  return run_rt<float>(a, rows, cols, lda, mu, tscale_in, sr, seed, stream_id, out, st);
}

}  // namespace averis
