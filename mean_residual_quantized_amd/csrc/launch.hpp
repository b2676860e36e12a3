// Internal interface between the C ABI (api.cpp) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace averis {

// rows per chunk of the stats and quant passes
constexpr int64_t kStatsRows = 128;
// columns per block of the plain statistics pass (its per-chunk maxima are
// kept per block of columns)
constexpr int64_t kPlainStatsCols = 128;
constexpr int64_t kQuantRows = 16;
// cap on the blocks of the weight amax pass
constexpr int64_t kAmaxBlocks = 1024;
// columns per workgroup of the split-quant finalize pass
constexpr int64_t kFinCols = 16;

struct QuantOut {
  uint8_t* codes;
  uint8_t* scales;
  float* tscale;
};

// Workspace carve-up of the split / plain quant passes.
struct SplitWs {
  double* psum;    // [chunks][cols] partial column sums
  float* pmax;     // [chunks][cols]
  float* pmin;     // [chunks][cols]
  float* pmnz;     // [chunks][cols] smallest nonzero |a| (the exactness certificate)
  float* pamax;    // [chunks][col tiles] plain-pass max |a|
  float* mu;       // [nseg][cols]
  float* tmax_r;   // [nseg][col tiles] residual max |r| per column tile
  float* tmax_mu;  // [nseg][col tiles] max |mu| per column tile
  double* psq;     // [chunks][cols] partial column sums of squares (mean-energy ratio)
  double* tssq;    // [nseg][col tiles] sum of squares per column tile
  double* tmu2;    // [nseg][col tiles] sum of squared fp64 means per column tile
};

// A quantized GEMM operand as the kernels see it.
struct QOperand {
  const uint8_t* codes;
  const uint8_t* scales;
  const float* tscale;
};

// Column statistics of a GEMM's bf16 output, written by its epilogue for the
// split that will read that output: per row tile of kGemmRows rows (a chunk
// of that split) and column, the fp64 sum, max, min and smallest nonzero
// magnitude of the stored values, in the split workspace's partial arrays
// ([chunk][cols]).  psum == nullptr: none.
constexpr int64_t kGemmRows = 256;
struct ColStats {
  double* psum;
  float* pmax;
  float* pmin;
  float* pmnz;
};

// The rank-one rows a split can compute for the GEMMs that take it: for
// each of `count` B operands, rho_i[s][j] = deq(Q4(mu_s)) . deq(b_i,s,j) for
// the n_i rows of each segment's b_i (b_i holds nseg stacked n_i x cols
// matrices).  More than one B operand: one segment (GEMMs of one input).
constexpr int kMaxRank1 = 4;
struct Rank1Out {
  QOperand b[kMaxRank1];
  int64_t n[kMaxRank1];
  float* rho[kMaxRank1];
  int count;
};
inline Rank1Out rank1_one(const QOperand& b, int64_t n, float* rho) {
  Rank1Out r{};
  r.b[0] = b;
  r.n[0] = n;
  r.rho[0] = rho;
  r.count = 1;
  return r;
}

size_t split_ws_bytes(int64_t rows, int64_t cols, int nseg);
SplitWs split_ws_carve(void* ws, int64_t rows, int64_t cols, int nseg);
size_t batched_ws_bytes(int64_t rows, int64_t cols, int batch);

hipError_t launch_split_or_plain(const void* a, bool bf16, int64_t rows, int64_t cols,
                                 int64_t lda, const int64_t* offs, int nseg, bool split, bool sr,
                                 uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                 const QuantOut* mean, float* mean_f32, const SplitWs& ws,
                                 hipStream_t st, float* ratio = nullptr,
                                 const Rank1Out* r1 = nullptr);

hipError_t launch_quant_batched(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                                int64_t lda, int64_t bstride, int transpose, bool sr,
                                uint64_t seed, uint32_t stream_id, const QuantOut& out,
                                float* part, hipStream_t st);

// Q4(W_b) (out, blocks along cols) and Q4(W_b^T) (out_t, blocks along rows)
// of `batch` stored rows x cols matrices; part: batch x kAmaxBlocks floats.
hipError_t launch_quant_pair(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                             int64_t lda, int64_t bstride, bool sr, uint64_t seed,
                             uint32_t stream_id, const QuantOut& out, const QuantOut& out_t,
                             float* part, hipStream_t st);
// Both copies (as launch_quant_pair with batch 1) of each of n <= kMaxWeights
// stored matrices of their own shapes, in one amax and one pair launch;
// part: n x kAmaxBlocks floats.
constexpr int kMaxWeights = 16;
struct WeightPair {
  const void* a;
  int64_t rows, cols, lda;
  uint64_t seed;
  QuantOut out, out_t;
};
hipError_t launch_quant_pair_multi(int n, const WeightPair* w, bool bf16, bool sr,
                                   uint32_t stream_id, float* part, hipStream_t st);
hipError_t launch_quant_pair2d(const void* a, bool bf16, int batch, int64_t rows, int64_t cols,
                               int64_t lda, int64_t bstride, bool sr, uint64_t seed,
                               uint32_t stream_id, const QuantOut& out, const QuantOut& out_t,
                               float* part, hipStream_t st);

// Q4((a - 1 mu)^T) (cols x rows, blocks along the rows) with the residual's
// tensor scale tscale_in (2 floats); rows % 16 == 0, cols % 16 == 0.
hipError_t launch_quant_rt(const void* a, bool bf16, int64_t rows, int64_t cols, int64_t lda,
                           const float* mu, const float* tscale_in, bool sr, uint64_t seed,
                           uint32_t stream_id, const QuantOut& out, hipStream_t st);

// C[M x N] = deq(A) deq(B)^T (+ 1 deq(mean) deq(B)^T); grouped when offs != nullptr
// (B then holds nseg stacked N x K matrices).
hipError_t launch_gemm(const QOperand& a, const QOperand* mean, const QOperand& b, int64_t m,
                       int64_t n, int64_t k, const int64_t* offs, int nseg, void* c, bool c_bf16,
                       int64_t ldc, void* ws, hipStream_t st);

// C = deq(A) deq(B)^T + 1 rho^T with rho precomputed (n floats per segment;
// grouped when offs != nullptr, B then holding nseg stacked N x K matrices).
hipError_t launch_gemm_rho(const QOperand& a, const float* rho, const QOperand& b, int64_t m,
                           int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                           bool c_bf16, int64_t ldc, hipStream_t st);

// The same GEMM (bf16 output, K % 64 == 0) also writing the column statistics
// of its output into cs (kGemmRows-row chunks).
hipError_t launch_gemm_rho_stats(const QOperand& a, const float* rho, const QOperand& b, int64_t m,
                                 int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                                 int64_t ldc, const ColStats& cs, hipStream_t st);

// Split-quant from the column statistics a producer wrote (chunks of ch rows)
// into ws's partial arrays: the finalize and quant passes only (one read of a).
hipError_t launch_split_from_stats(const void* a, bool bf16, int64_t rows, int64_t cols,
                                   int64_t lda, const int64_t* offs, int nseg, int64_t ch, bool sr,
                                   uint64_t seed, const QuantOut& out, const QuantOut& mean,
                                   float* mean_f32, const SplitWs& ws, hipStream_t st,
                                   const Rank1Out* r1 = nullptr);

// Workspace of a GEMM call (rho, the rank-one term per segment and column).
size_t gemm_ws_bytes(int64_t n, int64_t k, int nseg);

// Warp-specialized GEMM (K % 64 == 0): variant for a shape (0 = not
// applicable) and its launch.  mean: the quantized mean rows (nseg x k),
// whose rank-one term the kernel adds itself, or nullptr for the vanilla
// product.
int ws_pick(int64_t m, int64_t n, int64_t k, int nseg_eff, bool has_mean);
hipError_t launch_gemm_ws(int variant, const QOperand& a, const QOperand* mean, const QOperand& b,
                          int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg, void* c,
                          bool c_bf16, int64_t ldc, hipStream_t st);
hipError_t launch_gemm_ws_rho(int variant, const QOperand& a, const float* rho, const QOperand& b,
                              int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
                              void* c, bool c_bf16, int64_t ldc, hipStream_t st,
                              const ColStats& cs = ColStats{nullptr, nullptr, nullptr, nullptr});

// GEMM with the operands staged in LDS as codes (K per split % 256 == 0):
// tile width 64 fn for a shape (0 = not applicable) and its launch.  rho:
// the rank-one row (n floats per segment) or nullptr; splits > 1: split-K
// into c + z c_split (fp32); cs.psum set: bf16 output with its column
// statistics (kGemmRows-row chunks).
int win_pick(int64_t m, int64_t n, int64_t k_split, int nseg_eff, int splits);
hipError_t launch_gemm_win(int fn, const QOperand& a, const float* rho, const QOperand& b,
                           int64_t m, int64_t n, int64_t k, const int64_t* offs, int nseg,
                           void* c, bool c_bf16, int64_t ldc, hipStream_t st, int splits = 1,
                           int64_t c_split = 0,
                           const ColStats& cs = ColStats{nullptr, nullptr, nullptr, nullptr});

// Split-K product into fp32 partials part[z] (m x n each, row stride n).
hipError_t launch_gemm_ws_splitk(const QOperand& a, const QOperand& b, int64_t m, int64_t n,
                                 int64_t k, int splits, float* part, hipStream_t st);

// wgrad: out (m x n, row stride ldo) = deq(xt) deq(dt)^T + l mu_x mu_d^T with
// xt m x l and dt n x l (blocks along the tokens); m, n % 16 == 0.
int wgrad_splits(int64_t m, int64_t n, int64_t l);
size_t wgrad_ws_bytes(int64_t m, int64_t n, int64_t l);
hipError_t launch_wgrad(const QOperand& xt, const QOperand& dt, const float* mu_x,
                        const float* mu_d, int64_t m, int64_t n, int64_t l, void* out, bool bf16,
                        int64_t ldo, void* ws, hipStream_t st);

}  // namespace averis
