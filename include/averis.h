/*
 * libaveris -- C ABI of the Averis mean-residual split FP4 linear on MI355X
 * (gfx950): split-quant, plain quant, and the quantized GEMMs of the forward
 * and dgrad passes, plus the vanilla-FP4 comparison arm.
 *
 * The method (from "The Curse and Blessing of Mean Bias in FP4-Quantized LLM
 * Training", as reviewed on the "Lighthouse" blog, §2.1-§2.2, and summarised
 * in the paper's arXiv abstract and the gist.science technical summary §2):
 *   mu_X   = (1/l) 1^T X                       column mean over the l tokens
 *   X_R    = X - 1 mu_X^T                      residual (unquantized mean)
 *   Y      = 1 (Q4(mu_X) Q4(W)) + Q4(X_R) Q4(W)          forward
 *   dX     = 1 (Q4(mu_D) Q4(W)^T) + Q4(D_R) Q4(W)^T      dgrad (D = dL/dY)
 * Q4 is NVFP4-style E2M1 with stochastic rounding by default (Lighthouse
 * §3.1; two-level "hierarchical" microscaling per "Dissecting Outlier
 * Dynamics in LLM NVFP4 Pretraining", abstract).
 *
 * Q4 as implemented (a reading; the pages give no bit-level recipe):
 *   blocks of 16 along the GEMM contraction axis (the tensor's columns);
 *   amax   = max |T| over the tensor (per segment for grouped calls)
 *   S_enc  = fp32(2688 / amax), or 1 when amax == 0 or the quotient is not
 *            finite;  S_dec = fp32(1 / S_enc)
 *   s_b    = fp32(fp32(amax_b / 6) * S_enc) capped at 448 -> E4M3FN (RNE,
 *            subnormals kept) = the block's scale byte, value d_b
 *   e_b    = fp32(S_enc / d_b) (0 if d_b == 0);  v = fp32(t * e_b)
 *   E2M1 code (sign << 3 | index into {0,.5,1,1.5,2,3,4,6}) by
 *     RN: nearest, ties to the even index, |v| >= 6 -> 6, or
 *     SR: with lo <= |v| < hi the neighbouring grid points and
 *         frac = (|v| - lo) / (hi - lo), up iff floor(2^22 frac) + 64 u >= 2^22,
 *         u the element's 16-bit
 *         draw from Philox4x32-10: key = seed, counter = (g lo, g hi,
 *         stream, 0), g = idx >> 3, word (idx >> 1) & 3, half idx & 1,
 *         idx = row * cols + col (global row for grouped tensors).
 *   SR streams: 0 residual and vanilla activations, 1 means, 2 weights,
 *   3 transposed residuals (wgrad).
 *   The mean is fp32(RN64(exact column sum) / l); the residual is
 *   fp32(x - mu) with the unquantized mean.
 *
 * Conventions for every entry point:
 *   - All tensor pointers are DEVICE pointers owned by the caller.  The
 *     library allocates nothing and keeps no state between calls beyond a
 *     per-device record that a kernel's LDS limit was raised (set once,
 *     atomically); calls may come from several threads.
 *   - Work is enqueued on `stream` (NULL = the default stream) and the call
 *     returns without synchronising.  Scales flow device to device.
 *   - Arguments are validated before any HIP call; a rejected call enqueues
 *     nothing and returns the status.  Nothing aborts.
 *   - The workspace `ws` (device, >= averis_workspace_bytes(...) bytes,
 *     256-byte aligned) holds intermediate results only; its contents on
 *     entry do not matter.  Calls that share a workspace must be ordered on
 *     one stream.
 *   - Values that are not finite in an input give unspecified codes.
 */
#ifndef AVERIS_H
#define AVERIS_H

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define AVERIS_ABI_VERSION 1

typedef enum {
  AVERIS_OK = 0,
  AVERIS_E_NULL = 1,       /* a required pointer is NULL                      */
  AVERIS_E_SHAPE = 2,      /* negative size, cols % 16 != 0, operand mismatch */
  AVERIS_E_DTYPE = 3,      /* unknown dtype                                   */
  AVERIS_E_ALIGN = 4,      /* pointer or leading dimension misaligned         */
  AVERIS_E_WORKSPACE = 5,  /* workspace missing or smaller than required      */
  AVERIS_E_ARG = 6,        /* other invalid argument (rounding, stream, nseg) */
  AVERIS_E_HIP = 7         /* a kernel launch failed                          */
} averis_status_t;

typedef enum { AVERIS_F32 = 0, AVERIS_BF16 = 1 } averis_dtype_t;
typedef enum { AVERIS_RN = 0, AVERIS_SR = 1 } averis_round_t;

/* Workspace queries, see averis_workspace_bytes. */
typedef enum {
  AVERIS_OP_SPLIT_QUANT = 0,  /* rows, cols, nseg (nseg = 0: not grouped)     */
  AVERIS_OP_QUANT = 1,        /* rows, cols, nseg (batch for batched quant)   */
  AVERIS_OP_GEMM = 2,         /* rows = M, cols = K, n = N, nseg              */
  AVERIS_OP_WGRAD = 3,        /* rows = m, cols = l (tokens), n               */
  AVERIS_OP_QUANT_PAIR_MULTI = 4  /* n = number of weights (rows, cols unused) */
} averis_op_t;

/* An NVFP4-style tensor of rows x cols logical elements, 16-blocks along
 * cols.  codes: rows * cols/2 bytes, row-major, byte j of a row holds element
 * 2j in bits 3:0 and element 2j+1 in bits 7:4; 16-byte aligned.
 * scales: rows * cols/16 E4M3FN bytes, row-major; 16-byte aligned.
 * tscale: 2 floats [S_enc, S_dec] per tensor (per segment / batch entry for
 * grouped calls).
 * All three are device pointers. */
typedef struct {
  uint8_t* codes;
  uint8_t* scales;
  float*   tscale;
  int64_t  rows;
  int64_t  cols;
} averis_nvfp4_t;

/* ---------------------------------------------------------------------- */
/* Split-quant (Lighthouse §2.1 column mean; §2.2 X_R = X - 1 mu, separate */
/* quantization of mean and residual; gist.science summary §2).            */
/* ---------------------------------------------------------------------- */

/* a: rows x cols activation or output gradient (dtype F32 or BF16), row
 * stride lda elements (lda >= cols, lda * element size a multiple of 16
 * bytes, a 16-byte aligned).  Writes
 *   residual: rows x cols, Q4(a - 1 mu) with SR stream 0 (or RN),
 *   mean:     1 x cols,    Q4(mu) with SR stream 1 (or RN),
 *   mean_f32: the fp32 mean (optional, may be NULL), cols floats.
 * rows == 0 gives mu = 0 and an all-zero mean tensor with S_enc = 1.
 * Workspace: averis_workspace_bytes(AVERIS_OP_SPLIT_QUANT, rows, cols, 0, 0). */
averis_status_t averis_split_quant(const void* a, averis_dtype_t dtype, int64_t rows, int64_t cols,
                                   int64_t lda, uint64_t seed, averis_round_t rnd,
                                   const averis_nvfp4_t* residual, const averis_nvfp4_t* mean,
                                   float* mean_f32, void* ws, size_t ws_bytes, hipStream_t stream);

/* Grouped split-quant over expert segments (the paper's MoE runs, arXiv
 * abstract): rows seg_offsets[s] .. seg_offsets[s+1]-1 form segment s, each
 * with its own mean (row s of `mean`, nseg x cols, SR index s*cols + col)
 * and its own residual tensor scale (residual->tscale holds 2*nseg floats,
 * as does mean->tscale).  seg_offsets: DEVICE int64[nseg+1], non-decreasing,
 * seg_offsets[0] = 0, seg_offsets[nseg] = rows (the kernels clamp values
 * outside [0, rows]).  mean_f32 (optional): nseg x cols.  An empty segment
 * has mean 0.  Workspace: AVERIS_OP_SPLIT_QUANT with nseg. */
averis_status_t averis_split_quant_grouped(const void* a, averis_dtype_t dtype, int64_t rows,
                                           int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                           int nseg, uint64_t seed, averis_round_t rnd,
                                           const averis_nvfp4_t* residual,
                                           const averis_nvfp4_t* mean, float* mean_f32, void* ws,
                                           size_t ws_bytes, hipStream_t stream);

/* Split-quant with the mean-energy ratio ([Lighthouse] §7 recommends
 * monitoring R = ||mu||_2 / sqrt(E||X||^2 / N) as a free stability signal).
 * Reading: E||X||^2 is the operand's sum of squares ||A||_F^2 and N its row
 * count l, so R = ||mu||_2 / sqrt(||A||_F^2 / l) in [0, 1] (1 when every row
 * equals mu), computed from fp64 column sums and sums of squares gathered in
 * the statistics pass; R = 0 for an empty segment or an all-zero one.
 * seg_offsets = NULL with nseg = 1 is averis_split_quant, otherwise
 * averis_split_quant_grouped; the quantized outputs are bit for bit those of
 * that call.  ratio: device float[nseg] (4-byte aligned), required.
 * Workspace: AVERIS_OP_SPLIT_QUANT as for the call it extends. */
averis_status_t averis_split_quant_ratio(const void* a, averis_dtype_t dtype, int64_t rows,
                                         int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                         int nseg, uint64_t seed, averis_round_t rnd,
                                         const averis_nvfp4_t* residual,
                                         const averis_nvfp4_t* mean, float* mean_f32, float* ratio,
                                         void* ws, size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Plain quant: the vanilla-FP4 arm (arXiv abstract: "vanilla NVFP4") and  */
/* the weight operand W (Lighthouse §2.2, both equations).                 */
/* ---------------------------------------------------------------------- */

/* Q4 of the logical rows x cols tensor T, blocks along cols, one tensor
 * scale.  transpose = 0: T[r][c] = a[r*lda + c]; transpose = 1:
 * T[r][c] = a[c*lda + r] (a stored cols x rows; used for the forward copy
 * of W, Q4(W^T)).  sr_stream: 0 for activations, 2 for weights.
 * Workspace: AVERIS_OP_QUANT (rows, cols, 0). */
averis_status_t averis_quant(const void* a, averis_dtype_t dtype, int64_t rows, int64_t cols,
                             int64_t lda, int transpose, uint64_t seed, averis_round_t rnd,
                             uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream);

/* Batched plain quant: `batch` independent rows x cols tensors (matrix b at
 * a + b*batch_stride elements), each with its own tensor scale
 * (out->tscale: 2*batch floats); out is (batch*rows) x cols and the SR index
 * uses the global row b*rows + r.  Used for per-expert weights.
 * Workspace: AVERIS_OP_QUANT (rows, cols, batch). */
averis_status_t averis_quant_batched(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                     int64_t cols, int64_t lda, int64_t batch_stride,
                                     int transpose, uint64_t seed, averis_round_t rnd,
                                     uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* Both quantized copies of a weight in one call (Lighthouse §2.2: the
 * forward product takes Q4(W^T) with blocks along m, the dgrad product Q4(W)
 * with blocks along n).  a holds `batch` stored rows x cols matrices W_b
 * (row stride lda, matrix b at a + b*batch_stride elements).  Writes
 *   out   = Q4(W_b),   (batch*rows) x cols, blocks along cols, and
 *   out_t = Q4(W_b^T), (batch*cols) x rows, blocks along rows,
 * with one tensor scale per matrix (max |W_b|, shared by both copies).
 * Codes, scales and tensor scales are those of averis_quant_batched with
 * transpose = 0 (out) and transpose = 1 (out_t), the same seed and stream,
 * bit for bit.  Needs rows % 16 == 0, cols % 16 == 0, both > 0, 16-byte
 * aligned a and lda * element size % 16 == 0.
 * Workspace: AVERIS_OP_QUANT (rows, cols, batch). */
averis_status_t averis_quant_pair(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                  int64_t cols, int64_t lda, int64_t batch_stride, uint64_t seed,
                                  averis_round_t rnd, uint32_t sr_stream,
                                  const averis_nvfp4_t* out, const averis_nvfp4_t* out_t,
                                  void* ws, size_t ws_bytes, hipStream_t stream);

/* Both GEMM copies of a weight from ONE quantization in 16 x 16 tiles (the
 * shared weight that Lighthouse §2.2 implies by writing the dgrad operand as
 * the transpose of the forward one).  Same arguments, shapes, layouts and
 * workspace as averis_quant_pair; the difference: each 16 x 16 tile of W_b
 * has one E4M3 scale, from the tile's largest magnitude, and the codes are
 * encoded once (SR draw of element (r, c) of W_b: index (b*rows + r) * cols
 * + c, stream sr_stream) and written in both layouts, so that
 * deq(out_t) = deq(out)^T exactly.  Every 16-run of out and of out_t carries
 * its tile's scale byte; the GEMM calls take both copies unchanged.
 * Errors as averis_quant_pair. */
averis_status_t averis_quant_pair_2d(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                     int64_t cols, int64_t lda, int64_t batch_stride,
                                     uint64_t seed, averis_round_t rnd, uint32_t sr_stream,
                                     const averis_nvfp4_t* out, const averis_nvfp4_t* out_t,
                                     void* ws, size_t ws_bytes, hipStream_t stream);

/* One weight of averis_quant_pair_multi: the stored rows x cols matrix W at
 * a (device, row stride lda elements), its seed and its two outputs (host
 * pointers to descriptors of device buffers): out = Q4(W), rows x cols, and
 * out_t = Q4(W^T), cols x rows, as averis_quant_pair writes them with
 * batch 1. */
typedef struct {
  const void* a;
  int64_t rows;
  int64_t cols;
  int64_t lda;
  uint64_t seed;
  const averis_nvfp4_t* out;
  const averis_nvfp4_t* out_t;
} averis_weight_t;

#define AVERIS_MAX_WEIGHTS 16

/* Both quantized copies of each of n weights of their own shapes (Lighthouse
 * §2.2, as averis_quant_pair; e.g. the seven linears of a transformer block,
 * all known when a step starts) in two launches instead of two per weight.
 * For every i the codes, scales and tensor scales are those of
 * averis_quant_pair(w[i].a, dtype, 1, w[i].rows, w[i].cols, w[i].lda, 0,
 * w[i].seed, rnd, sr_stream, w[i].out, w[i].out_t, ...), bit for bit.
 * w: host array of n entries (1 <= n <= AVERIS_MAX_WEIGHTS), read during the
 * call only; every entry must meet averis_quant_pair's requirements (else
 * that call's status, nothing launched).  The outputs of different entries
 * must not overlap.  Workspace: AVERIS_OP_QUANT_PAIR_MULTI with n. */
averis_status_t averis_quant_pair_multi(int n, const averis_weight_t* w, averis_dtype_t dtype,
                                        averis_round_t rnd, uint32_t sr_stream, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* Grouped plain quant of activations: one tensor scale per segment
 * (vanilla arm of the grouped case).  Workspace: AVERIS_OP_QUANT with nseg. */
averis_status_t averis_quant_grouped(const void* a, averis_dtype_t dtype, int64_t rows,
                                     int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                     int nseg, uint64_t seed, averis_round_t rnd,
                                     uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Quantized GEMMs (Lighthouse §2.2; gist.science summary §2).             */
/* C = deq(A) deq(B)^T (+ 1 deq(mean) deq(B)^T), FP32 accumulation.        */
/* ---------------------------------------------------------------------- */

/* Forward: y (xr->rows x wt->rows) = 1 (mean W) + X_R W with
 *   xr:   Q4(X - 1 mu), l x m
 *   mean: Q4(mu), 1 x m
 *   wt:   Q4(W^T), n x m (blocks along m)
 * y: F32 or BF16, row stride ldy >= n elements.  Workspace: AVERIS_OP_GEMM
 * (l, m, n, 0). */
averis_status_t averis_gemm_fwd(const averis_nvfp4_t* xr, const averis_nvfp4_t* mean,
                                const averis_nvfp4_t* wt, void* y, averis_dtype_t ydtype,
                                int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream);

/* Dgrad: dx (dr->rows x w->rows) = 1 (mean_d W^T) + D_R W^T with
 *   dr:     Q4(D - 1 mu_D), l x n
 *   mean_d: Q4(mu_D), 1 x n
 *   w:      Q4(W), m x n (blocks along n)
 * Same kernel as the forward; only the quantized copy of W differs. */
averis_status_t averis_gemm_dgrad(const averis_nvfp4_t* dr, const averis_nvfp4_t* mean_d,
                                  const averis_nvfp4_t* w, void* dx, averis_dtype_t dxdtype,
                                  int64_t lddx, void* ws, size_t ws_bytes, hipStream_t stream);

/* The rank-one row formed once, by the split ([Lighthouse] §2.2: the term
 * 1(mu_bar W_bar) is a row vector added to every output row).
 * averis_split_quant_rank1 is averis_split_quant (bit for bit the same
 * residual, mean and mean_f32) that also writes
 *   rho[j] = deq(mean) . deq(b_j),  j < b->rows,
 * for the B operand of the GEMM that will take this split (wt for the
 * forward, w for dgrad: b->cols == cols), fp32 accumulation of exact
 * products, times the two tensor scales.  rho: device float[b->rows], 4-byte
 * aligned.  cols <= 32768 (the dequantized mean is staged in on-chip memory).
 * Workspace: AVERIS_OP_SPLIT_QUANT (rows, cols, 0, 0).
 * averis_gemm_rank1 then computes c = deq(a) deq(b)^T + 1 rho^T (a: the
 * residual, b as above) with no mean row of its own; it equals averis_gemm_fwd
 * / averis_gemm_dgrad of the same operands up to fp32 summation order.  No
 * workspace. */
averis_status_t averis_split_quant_rank1(const void* a, averis_dtype_t dtype, int64_t rows,
                                         int64_t cols, int64_t lda, uint64_t seed,
                                         averis_round_t rnd, const averis_nvfp4_t* residual,
                                         const averis_nvfp4_t* mean, float* mean_f32,
                                         const averis_nvfp4_t* b, float* rho, void* ws,
                                         size_t ws_bytes, hipStream_t stream);
averis_status_t averis_gemm_rank1(const averis_nvfp4_t* a, const float* rho,
                                  const averis_nvfp4_t* b, void* c, averis_dtype_t cdtype,
                                  int64_t ldc, hipStream_t stream);

/* The rank-one rows of several GEMMs that take the same split (the
 * projections that read one input, e.g. q, k and v of a transformer block;
 * [Lighthouse] §2.2 as above): averis_split_quant_rank1 with nb B operands
 * (1 <= nb <= AVERIS_MAX_RANK1), b[i]->cols == cols, writing
 *   rho[i][j] = deq(mean) . deq(b[i]_j),  j < b[i]->rows,
 * each bit for bit the row averis_split_quant_rank1 with b[i] alone writes,
 * and the same residual, mean and mean_f32.  b, rho: host arrays of nb
 * pointers (descriptors of device tensors; device float[b[i]->rows], 4-byte
 * aligned), read during the call only.  Workspace as averis_split_quant_rank1.
 * Errors as averis_split_quant_rank1, for any entry. */
#define AVERIS_MAX_RANK1 4
averis_status_t averis_split_quant_rank1_multi(const void* a, averis_dtype_t dtype, int64_t rows,
                                               int64_t cols, int64_t lda, uint64_t seed,
                                               averis_round_t rnd, const averis_nvfp4_t* residual,
                                               const averis_nvfp4_t* mean, float* mean_f32,
                                               int nb, const averis_nvfp4_t* const* b,
                                               float* const* rho, void* ws, size_t ws_bytes,
                                               hipStream_t stream);

/* Grouped forms (expert segments, as averis_split_quant_grouped and
 * averis_gemm_grouped): b holds nseg stacked N x cols matrices (expert s =
 * rows s*N .. s*N+N-1, its own tensor scale b->tscale[2s..2s+1]) and
 *   rho[s*N + j] = deq(mean_s) . deq(b_s,j)   (device float[nseg*N]);
 * an empty segment has mean 0 and so rho_s = 0.  averis_gemm_grouped_rank1:
 * c[rows of s] = deq(a_s) deq(b_s)^T + 1 rho_s^T. */
averis_status_t averis_split_quant_grouped_rank1(const void* a, averis_dtype_t dtype,
                                                 int64_t rows, int64_t cols, int64_t lda,
                                                 const int64_t* seg_offsets, int nseg,
                                                 uint64_t seed, averis_round_t rnd,
                                                 const averis_nvfp4_t* residual,
                                                 const averis_nvfp4_t* mean, float* mean_f32,
                                                 const averis_nvfp4_t* b, float* rho, void* ws,
                                                 size_t ws_bytes, hipStream_t stream);
averis_status_t averis_gemm_grouped_rank1(const averis_nvfp4_t* a, const float* rho,
                                          const averis_nvfp4_t* b, const int64_t* seg_offsets,
                                          int nseg, void* c, averis_dtype_t cdtype, int64_t ldc,
                                          hipStream_t stream);

/* Vanilla arm: c = deq(a) deq(b)^T, no mean term. */
averis_status_t averis_gemm_vanilla(const averis_nvfp4_t* a, const averis_nvfp4_t* b, void* c,
                                    averis_dtype_t cdtype, int64_t ldc, void* ws, size_t ws_bytes,
                                    hipStream_t stream);

/* Grouped GEMM: for each segment s (rows seg_offsets[s] .. [s+1]-1 of a),
 * c[rows of s] = deq(a_s) deq(b_s)^T (+ 1 deq(mean_s) deq(b_s)^T), where
 * b is (nseg * N) x K (expert s = rows s*N .. s*N+N-1, its own tensor scale
 * b->tscale[2s..2s+1]), a->tscale and mean->tscale hold 2*nseg floats,
 * mean is nseg x K or NULL (vanilla).  Workspace: AVERIS_OP_GEMM with nseg. */
averis_status_t averis_gemm_grouped(const averis_nvfp4_t* a, const averis_nvfp4_t* mean,
                                    const averis_nvfp4_t* b, const int64_t* seg_offsets, int nseg,
                                    void* c, averis_dtype_t cdtype, int64_t ldc, void* ws,
                                    size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* wgrad (the W4A4G4 setting of the arXiv abstract and Lighthouse §3.1    */
/* keeps weights, activations and gradients in FP4; §2.2 writes out only   */
/* the forward and dgrad products).  Reading: the split applied to both    */
/* operands of                                                             */
/* dW = X^T D.  The residuals' column sums vanish, so                      */
/*   dW = deq(Q4(X_R^T)) deq(Q4(D_R^T))^T + l mu_X mu_D^T,                 */
/* with the transposed residuals quantized in 16-blocks along the tokens   */
/* (the contraction axis of this product) and the outer product taken from */
/* the fp32 means (no contraction runs over them).                         */
/* ---------------------------------------------------------------------- */

/* out_t = Q4((a - 1 mu)^T): cols x rows, 16-blocks along the rows (tokens),
 * SR stream 3, element index col * rows + row.  a: rows x cols (F32 or BF16,
 * row stride lda, as for averis_split_quant); rows % 16 == 0 (rows may be 0).
 * mu: the fp32 column means averis_split_quant wrote for the same a (cols
 * floats, device, 16-byte aligned).  residual_tscale: the residual tensor's
 * [S_enc, S_dec] from that call (device, 2 floats); the transposed residual
 * holds the same values and takes the same tensor scale, copied to
 * out_t->tscale.  No workspace.  Other arguments as for averis_split_quant. */
averis_status_t averis_residual_t_quant(const void* a, averis_dtype_t dtype, int64_t rows,
                                        int64_t cols, int64_t lda, const float* mu,
                                        const float* residual_tscale, uint64_t seed,
                                        averis_round_t rnd, const averis_nvfp4_t* out_t,
                                        hipStream_t stream);

/* dw (m x n, F32 or BF16, row stride lddw >= n) =
 *   deq(xt) deq(dt)^T + l mu_x mu_d^T
 * with xt = Q4(X_R^T) (m x l) and dt = Q4(D_R^T) (n x l) from
 * averis_residual_t_quant, mu_x (m floats) and mu_d (n floats) the fp32
 * means of X and D (device, 16-byte aligned); m, n, l multiples of 16 (l may
 * be 0: dw = l mu_x mu_d^T = 0).  FP32 accumulation; the token axis is split
 * into fp32 partials that are summed in a fixed order, so repeated calls
 * give the same bits.  Workspace: averis_workspace_bytes(AVERIS_OP_WGRAD,
 * m, l, n, 0). */
averis_status_t averis_gemm_wgrad(const averis_nvfp4_t* xt, const averis_nvfp4_t* dt,
                                  const float* mu_x, const float* mu_d, void* dw,
                                  averis_dtype_t dwdtype, int64_t lddw, void* ws, size_t ws_bytes,
                                  hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Column statistics fused into the producer (Lighthouse §2.2 cost note:   */
/* the split adds two column reductions and two subtractions; §4.2: it     */
/* changes the quantization kernel's pre-processing).  The GEMM that makes */
/* the next split's input gathers that input's column statistics in its   */
/* epilogue, so the split reads its input once.                            */
/* ---------------------------------------------------------------------- */

/* averis_gemm_rank1 with bf16 output c (n = b->rows columns, row stride ldc)
 * that also writes the column statistics of c, as stored, into ws: per
 * 256-row tile and column, the fp64 sum, max, min and smallest nonzero
 * magnitude.  ws is the split-quant workspace of c:
 * averis_workspace_bytes(AVERIS_OP_SPLIT_QUANT, a->rows, n, 0, 0) bytes, to
 * be passed unchanged to averis_split_quant_from_stats for this c (nothing
 * else may use it in between).  Needs a->cols % 64 == 0, n % 16 == 0, c
 * 16-byte aligned and ldc * 2 % 16 == 0 (c is then a valid split input).
 * c equals averis_gemm_rank1's bf16 output bit for bit. */
averis_status_t averis_gemm_rank1_stats(const averis_nvfp4_t* a, const float* rho,
                                        const averis_nvfp4_t* b, void* c, int64_t ldc, void* ws,
                                        size_t ws_bytes, hipStream_t stream);

/* averis_split_quant of the bf16 rows x cols tensor a (row stride lda) from
 * the column statistics that averis_gemm_rank1_stats wrote into ws when it
 * produced a: the mean, the tensor scales and the quantized outputs are
 * averis_split_quant's bit for bit, and a is read once (by the quant pass;
 * a column whose sum is not certified exact is re-summed from its tiles'
 * partials and, for a tile not exact on its own, from its rows).  b and rho:
 * both NULL, or the rank-one row of the GEMM that takes this split, as for
 * averis_split_quant_rank1.  Order this call after that GEMM (same stream). */
averis_status_t averis_split_quant_from_stats(const void* a, int64_t rows, int64_t cols,
                                              int64_t lda, uint64_t seed, averis_round_t rnd,
                                              const averis_nvfp4_t* residual,
                                              const averis_nvfp4_t* mean, float* mean_f32,
                                              const averis_nvfp4_t* b, float* rho, void* ws,
                                              size_t ws_bytes, hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Allocation-free split-quant                                             */
/* ---------------------------------------------------------------------- */

/* Bytes of the device array that averis_split_quant_noalloc uses as its
 * workspace (one copy per device). */
#define AVERIS_NOALLOC_SCRATCH_BYTES ((size_t)16 << 20)

/* For callers that cannot allocate device memory or pass a workspace: code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc.  averis_split_quant with the same arguments and results, bit for
 * bit, whose workspace is a file-scope device array of
 * AVERIS_NOALLOC_SCRATCH_BYTES inside the library: the call allocates
 * nothing.  The array holds the split's intermediate results, which depend on
 * the shape: averis_workspace_bytes(AVERIS_OP_SPLIT_QUANT, rows, cols, 0, 0)
 * must not exceed AVERIS_NOALLOC_SCRATCH_BYTES (about rows / 128 * cols * 28
 * bytes: a 16384 x 3072 input fits), else the call returns
 * AVERIS_E_WORKSPACE, enqueues nothing, and averis_last_error() names both
 * sizes.  Every call on one device shares that device's array: calls that
 * overlap on one device (several streams or threads at once) race and give
 * wrong results; order them on one stream.  The first call on a device looks
 * up the array's address there (once; the lookup is not captured). */
averis_status_t averis_split_quant_noalloc(const void* a, averis_dtype_t dtype, int64_t rows,
                                           int64_t cols, int64_t lda, uint64_t seed,
                                           averis_round_t rnd, const averis_nvfp4_t* residual,
                                           const averis_nvfp4_t* mean, float* mean_f32,
                                           hipStream_t stream);

/* ---------------------------------------------------------------------- */
/* Utilities                                                               */
/* ---------------------------------------------------------------------- */

/* Bytes of workspace an entry point needs (0 if none); a bad query returns
 * 0 and the entry point then rejects the call with AVERIS_E_SHAPE. */
size_t averis_workspace_bytes(averis_op_t op, int64_t rows, int64_t cols, int64_t n, int64_t nseg);

/* Static string for a status code. */
const char* averis_status_str(averis_status_t status);

/* AVERIS_ABI_VERSION of the built library. */
int averis_abi_version(void);

/* Text of the last HIP error an entry point on the calling thread returned
 * AVERIS_E_HIP for, or of the size check averis_split_quant_noalloc returned
 * AVERIS_E_WORKSPACE for ("" if none).  The string is owned by the library and is
 * valid until the next call on the same thread. */
const char* averis_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* AVERIS_H */
