// libaveris C ABI: argument validation, workspace carve-up and launches.
// Every check runs before the first HIP call, so a rejected call touches no
// device state and the checks can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstddef>
#include <cstdint>
#include <cstdio>

#include "../../include/averis.h"
#include "launch.hpp"
#include "segments.hpp"

using namespace averis;

namespace {

constexpr int kMaxSeg = 4096;
// the split stages the dequantized mean (2 bytes per column) in LDS to form
// the rank-one row
constexpr int64_t kRank1MaxK = 32768;

inline size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }
inline bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
inline size_t elem_size(averis_dtype_t d) { return d == AVERIS_BF16 ? 2 : 4; }
inline bool dtype_ok(averis_dtype_t d) { return d == AVERIS_F32 || d == AVERIS_BF16; }

averis_status_t check_tensor(const averis_nvfp4_t* t, int64_t rows, int64_t cols) {
  if (!t || !t->tscale) return AVERIS_E_NULL;
  if (t->rows != rows || t->cols != cols) return AVERIS_E_SHAPE;
  if (rows > 0 && cols > 0 && (!t->codes || !t->scales)) return AVERIS_E_NULL;
  if (!aligned(t->codes, 16) || !aligned(t->scales, 16) || !aligned(t->tscale, 4))
    return AVERIS_E_ALIGN;
  return AVERIS_OK;
}

averis_status_t check_input(const void* a, averis_dtype_t dtype, int64_t rows, int64_t cols,
                            int64_t lda, int64_t min_lda) {
  if (!dtype_ok(dtype)) return AVERIS_E_DTYPE;
  if (rows < 0 || cols <= 0 || (cols % 16) != 0) return AVERIS_E_SHAPE;
  if (lda < min_lda) return AVERIS_E_SHAPE;
  if (rows > 0 && !a) return AVERIS_E_NULL;
  if (!aligned(a, 16) || ((size_t)lda * elem_size(dtype)) % 16 != 0) return AVERIS_E_ALIGN;
  return AVERIS_OK;
}

thread_local char g_last_error[256] = "";

inline averis_status_t hip_status(hipError_t e) {
  if (e == hipSuccess) return AVERIS_OK;
  std::snprintf(g_last_error, sizeof(g_last_error), "%s: %s", hipGetErrorName(e),
                hipGetErrorString(e));
  return AVERIS_E_HIP;
}

// ---------------------------------------------------------------------------
// The allocation-free split-quant keeps its workspace in this file-scope
// device array (one copy per device, allocated with the code object).  Host
// code never passes the array's name to a kernel: the name is a host-side
// stand-in, not a device address.  The device address is looked up once per
// device with hipGetSymbolAddress, with that device current, and kept.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = AVERIS_NOALLOC_SCRATCH_BYTES;
__device__ __attribute__((aligned(256))) unsigned char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

hipError_t scratch_address(void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (!p) {
    // concurrent first calls on one device look up the same address
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch[dev].store(p, std::memory_order_release);
  }
  *out = p;
  return hipSuccess;
}

}  // namespace

namespace averis {

size_t split_ws_bytes(int64_t rows, int64_t cols, int nseg) {
  const int ns = nseg > 0 ? nseg : 1;
  const int64_t nch = chunk_upper_bound(rows, nseg > 0 ? nseg : 1, kStatsRows);
  const int64_t ct_s = (cols + kPlainStatsCols - 1) / kPlainStatsCols,
                ct_f = (cols + kFinCols - 1) / kFinCols;
  size_t b = 0;
  b += align256((size_t)(nch * cols * 8));      // psum
  b += align256((size_t)(nch * cols * 4)) * 3;  // pmax, pmin, pmnz
  b += align256((size_t)(nch * ct_s * 4));      // pamax
  b += align256((size_t)(ns * cols * 4));       // mu
  b += align256((size_t)(ns * (ct_f > 1 ? ct_f : 1) * 4)) * 2;  // tmax_r, tmax_mu
  b += align256((size_t)(nch * cols * 8));      // psq
  b += align256((size_t)(ns * (ct_f > 1 ? ct_f : 1) * 8)) * 2;  // tssq, tmu2
  return b;
}

SplitWs split_ws_carve(void* ws, int64_t rows, int64_t cols, int nseg) {
  const int ns = nseg > 0 ? nseg : 1;
  const int64_t nch = chunk_upper_bound(rows, nseg > 0 ? nseg : 1, kStatsRows);
  const int64_t ct_s = (cols + kPlainStatsCols - 1) / kPlainStatsCols,
                ct_f = (cols + kFinCols - 1) / kFinCols;
  char* p = static_cast<char*>(ws);
  SplitWs w;
  w.psum = reinterpret_cast<double*>(p); p += align256((size_t)(nch * cols * 8));
  w.pmax = reinterpret_cast<float*>(p);  p += align256((size_t)(nch * cols * 4));
  w.pmin = reinterpret_cast<float*>(p);  p += align256((size_t)(nch * cols * 4));
  w.pmnz = reinterpret_cast<float*>(p);  p += align256((size_t)(nch * cols * 4));
  w.pamax = reinterpret_cast<float*>(p); p += align256((size_t)(nch * ct_s * 4));
  w.mu = reinterpret_cast<float*>(p);    p += align256((size_t)(ns * cols * 4));
  w.tmax_r = reinterpret_cast<float*>(p); p += align256((size_t)(ns * (ct_f > 1 ? ct_f : 1) * 4));
  w.tmax_mu = reinterpret_cast<float*>(p); p += align256((size_t)(ns * (ct_f > 1 ? ct_f : 1) * 4));
  w.psq = reinterpret_cast<double*>(p);  p += align256((size_t)(nch * cols * 8));
  w.tssq = reinterpret_cast<double*>(p); p += align256((size_t)(ns * (ct_f > 1 ? ct_f : 1) * 8));
  w.tmu2 = reinterpret_cast<double*>(p);
  return w;
}

size_t batched_ws_bytes(int64_t, int64_t, int batch) {
  return align256((size_t)(batch > 0 ? batch : 1) * (size_t)kAmaxBlocks * 4);
}

}  // namespace averis

extern "C" {

size_t averis_workspace_bytes(averis_op_t op, int64_t rows, int64_t cols, int64_t n, int64_t nseg) {
  if (op == AVERIS_OP_QUANT_PAIR_MULTI)
    return (n >= 1 && n <= kMaxWeights) ? (size_t)n * kAmaxBlocks * sizeof(float) : 0;
  if (op == AVERIS_OP_WGRAD) {
    // cols = l may be 0 (no tokens)
    if (rows < 0 || cols < 0 || cols % 16 != 0 || n < 0) return 0;
    return wgrad_ws_bytes(rows, n, cols);
  }
  if (rows < 0 || cols <= 0 || cols % 16 != 0 || nseg < 0 || nseg > kMaxSeg) return 0;
  switch (op) {
    case AVERIS_OP_SPLIT_QUANT:
      return split_ws_bytes(rows, cols, (int)nseg);
    case AVERIS_OP_QUANT: {
      const size_t a = split_ws_bytes(rows, cols, (int)nseg);
      const size_t b = batched_ws_bytes(rows, cols, (int)nseg);
      return a > b ? a : b;
    }
    case AVERIS_OP_GEMM:
      if (n < 0) return 0;
      return gemm_ws_bytes(n, cols, (int)nseg);
    case AVERIS_OP_WGRAD:
    case AVERIS_OP_QUANT_PAIR_MULTI:
      break;
  }
  return 0;
}

const char* averis_status_str(averis_status_t s) {
  switch (s) {
    case AVERIS_OK: return "ok";
    case AVERIS_E_NULL: return "a required pointer is NULL";
    case AVERIS_E_SHAPE: return "invalid or mismatched shape";
    case AVERIS_E_DTYPE: return "unsupported dtype";
    case AVERIS_E_ALIGN: return "misaligned pointer or leading dimension";
    case AVERIS_E_WORKSPACE: return "workspace missing or too small";
    case AVERIS_E_ARG: return "invalid argument";
    case AVERIS_E_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

int averis_abi_version(void) { return AVERIS_ABI_VERSION; }

const char* averis_last_error(void) { return g_last_error; }

static averis_status_t split_common(const void* a, averis_dtype_t dtype, int64_t rows,
                                    int64_t cols, int64_t lda, const int64_t* offs, int nseg,
                                    uint64_t seed, averis_round_t rnd,
                                    const averis_nvfp4_t* residual, const averis_nvfp4_t* mean,
                                    float* mean_f32, void* ws, size_t ws_bytes,
                                    hipStream_t stream, float* ratio = nullptr,
                                    const Rank1Out* r1 = nullptr) {
  averis_status_t s = check_input(a, dtype, rows, cols, lda, cols);
  if (s != AVERIS_OK) return s;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (nseg < 1 || nseg > kMaxSeg) return AVERIS_E_ARG;
  if ((s = check_tensor(residual, rows, cols)) != AVERIS_OK) return s;
  if ((s = check_tensor(mean, offs ? nseg : 1, cols)) != AVERIS_OK) return s;
  if (!aligned(mean_f32, 4)) return AVERIS_E_ALIGN;
  const size_t need = split_ws_bytes(rows, cols, nseg);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const SplitWs w = split_ws_carve(ws, rows, cols, nseg);
  const QuantOut ro{residual->codes, residual->scales, residual->tscale};
  const QuantOut mo{mean->codes, mean->scales, mean->tscale};
  return hip_status(launch_split_or_plain(a, dtype == AVERIS_BF16, rows, cols, lda, offs, nseg,
                                          true, rnd == AVERIS_SR, seed, 0u, ro, &mo, mean_f32, w,
                                          stream, ratio, r1));
}

averis_status_t averis_split_quant(const void* a, averis_dtype_t dtype, int64_t rows, int64_t cols,
                                   int64_t lda, uint64_t seed, averis_round_t rnd,
                                   const averis_nvfp4_t* residual, const averis_nvfp4_t* mean,
                                   float* mean_f32, void* ws, size_t ws_bytes,
                                   hipStream_t stream) {
  return split_common(a, dtype, rows, cols, lda, nullptr, 1, seed, rnd, residual, mean, mean_f32,
                      ws, ws_bytes, stream);
}

averis_status_t averis_split_quant_grouped(const void* a, averis_dtype_t dtype, int64_t rows,
                                           int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                           int nseg, uint64_t seed, averis_round_t rnd,
                                           const averis_nvfp4_t* residual,
                                           const averis_nvfp4_t* mean, float* mean_f32, void* ws,
                                           size_t ws_bytes, hipStream_t stream) {
  if (!seg_offsets) return AVERIS_E_NULL;
  if (!aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return split_common(a, dtype, rows, cols, lda, seg_offsets, nseg, seed, rnd, residual, mean,
                      mean_f32, ws, ws_bytes, stream);
}

averis_status_t averis_split_quant_ratio(const void* a, averis_dtype_t dtype, int64_t rows,
                                         int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                         int nseg, uint64_t seed, averis_round_t rnd,
                                         const averis_nvfp4_t* residual,
                                         const averis_nvfp4_t* mean, float* mean_f32, float* ratio,
                                         void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!ratio) return AVERIS_E_NULL;
  if (!aligned(ratio, 4)) return AVERIS_E_ALIGN;
  if (!seg_offsets && nseg != 1) return AVERIS_E_ARG;
  if (seg_offsets && !aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return split_common(a, dtype, rows, cols, lda, seg_offsets, nseg, seed, rnd, residual, mean,
                      mean_f32, ws, ws_bytes, stream, ratio);
}

static averis_status_t split_rank1_common(const void* a, averis_dtype_t dtype, int64_t rows,
                                          int64_t cols, int64_t lda, const int64_t* offs,
                                          int nseg, uint64_t seed, averis_round_t rnd,
                                          const averis_nvfp4_t* residual,
                                          const averis_nvfp4_t* mean, float* mean_f32,
                                          const averis_nvfp4_t* b, float* rho, void* ws,
                                          size_t ws_bytes, hipStream_t stream) {
  if (!b || !rho) return AVERIS_E_NULL;
  if (!aligned(rho, 4)) return AVERIS_E_ALIGN;
  if (cols > kRank1MaxK) return AVERIS_E_SHAPE;
  if (nseg < 1 || nseg > kMaxSeg) return AVERIS_E_ARG;
  averis_status_t s = check_tensor(b, b->rows, cols);
  if (s != AVERIS_OK) return s;
  const int64_t ns = offs ? nseg : 1;
  if (b->rows <= 0 || b->rows % ns != 0) return AVERIS_E_SHAPE;
  const Rank1Out r1 = rank1_one(QOperand{b->codes, b->scales, b->tscale}, b->rows / ns, rho);
  return split_common(a, dtype, rows, cols, lda, offs, nseg, seed, rnd, residual, mean, mean_f32,
                      ws, ws_bytes, stream, nullptr, &r1);
}

averis_status_t averis_split_quant_rank1(const void* a, averis_dtype_t dtype, int64_t rows,
                                         int64_t cols, int64_t lda, uint64_t seed,
                                         averis_round_t rnd, const averis_nvfp4_t* residual,
                                         const averis_nvfp4_t* mean, float* mean_f32,
                                         const averis_nvfp4_t* b, float* rho, void* ws,
                                         size_t ws_bytes, hipStream_t stream) {
  return split_rank1_common(a, dtype, rows, cols, lda, nullptr, 1, seed, rnd, residual, mean,
                            mean_f32, b, rho, ws, ws_bytes, stream);
}

static_assert(AVERIS_MAX_RANK1 == kMaxRank1, "rank-one operands per split");

averis_status_t averis_split_quant_rank1_multi(const void* a, averis_dtype_t dtype, int64_t rows,
                                               int64_t cols, int64_t lda, uint64_t seed,
                                               averis_round_t rnd, const averis_nvfp4_t* residual,
                                               const averis_nvfp4_t* mean, float* mean_f32,
                                               int nb, const averis_nvfp4_t* const* b,
                                               float* const* rho, void* ws, size_t ws_bytes,
                                               hipStream_t stream) {
  if (!b || !rho) return AVERIS_E_NULL;
  if (nb < 1 || nb > kMaxRank1) return AVERIS_E_ARG;
  if (cols > kRank1MaxK) return AVERIS_E_SHAPE;
  Rank1Out r1{};
  for (int i = 0; i < nb; ++i) {
    if (!b[i] || !rho[i]) return AVERIS_E_NULL;
    if (!aligned(rho[i], 4)) return AVERIS_E_ALIGN;
    const averis_status_t s = check_tensor(b[i], b[i]->rows, cols);
    if (s != AVERIS_OK) return s;
    if (b[i]->rows <= 0) return AVERIS_E_SHAPE;
    r1.b[i] = QOperand{b[i]->codes, b[i]->scales, b[i]->tscale};
    r1.n[i] = b[i]->rows;
    r1.rho[i] = rho[i];
  }
  r1.count = nb;
  return split_common(a, dtype, rows, cols, lda, nullptr, 1, seed, rnd, residual, mean, mean_f32,
                      ws, ws_bytes, stream, nullptr, &r1);
}

averis_status_t averis_split_quant_grouped_rank1(const void* a, averis_dtype_t dtype,
                                                 int64_t rows, int64_t cols, int64_t lda,
                                                 const int64_t* seg_offsets, int nseg,
                                                 uint64_t seed, averis_round_t rnd,
                                                 const averis_nvfp4_t* residual,
                                                 const averis_nvfp4_t* mean, float* mean_f32,
                                                 const averis_nvfp4_t* b, float* rho, void* ws,
                                                 size_t ws_bytes, hipStream_t stream) {
  if (!seg_offsets) return AVERIS_E_NULL;
  if (!aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return split_rank1_common(a, dtype, rows, cols, lda, seg_offsets, nseg, seed, rnd, residual,
                            mean, mean_f32, b, rho, ws, ws_bytes, stream);
}

static averis_status_t gemm_rank1_common(const averis_nvfp4_t* a, const float* rho,
                                         const averis_nvfp4_t* b, const int64_t* offs, int nseg,
                                         void* c, averis_dtype_t cdtype, int64_t ldc,
                                         hipStream_t stream) {
  if (!a || !b || !rho) return AVERIS_E_NULL;
  if (!dtype_ok(cdtype)) return AVERIS_E_DTYPE;
  if (nseg < 1 || nseg > kMaxSeg) return AVERIS_E_ARG;
  const int64_t m = a->rows, k = a->cols;
  const int64_t ns = offs ? nseg : 1;
  if (m < 0 || k <= 0 || k % 16 != 0 || b->cols != k) return AVERIS_E_SHAPE;
  if (b->rows < 0 || b->rows % ns != 0) return AVERIS_E_SHAPE;
  const int64_t n = b->rows / ns;
  averis_status_t s;
  if ((s = check_tensor(a, m, k)) != AVERIS_OK) return s;
  if ((s = check_tensor(b, b->rows, k)) != AVERIS_OK) return s;
  if (!aligned(rho, 4)) return AVERIS_E_ALIGN;
  if (ldc < n) return AVERIS_E_SHAPE;
  if (m > 0 && n > 0 && !c) return AVERIS_E_NULL;
  if (!aligned(c, elem_size(cdtype))) return AVERIS_E_ALIGN;
  const QOperand qa{a->codes, a->scales, a->tscale};
  const QOperand qb{b->codes, b->scales, b->tscale};
  return hip_status(launch_gemm_rho(qa, rho, qb, m, n, k, offs, nseg, c, cdtype == AVERIS_BF16, ldc,
                                    stream));
}

averis_status_t averis_gemm_rank1(const averis_nvfp4_t* a, const float* rho,
                                  const averis_nvfp4_t* b, void* c, averis_dtype_t cdtype,
                                  int64_t ldc, hipStream_t stream) {
  return gemm_rank1_common(a, rho, b, nullptr, 1, c, cdtype, ldc, stream);
}

averis_status_t averis_gemm_grouped_rank1(const averis_nvfp4_t* a, const float* rho,
                                          const averis_nvfp4_t* b, const int64_t* seg_offsets,
                                          int nseg, void* c, averis_dtype_t cdtype, int64_t ldc,
                                          hipStream_t stream) {
  if (!seg_offsets) return AVERIS_E_NULL;
  if (!aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return gemm_rank1_common(a, rho, b, seg_offsets, nseg, c, cdtype, ldc, stream);
}

static averis_status_t quant_common(const void* a, averis_dtype_t dtype, int64_t rows,
                                    int64_t cols, int64_t lda, const int64_t* offs, int nseg,
                                    uint64_t seed, averis_round_t rnd, uint32_t sr_stream,
                                    const averis_nvfp4_t* out, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  averis_status_t s = check_input(a, dtype, rows, cols, lda, cols);
  if (s != AVERIS_OK) return s;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (sr_stream > 0xFFFFu || nseg < 1 || nseg > kMaxSeg) return AVERIS_E_ARG;
  if ((s = check_tensor(out, rows, cols)) != AVERIS_OK) return s;
  const size_t need = split_ws_bytes(rows, cols, nseg);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const SplitWs w = split_ws_carve(ws, rows, cols, nseg);
  const QuantOut o{out->codes, out->scales, out->tscale};
  return hip_status(launch_split_or_plain(a, dtype == AVERIS_BF16, rows, cols, lda, offs, nseg,
                                          false, rnd == AVERIS_SR, seed, sr_stream, o, nullptr,
                                          nullptr, w, stream));
}

averis_status_t averis_quant_batched(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                     int64_t cols, int64_t lda, int64_t batch_stride,
                                     int transpose, uint64_t seed, averis_round_t rnd,
                                     uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return AVERIS_E_DTYPE;
  if (batch < 1 || batch > kMaxSeg) return AVERIS_E_ARG;
  if (transpose != 0 && transpose != 1) return AVERIS_E_ARG;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (sr_stream > 0xFFFFu) return AVERIS_E_ARG;
  if (rows < 0 || cols <= 0 || cols % 16 != 0) return AVERIS_E_SHAPE;
  const int64_t scols = transpose ? rows : cols, srows = transpose ? cols : rows;
  if (lda < scols || batch_stride < 0) return AVERIS_E_SHAPE;
  if (batch > 1 && batch_stride < srows * lda) return AVERIS_E_SHAPE;
  if (rows > 0 && !a) return AVERIS_E_NULL;
  if (!aligned(a, elem_size(dtype))) return AVERIS_E_ALIGN;
  averis_status_t s = check_tensor(out, (int64_t)batch * rows, cols);
  if (s != AVERIS_OK) return s;
  const size_t need = batched_ws_bytes(rows, cols, batch);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const QuantOut o{out->codes, out->scales, out->tscale};
  return hip_status(launch_quant_batched(a, dtype == AVERIS_BF16, batch, rows, cols, lda,
                                         batch_stride, transpose, rnd == AVERIS_SR, seed,
                                         sr_stream, o, static_cast<float*>(ws), stream));
}

averis_status_t averis_quant(const void* a, averis_dtype_t dtype, int64_t rows, int64_t cols,
                             int64_t lda, int transpose, uint64_t seed, averis_round_t rnd,
                             uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                             size_t ws_bytes, hipStream_t stream) {
  if (transpose == 1)
    return averis_quant_batched(a, dtype, 1, rows, cols, lda, 0, 1, seed, rnd, sr_stream, out, ws,
                                ws_bytes, stream);
  if (transpose != 0) return AVERIS_E_ARG;
  return quant_common(a, dtype, rows, cols, lda, nullptr, 1, seed, rnd, sr_stream, out, ws,
                      ws_bytes, stream);
}

averis_status_t averis_quant_grouped(const void* a, averis_dtype_t dtype, int64_t rows,
                                     int64_t cols, int64_t lda, const int64_t* seg_offsets,
                                     int nseg, uint64_t seed, averis_round_t rnd,
                                     uint32_t sr_stream, const averis_nvfp4_t* out, void* ws,
                                     size_t ws_bytes, hipStream_t stream) {
  if (!seg_offsets) return AVERIS_E_NULL;
  if (!aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return quant_common(a, dtype, rows, cols, lda, seg_offsets, nseg, seed, rnd, sr_stream, out, ws,
                      ws_bytes, stream);
}

static averis_status_t pair_common(bool tiles2d, const void* a, averis_dtype_t dtype, int batch,
                                   int64_t rows, int64_t cols, int64_t lda, int64_t batch_stride,
                                   uint64_t seed, averis_round_t rnd, uint32_t sr_stream,
                                   const averis_nvfp4_t* out, const averis_nvfp4_t* out_t,
                                   void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!dtype_ok(dtype)) return AVERIS_E_DTYPE;
  if (batch < 1 || batch > kMaxSeg) return AVERIS_E_ARG;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (sr_stream > 0xFFFFu) return AVERIS_E_ARG;
  if (rows <= 0 || cols <= 0 || rows % 16 != 0 || cols % 16 != 0) return AVERIS_E_SHAPE;
  if (lda < cols || batch_stride < 0) return AVERIS_E_SHAPE;
  if (batch > 1 && batch_stride < rows * lda) return AVERIS_E_SHAPE;
  if (!a) return AVERIS_E_NULL;
  const size_t es = elem_size(dtype);
  if (!aligned(a, 16) || ((size_t)lda * es) % 16 != 0 || ((size_t)batch_stride * es) % 16 != 0)
    return AVERIS_E_ALIGN;
  averis_status_t s = check_tensor(out, (int64_t)batch * rows, cols);
  if (s != AVERIS_OK) return s;
  if ((s = check_tensor(out_t, (int64_t)batch * cols, rows)) != AVERIS_OK) return s;
  const size_t need = batched_ws_bytes(rows, cols, batch);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const QuantOut o{out->codes, out->scales, out->tscale};
  const QuantOut ot{out_t->codes, out_t->scales, out_t->tscale};
  if (tiles2d)
    return hip_status(launch_quant_pair2d(a, dtype == AVERIS_BF16, batch, rows, cols, lda,
                                          batch_stride, rnd == AVERIS_SR, seed, sr_stream, o, ot,
                                          static_cast<float*>(ws), stream));
  return hip_status(launch_quant_pair(a, dtype == AVERIS_BF16, batch, rows, cols, lda,
                                      batch_stride, rnd == AVERIS_SR, seed, sr_stream, o, ot,
                                      static_cast<float*>(ws), stream));
}

averis_status_t averis_quant_pair(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                  int64_t cols, int64_t lda, int64_t batch_stride, uint64_t seed,
                                  averis_round_t rnd, uint32_t sr_stream,
                                  const averis_nvfp4_t* out, const averis_nvfp4_t* out_t,
                                  void* ws, size_t ws_bytes, hipStream_t stream) {
  return pair_common(false, a, dtype, batch, rows, cols, lda, batch_stride, seed, rnd, sr_stream,
                     out, out_t, ws, ws_bytes, stream);
}

averis_status_t averis_quant_pair_2d(const void* a, averis_dtype_t dtype, int batch, int64_t rows,
                                     int64_t cols, int64_t lda, int64_t batch_stride,
                                     uint64_t seed, averis_round_t rnd, uint32_t sr_stream,
                                     const averis_nvfp4_t* out, const averis_nvfp4_t* out_t,
                                     void* ws, size_t ws_bytes, hipStream_t stream) {
  return pair_common(true, a, dtype, batch, rows, cols, lda, batch_stride, seed, rnd, sr_stream,
                     out, out_t, ws, ws_bytes, stream);
}

static_assert(AVERIS_MAX_WEIGHTS == kMaxWeights, "weights per multi-weight call");

averis_status_t averis_quant_pair_multi(int n, const averis_weight_t* w, averis_dtype_t dtype,
                                        averis_round_t rnd, uint32_t sr_stream, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  if (!w) return AVERIS_E_NULL;
  if (n < 1 || n > kMaxWeights) return AVERIS_E_ARG;
  if (!dtype_ok(dtype)) return AVERIS_E_DTYPE;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (sr_stream > 0xFFFFu) return AVERIS_E_ARG;
  const size_t es = elem_size(dtype);
  WeightPair wp[kMaxWeights];
  for (int i = 0; i < n; ++i) {
    const averis_weight_t& e = w[i];
    if (e.rows <= 0 || e.cols <= 0 || e.rows % 16 != 0 || e.cols % 16 != 0)
      return AVERIS_E_SHAPE;
    if (e.lda < e.cols) return AVERIS_E_SHAPE;
    if (!e.a) return AVERIS_E_NULL;
    if (!aligned(e.a, 16) || ((size_t)e.lda * es) % 16 != 0) return AVERIS_E_ALIGN;
    averis_status_t s = check_tensor(e.out, e.rows, e.cols);
    if (s != AVERIS_OK) return s;
    if ((s = check_tensor(e.out_t, e.cols, e.rows)) != AVERIS_OK) return s;
    wp[i] = WeightPair{e.a, e.rows, e.cols, e.lda, e.seed,
                       QuantOut{e.out->codes, e.out->scales, e.out->tscale},
                       QuantOut{e.out_t->codes, e.out_t->scales, e.out_t->tscale}};
  }
  const size_t need = (size_t)n * kAmaxBlocks * sizeof(float);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  return hip_status(launch_quant_pair_multi(n, wp, dtype == AVERIS_BF16, rnd == AVERIS_SR,
                                            sr_stream, static_cast<float*>(ws), stream));
}

static averis_status_t gemm_common(const averis_nvfp4_t* a, const averis_nvfp4_t* mean,
                                   const averis_nvfp4_t* b, const int64_t* offs, int nseg,
                                   void* c, averis_dtype_t cdtype, int64_t ldc, void* ws,
                                   size_t ws_bytes, hipStream_t stream) {
  if (!a || !b) return AVERIS_E_NULL;
  if (!dtype_ok(cdtype)) return AVERIS_E_DTYPE;
  if (nseg < 1 || nseg > kMaxSeg) return AVERIS_E_ARG;
  const int64_t m = a->rows, k = a->cols;
  if (m < 0 || k <= 0 || k % 16 != 0 || b->cols != k) return AVERIS_E_SHAPE;
  const int64_t ns = offs ? nseg : 1;
  if (b->rows < 0 || b->rows % ns != 0) return AVERIS_E_SHAPE;
  const int64_t n = b->rows / ns;
  averis_status_t s;
  if ((s = check_tensor(a, m, k)) != AVERIS_OK) return s;
  if ((s = check_tensor(b, b->rows, k)) != AVERIS_OK) return s;
  if (mean && (s = check_tensor(mean, ns, k)) != AVERIS_OK) return s;
  if (ldc < n) return AVERIS_E_SHAPE;
  if (m > 0 && n > 0 && !c) return AVERIS_E_NULL;
  if (!aligned(c, elem_size(cdtype))) return AVERIS_E_ALIGN;
  const size_t need = mean ? gemm_ws_bytes(n, k, (int)ns) : 0;
  if (need && (!ws || ws_bytes < need)) return AVERIS_E_WORKSPACE;
  if (ws && !aligned(ws, 256)) return AVERIS_E_ALIGN;
  const QOperand qa{a->codes, a->scales, a->tscale};
  const QOperand qb{b->codes, b->scales, b->tscale};
  QOperand qm{};
  if (mean) qm = QOperand{mean->codes, mean->scales, mean->tscale};
  return hip_status(launch_gemm(qa, mean ? &qm : nullptr, qb, m, n, k, offs, nseg, c,
                                cdtype == AVERIS_BF16, ldc, ws, stream));
}

averis_status_t averis_gemm_fwd(const averis_nvfp4_t* xr, const averis_nvfp4_t* mean,
                                const averis_nvfp4_t* wt, void* y, averis_dtype_t ydtype,
                                int64_t ldy, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!mean) return AVERIS_E_NULL;
  return gemm_common(xr, mean, wt, nullptr, 1, y, ydtype, ldy, ws, ws_bytes, stream);
}

averis_status_t averis_gemm_dgrad(const averis_nvfp4_t* dr, const averis_nvfp4_t* mean_d,
                                  const averis_nvfp4_t* w, void* dx, averis_dtype_t dxdtype,
                                  int64_t lddx, void* ws, size_t ws_bytes, hipStream_t stream) {
  if (!mean_d) return AVERIS_E_NULL;
  return gemm_common(dr, mean_d, w, nullptr, 1, dx, dxdtype, lddx, ws, ws_bytes, stream);
}

averis_status_t averis_gemm_vanilla(const averis_nvfp4_t* a, const averis_nvfp4_t* b, void* c,
                                    averis_dtype_t cdtype, int64_t ldc, void* ws, size_t ws_bytes,
                                    hipStream_t stream) {
  return gemm_common(a, nullptr, b, nullptr, 1, c, cdtype, ldc, ws, ws_bytes, stream);
}

averis_status_t averis_gemm_grouped(const averis_nvfp4_t* a, const averis_nvfp4_t* mean,
                                    const averis_nvfp4_t* b, const int64_t* seg_offsets, int nseg,
                                    void* c, averis_dtype_t cdtype, int64_t ldc, void* ws,
                                    size_t ws_bytes, hipStream_t stream) {
  if (!seg_offsets) return AVERIS_E_NULL;
  if (!aligned(seg_offsets, 8)) return AVERIS_E_ALIGN;
  return gemm_common(a, mean, b, seg_offsets, nseg, c, cdtype, ldc, ws, ws_bytes, stream);
}

averis_status_t averis_residual_t_quant(const void* a, averis_dtype_t dtype, int64_t rows,
                                        int64_t cols, int64_t lda, const float* mu,
                                        const float* residual_tscale, uint64_t seed,
                                        averis_round_t rnd, const averis_nvfp4_t* out_t,
                                        hipStream_t stream) {
  averis_status_t s = check_input(a, dtype, rows, cols, lda, cols);
  if (s != AVERIS_OK) return s;
  if (rows % 16 != 0) return AVERIS_E_SHAPE;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if (!mu || !residual_tscale) return AVERIS_E_NULL;
  if (!aligned(mu, 16) || !aligned(residual_tscale, 4)) return AVERIS_E_ALIGN;
  if ((s = check_tensor(out_t, cols, rows)) != AVERIS_OK) return s;
  const QuantOut o{out_t->codes, out_t->scales, out_t->tscale};
  return hip_status(launch_quant_rt(a, dtype == AVERIS_BF16, rows, cols, lda, mu, residual_tscale,
                                    rnd == AVERIS_SR, seed, 3u, o, stream));
}

averis_status_t averis_gemm_wgrad(const averis_nvfp4_t* xt, const averis_nvfp4_t* dt,
                                  const float* mu_x, const float* mu_d, void* dw,
                                  averis_dtype_t dwdtype, int64_t lddw, void* ws, size_t ws_bytes,
                                  hipStream_t stream) {
  if (!xt || !dt || !mu_x || !mu_d) return AVERIS_E_NULL;
  if (!dtype_ok(dwdtype)) return AVERIS_E_DTYPE;
  const int64_t m = xt->rows, n = dt->rows, l = xt->cols;
  if (m < 0 || n < 0 || l < 0 || l % 16 != 0 || dt->cols != l) return AVERIS_E_SHAPE;
  if (m % 16 != 0 || n % 16 != 0) return AVERIS_E_SHAPE;
  averis_status_t s;
  if ((s = check_tensor(xt, m, l)) != AVERIS_OK) return s;
  if ((s = check_tensor(dt, n, l)) != AVERIS_OK) return s;
  if (!aligned(mu_x, 16) || !aligned(mu_d, 16)) return AVERIS_E_ALIGN;
  if (lddw < n) return AVERIS_E_SHAPE;
  if (m > 0 && n > 0 && !dw) return AVERIS_E_NULL;
  if (!aligned(dw, elem_size(dwdtype))) return AVERIS_E_ALIGN;
  const size_t need = wgrad_ws_bytes(m, n, l);
  if (need && (!ws || ws_bytes < need)) return AVERIS_E_WORKSPACE;
  if (ws && !aligned(ws, 256)) return AVERIS_E_ALIGN;
  const QOperand qx{xt->codes, xt->scales, xt->tscale};
  const QOperand qd{dt->codes, dt->scales, dt->tscale};
  return hip_status(launch_wgrad(qx, qd, mu_x, mu_d, m, n, l, dw, dwdtype == AVERIS_BF16, lddw, ws,
                                 stream));
}

averis_status_t averis_gemm_rank1_stats(const averis_nvfp4_t* a, const float* rho,
                                        const averis_nvfp4_t* b, void* c, int64_t ldc, void* ws,
                                        size_t ws_bytes, hipStream_t stream) {
  if (!a || !b || !rho) return AVERIS_E_NULL;
  const int64_t m = a->rows, k = a->cols, n = b->rows;
  // the warp-specialized kernel (K % 64 == 0); c must be a valid split input
  if (m < 0 || k <= 0 || k % 64 != 0 || b->cols != k) return AVERIS_E_SHAPE;
  if (n <= 0 || n % 16 != 0 || ldc < n) return AVERIS_E_SHAPE;
  averis_status_t s;
  if ((s = check_tensor(a, m, k)) != AVERIS_OK) return s;
  if ((s = check_tensor(b, n, k)) != AVERIS_OK) return s;
  if (!aligned(rho, 4)) return AVERIS_E_ALIGN;
  if (m > 0 && !c) return AVERIS_E_NULL;
  if (!aligned(c, 16) || (ldc * 2) % 16 != 0) return AVERIS_E_ALIGN;
  const size_t need = split_ws_bytes(m, n, 1);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const SplitWs w = split_ws_carve(ws, m, n, 1);
  const ColStats cs{w.psum, w.pmax, w.pmin, w.pmnz};
  const QOperand qa{a->codes, a->scales, a->tscale};
  const QOperand qb{b->codes, b->scales, b->tscale};
  return hip_status(launch_gemm_rho_stats(qa, rho, qb, m, n, k, nullptr, 1, c, ldc, cs, stream));
}

averis_status_t averis_split_quant_from_stats(const void* a, int64_t rows, int64_t cols,
                                              int64_t lda, uint64_t seed, averis_round_t rnd,
                                              const averis_nvfp4_t* residual,
                                              const averis_nvfp4_t* mean, float* mean_f32,
                                              const averis_nvfp4_t* b, float* rho, void* ws,
                                              size_t ws_bytes, hipStream_t stream) {
  averis_status_t s = check_input(a, AVERIS_BF16, rows, cols, lda, cols);
  if (s != AVERIS_OK) return s;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if ((s = check_tensor(residual, rows, cols)) != AVERIS_OK) return s;
  if ((s = check_tensor(mean, 1, cols)) != AVERIS_OK) return s;
  if (!aligned(mean_f32, 4)) return AVERIS_E_ALIGN;
  Rank1Out r1{};
  if (b || rho) {
    if (!b || !rho) return AVERIS_E_NULL;
    if (!aligned(rho, 4)) return AVERIS_E_ALIGN;
    if (cols > kRank1MaxK) return AVERIS_E_SHAPE;
    if ((s = check_tensor(b, b->rows, cols)) != AVERIS_OK) return s;
    if (b->rows <= 0) return AVERIS_E_SHAPE;
    r1 = rank1_one(QOperand{b->codes, b->scales, b->tscale}, b->rows, rho);
  }
  const size_t need = split_ws_bytes(rows, cols, 1);
  if (!ws || ws_bytes < need) return AVERIS_E_WORKSPACE;
  if (!aligned(ws, 256)) return AVERIS_E_ALIGN;
  const SplitWs w = split_ws_carve(ws, rows, cols, 1);
  const QuantOut ro{residual->codes, residual->scales, residual->tscale};
  const QuantOut mo{mean->codes, mean->scales, mean->tscale};
  return hip_status(launch_split_from_stats(a, true, rows, cols, lda, nullptr, 1, kGemmRows,
                                            rnd == AVERIS_SR, seed, ro, mo, mean_f32, w, stream,
                                            b ? &r1 : nullptr));
}

averis_status_t averis_split_quant_noalloc(const void* a, averis_dtype_t dtype, int64_t rows,
                                           int64_t cols, int64_t lda, uint64_t seed,
                                           averis_round_t rnd, const averis_nvfp4_t* residual,
                                           const averis_nvfp4_t* mean, float* mean_f32,
                                           hipStream_t stream) {
  // the argument checks of averis_split_quant and the scratch limit, before
  // any HIP call
  averis_status_t s = check_input(a, dtype, rows, cols, lda, cols);
  if (s != AVERIS_OK) return s;
  if (rnd != AVERIS_RN && rnd != AVERIS_SR) return AVERIS_E_ARG;
  if ((s = check_tensor(residual, rows, cols)) != AVERIS_OK) return s;
  if ((s = check_tensor(mean, 1, cols)) != AVERIS_OK) return s;
  if (!aligned(mean_f32, 4)) return AVERIS_E_ALIGN;
  const size_t need = split_ws_bytes(rows, cols, 1);
  if (need > kScratchBytes) {
    std::snprintf(g_last_error, sizeof(g_last_error),
                  "averis_split_quant_noalloc: a %lld x %lld input needs %zu bytes of scratch; "
                  "the library's device array holds %zu",
                  (long long)rows, (long long)cols, need, kScratchBytes);
    return AVERIS_E_WORKSPACE;
  }
  void* ws = nullptr;
  const hipError_t e = scratch_address(&ws);
  if (e != hipSuccess) return hip_status(e);
  return split_common(a, dtype, rows, cols, lda, nullptr, 1, seed, rnd, residual, mean, mean_f32,
                      ws, kScratchBytes, stream);
}

}  // extern "C"
