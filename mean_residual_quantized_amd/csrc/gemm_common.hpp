// Helpers shared by the quantized GEMM kernels (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace averis {

// Opts kernel KERN into `bytes` of dynamic LDS, once per device (the
// attribute is per device; a bit per device id, set after the call succeeds,
// so concurrent first calls only repeat the idempotent call).
template <auto KERN>
inline hipError_t lds_attr_once(int bytes) {
  static std::atomic<uint64_t> done{0};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (1ull << dev) : 0ull;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(reinterpret_cast<const void*>(KERN),
                          hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ half2_t h2(uint32_t u) { return __builtin_bit_cast(half2_t, u); }
__device__ __forceinline__ uint32_t u32(half2_t h) { return __builtin_bit_cast(uint32_t, h); }

// 8 E2M1 codes of one dword (k ascending from bits 3:0) -> 4 x (2 x fp16),
// times the block scale s2 = (s, s).  v_cvt_scalef32_pk_f16_fp4 with scale 1
// gives the code values exactly; an E2M1 value (<= 2 significant bits) times
// an E4M3 scale (<= 4 bits) is exact in fp16.
__device__ __forceinline__ uint4 deq8(uint32_t w, half2_t s2) {
  uint4 r;
  r.x = u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
  r.y = u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
  r.z = u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
  r.w = u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
  return r;
}

// the two E4M3 bytes in bits 15:0 -> (fp16, fp16); v_cvt_scalef32_pk_f16_fp8
// with scale 1 decodes every E4M3FN code exactly (subnormals included)
__device__ __forceinline__ half2_t scales2(uint32_t two_bytes) {
  return __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(two_bytes, 1.0f, false);
}

__device__ __forceinline__ uint16_t f32_to_bf16_rne(float f) {
  const uint32_t b = __float_as_uint(f);
  if ((b & 0x7F800000u) == 0x7F800000u) return (uint16_t)((b >> 16) | ((b & 0xFFFFu) ? 0x40u : 0u));
  return (uint16_t)((b + 0x7FFFu + ((b >> 16) & 1u)) >> 16);
}

// two fp32 -> two bf16 (round to nearest even, v_cvt_pk_bf16_f32), packed
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float lo, float hi) {
  const f32x2_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

// output stores: plain (L2 merges the partial lines of a row segment)
template <typename T>
__device__ __forceinline__ void store_out(T v, T* p) {
  *p = v;
}

// streaming output stores (nontemporal: whole 128-byte lines written by
// eight lanes go to memory without staying dirty in L2).  A GEMM's bf16
// output is not read again soon, and left dirty in L2 it is written back
// while the next kernels on the stream run: measured 1-2 us less per launch
// of the codes-in-LDS GEMM and about 25 us less for the splits that follow
// the GEMMs of the seven-linear step.  (Split-K partials, which the reduce
// reads right away, keep plain stores: streamed, that reduce got slower.)
template <typename T>
__device__ __forceinline__ void store_stream(T v, T* p) {
  __builtin_nontemporal_store(v, p);
}

constexpr int kXcds = 8;   // MI355X: 8 accelerator complex dies, one L2 each

// After the last MFMA of a K loop its accumulators must not be read for
// ~18 wait states (32x32 f16 MFMA, 8 passes).  The compiler's hazard check
// misses this when the loop exits through a branch straight into a barrier,
// so the kernels fence explicitly, in the block of the last MFMA.
__device__ __forceinline__ void mfma_drain() {
  __builtin_amdgcn_sched_barrier(0);
  asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 7" ::: "memory");
  __builtin_amdgcn_sched_barrier(0);
}

// Workgroups are dispatched round-robin over the 8 XCDs (linear id % 8).
// Renumber them so each XCD walks a contiguous, row-major run of tiles: the
// tiles an XCD runs together share operand rows in its L2.
__device__ __forceinline__ void xcd_tile(int64_t& tile_x, int64_t& tile_y) {
  const int64_t gx = gridDim.x, total = gx * gridDim.y;
  const int64_t lin = (int64_t)blockIdx.y * gx + blockIdx.x;
  const int64_t even = total - total % kXcds;
  int64_t id = lin;
  if (lin < even) id = (lin % kXcds) * (even / kXcds) + lin / kXcds;
  tile_y = id / gx;
  tile_x = id - tile_y * gx;
}

}  // namespace averis
