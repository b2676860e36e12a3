// Row segments (expert groups) and segment-aligned row chunks.
//
// A tensor's rows are split into nseg segments by a device array of offsets
// (nseg + 1 non-decreasing int64, first 0, last rows); offsets == nullptr
// means one segment of all rows.  Kernels cut each segment into chunks of
// `ch` rows so that no chunk straddles two segments; chunk c of the whole
// tensor maps to (segment, row range) through a prefix sum over the
// segments' chunk counts, computed by one wavefront.  Offsets outside
// [0, rows] are clamped and a decreasing pair counts as an empty segment, so
// malformed offsets never address memory outside the tensor.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace averis {

struct SegRange {
  int seg;          // segment index (-1: chunk past the end)
  int64_t r0, r1;   // row range [r0, r1) of this chunk (or segment)
  int64_t seg_r0, seg_r1;  // the whole segment's rows
  int64_t c0, c1;   // the segment's chunk index range
};

__device__ __forceinline__ int64_t clamp_row(int64_t v, int64_t rows) {
  return v < 0 ? 0 : (v > rows ? rows : v);
}

__device__ __forceinline__ void seg_bounds(const int64_t* offs, int s, int64_t rows, int64_t& a,
                                           int64_t& b) {
  a = clamp_row(offs[s], rows);
  b = clamp_row(offs[s + 1], rows);
  if (b < a) b = a;
}

// One segment of all rows (offsets == nullptr): the range in closed form.
__device__ __forceinline__ SegRange plain_range(int64_t rows, int64_t ch, int64_t key, int mode) {
  const int64_t n = (rows + ch - 1) / ch;
  SegRange r;
  r.seg = (mode == 1) ? (key == 0 ? 0 : -1) : (key < n ? 0 : -1);
  r.seg_r0 = 0;
  r.seg_r1 = rows;
  r.c0 = 0;
  r.c1 = n;
  r.r0 = mode == 1 ? 0 : key * ch;
  r.r1 = mode == 1 ? rows : (key * ch + ch < rows ? key * ch + ch : rows);
  return r;
}

// Wave-level scan.  Must be called by all 64 lanes of one wavefront; the lane
// that finds the answer writes it to *out.  mode 0: locate chunk `key`;
// mode 1: describe segment `key`.
__device__ inline void seg_scan(const int64_t* offs, int nseg, int64_t rows, int64_t ch,
                                int64_t key, int mode, SegRange* out) {
  const int lane = threadIdx.x & 63;
  if (offs == nullptr) {
    if (lane == 0) *out = plain_range(rows, ch, key, mode);
    return;
  }
  int64_t carry = 0;
  bool found = false;
  for (int base = 0; base < nseg; base += 64) {
    const int s = base + lane;
    int64_t a = 0, b = 0;
    if (s < nseg) seg_bounds(offs, s, rows, a, b);
    const int64_t n = (b - a + ch - 1) / ch;
    int64_t incl = n;
    for (int d = 1; d < 64; d <<= 1) {
      const int64_t t = __shfl_up(incl, d, 64);
      if (lane >= d) incl += t;
    }
    const int64_t excl = carry + incl - n;
    incl += carry;
    const bool hit = s < nseg && (mode == 1 ? (s == key) : (key >= excl && key < incl));
    if (hit) {
      SegRange r;
      r.seg = s;
      r.seg_r0 = a;
      r.seg_r1 = b;
      r.c0 = excl;
      r.c1 = incl;
      if (mode == 1) {
        r.r0 = a;
        r.r1 = b;
      } else {
        r.r0 = a + (key - excl) * ch;
        r.r1 = r.r0 + ch < b ? r.r0 + ch : b;
      }
      *out = r;
    }
    found = found || __any(hit);
    carry = __shfl(incl, 63, 64);
    if (found) break;
  }
  if (!found && lane == 0) {
    SegRange r;
    r.seg = -1;
    r.r0 = r.r1 = r.seg_r0 = r.seg_r1 = 0;
    r.c0 = r.c1 = 0;
    *out = r;
  }
}

// Block-level wrappers: every thread of the block gets the result (without
// offsets in closed form, with no block synchronization).
__device__ inline SegRange locate_chunk(const int64_t* offs, int nseg, int64_t rows, int64_t ch,
                                        int64_t chunk) {
  if (offs == nullptr) return plain_range(rows, ch, chunk, 0);
  __shared__ SegRange sr;
  if (threadIdx.x < 64) seg_scan(offs, nseg, rows, ch, chunk, 0, &sr);
  __syncthreads();
  SegRange r = sr;
  __syncthreads();
  return r;
}

__device__ inline SegRange describe_segment(const int64_t* offs, int nseg, int64_t rows,
                                            int64_t ch, int seg) {
  if (offs == nullptr) return plain_range(rows, ch, seg, 1);
  __shared__ SegRange sr;
  if (threadIdx.x < 64) seg_scan(offs, nseg, rows, ch, seg, 1, &sr);
  __syncthreads();
  SegRange r = sr;
  __syncthreads();
  return r;
}

// Upper bound on the total chunk count, known on the host.
static inline int64_t chunk_upper_bound(int64_t rows, int nseg, int64_t ch) {
  return (rows + ch - 1) / ch + (nseg > 1 ? nseg : 0);
}

}  // namespace averis
