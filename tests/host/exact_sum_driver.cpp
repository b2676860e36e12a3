// Host driver for the exact-sum arithmetic of the split-quant kernels
// (mean_residual_quantized_amd/csrc/exact_sum.hpp), used by
// tests/test_exact_sum_host.py.  Reads cases from stdin, one per line:
//   n32 n64 <n32 fp32 values as hex bits> <n64 fp64 values as hex bits>
// and prints the correctly rounded sum of each case as fp64 hex bits.
#include <cinttypes>
#include <cstdio>
#include <cstring>

#include "exact_sum.hpp"

int main() {
  int n32, n64;
  while (std::scanf("%d %d", &n32, &n64) == 2) {
    uint32_t acc[averis::kWideWords] = {0};
    for (int i = 0; i < n32; ++i) {
      uint32_t b;
      if (std::scanf("%" SCNx32, &b) != 1) return 1;
      float f;
      std::memcpy(&f, &b, 4);
      averis::wide_add_f32(acc, f);
    }
    for (int i = 0; i < n64; ++i) {
      uint64_t b;
      if (std::scanf("%" SCNx64, &b) != 1) return 1;
      double d;
      std::memcpy(&d, &b, 8);
      averis::wide_add_f64(acc, d);
    }
    const double r = averis::wide_to_double(acc);
    uint64_t rb;
    std::memcpy(&rb, &r, 8);
    std::printf("%016" PRIx64 "\n", rb);
  }
  return 0;
}
