// Host driver for the exact-sum arithmetic of the split-quant kernels
// (mean_residual_quantized_amd/csrc/exact_sum.hpp), used by
// tests/test_exact_sum_host.py.  Reads cases from stdin, one per line:
//   n32 n64 <n32 fp32 values as hex bits> <n64 fp64 values as hex bits>
// and prints the correctly rounded sum of each case as fp64 hex bits: the
// 320-bit sum, then the 64-bit grid sum (grid from the fp32 values' smallest
// nonzero magnitude, fp32 precision) or "x" where that grid does not fit.
#include <cinttypes>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <vector>

#include "exact_sum.hpp"

int main() {
  int n32, n64;
  while (std::scanf("%d %d", &n32, &n64) == 2) {
    uint32_t acc[averis::kWideWords] = {0};
    std::vector<double> vals;
    float mnz = __builtin_inff();
    double amax = 0.0;
    for (int i = 0; i < n32; ++i) {
      uint32_t b;
      if (std::scanf("%" SCNx32, &b) != 1) return 1;
      float f;
      std::memcpy(&f, &b, 4);
      averis::wide_add_f32(acc, f);
      vals.push_back((double)f);
      if (f != 0.0f && std::fabs(f) < mnz) mnz = std::fabs(f);
      amax = std::fmax(amax, std::fabs((double)f));
    }
    for (int i = 0; i < n64; ++i) {
      uint64_t b;
      if (std::scanf("%" SCNx64, &b) != 1) return 1;
      double d;
      std::memcpy(&d, &b, 8);
      averis::wide_add_f64(acc, d);
      vals.push_back(d);
      amax = std::fmax(amax, std::fabs(d));
    }
    const double r = averis::wide_to_double(acc);
    uint64_t rb;
    std::memcpy(&rb, &r, 8);
    std::printf("%016" PRIx64, rb);
    const int gexp = averis::value_grid_exp(mnz, 23);
    if (mnz < __builtin_inff() && averis::grid_sum_fits((double)(n32 + n64), amax, gexp)) {
      int64_t n = 0;
      for (double v : vals) n += averis::grid_int64(v, gexp);
      const double g = averis::grid_int64_to_double(n, gexp);
      uint64_t gb;
      std::memcpy(&gb, &g, 8);
      std::printf(" %016" PRIx64 "\n", gb);
    } else {
      std::printf(" x\n");
    }
  }
  return 0;
}
