// Independent Philox4x32-10 reference for the oracle's pin: rocRAND's own
// host-callable engine.  Prints the four 32-bit output words of Philox4x32-10
// for key = seed and counter = (g lo, g hi, stream, 0), one line per g.
// rocRAND's engine seeded with (seed, subsequence = stream, offset = 4 g)
// produces exactly that block as its first next4().
// Usage: rocrand_philox_ref <seed> <stream> <g> [<g> ...]
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc < 4) return 2;
  unsigned long long seed = strtoull(argv[1], nullptr, 0);
  unsigned long long stream = strtoull(argv[2], nullptr, 0);
  for (int i = 3; i < argc; ++i) {
    unsigned long long g = strtoull(argv[i], nullptr, 0);
    rocrand_device::philox4x32_10_engine e(seed, stream, 4ull * g);
    uint4 r = e.next4();
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
