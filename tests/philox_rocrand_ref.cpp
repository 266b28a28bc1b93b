// Host program printing Philox4x32-10 outputs from rocRAND's engine (an
// implementation independent of the oracle), used to pin the oracle's Philox.
// Usage: philox_rocrand_ref <seed> <subsequence> <count>
// Prints `count` lines of four hex words: call n uses counter
// (n_lo, n_hi, subsequence_lo, subsequence_hi) and key (seed_lo, seed_hi).
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>
#include <cstdlib>

int main(int argc, char** argv) {
  if (argc != 4) return 2;
  unsigned long long seed = strtoull(argv[1], nullptr, 0);
  unsigned long long sub = strtoull(argv[2], nullptr, 0);
  long count = strtol(argv[3], nullptr, 0);
  rocrand_device::philox4x32_10_engine eng(seed, sub, 0);
  for (long i = 0; i < count; i++) {
    uint4 r = eng.next4();
    printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
