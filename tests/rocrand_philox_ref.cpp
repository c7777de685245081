// Reference Philox4x32-10 blocks from rocRAND's engine (a library routine,
// called on the host): an independent check of the oracle's generator.
// Reads lines "seed subsequence offset" (decimal) from stdin and prints the
// four 32-bit outputs rocRAND returns after rocrand_init(seed, subsequence,
// offset), in hexadecimal, one line per request. With offset a multiple of 4
// these are the Philox block of counter (offset/4 low word, offset/4 high
// word, subsequence low word, subsequence high word) under key (seed low
// word, seed high word).
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed, sub, off;
  while (std::scanf("%llu %llu %llu", &seed, &sub, &off) == 3) {
    rocrand_state_philox4x32_10 s;
    rocrand_init(seed, sub, off, &s);
    unsigned int a = rocrand(&s), b = rocrand(&s), c = rocrand(&s), d = rocrand(&s);
    std::printf("%08x %08x %08x %08x\n", a, b, c, d);
  }
  return 0;
}
