// Prints Philox4x32-10 words from rocRAND's host-callable engine for (seed, P, v) triples read
// from stdin, one "seed P v" per line (decimal). Used only by the oracle's pin tests: rocRAND is
// an independent, installed implementation of the same generator (Salmon et al., SC'11).
// rocRAND's engine(seed, subsequence, offset) keys Philox with (lo32(seed), hi32(seed)) and
// starts at counter (offset / 4 as 64 bits, subsequence as 64 bits), returning word offset % 4
// first. The oracle's counter for vocab entry v at position P is (v >> 2, lo32(P), hi32(P), 0),
// so offset = (lo32(P) << 32 | v >> 2) * 4 + (v & 3) and subsequence = hi32(P).
#include <rocrand/rocrand_philox4x32_10.h>
#include <cstdio>
#include <cinttypes>
int main() {
  unsigned long long seed, P, v;
  while (std::scanf("%llu %llu %llu", &seed, &P, &v) == 3) {
    unsigned long long plo = P & 0xffffffffull, phi = P >> 32;
    unsigned long long offset = ((plo << 32) | (v >> 2)) * 4ull + (v & 3ull);
    rocrand_device::philox4x32_10_engine eng(seed, phi, offset);
    unsigned int w = eng();
    std::printf("%u\n", w);
  }
  return 0;
}
