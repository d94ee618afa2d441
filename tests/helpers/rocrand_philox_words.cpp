// Prints Philox4x32-10 output words computed by rocRAND's installed engine.
// Used only to cross-check the oracle's Philox implementation.
// Input (stdin): lines "seed c0 c1 c2 c3" (decimal); output: "x0 x1 x2 x3".
// rocRAND's state keys the generator with the 64-bit seed (lo, hi), puts the
// 64-bit subsequence in counter words 2..3 and offset/4 in counter words 0..1.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
  unsigned long long seed, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
    unsigned long long subseq = c2 | (c3 << 32);
    unsigned long long offset = 4ull * (c0 | (c1 << 32));
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, subseq, offset, &st);
    unsigned int w[4];
    for (int i = 0; i < 4; ++i) w[i] = rocrand(&st);
    std::printf("%u %u %u %u\n", w[0], w[1], w[2], w[3]);
  }
  return 0;
}
