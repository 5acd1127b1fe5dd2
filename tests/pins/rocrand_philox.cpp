// Test helper (not product code): prints rocRAND's Philox4x32-10 output
// words for counters read from stdin, one query per line:
//   seed c0 c1 c2 c3   ->   w0 w1 w2 w3
// rocRAND's state keys the generator with (seed mod 2^32, seed >> 32); its
// offset argument (in 32-bit words) advances counter words 0-1 and its
// subsequence argument advances counter words 2-3, so any counter can be
// reached.
#include <rocrand/rocrand_philox4x32_10.h>

#include <cstdio>

int main() {
  unsigned long long seed, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)), &st);
    uint4 r = rocrand4(&st);
    std::printf("%u %u %u %u\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
