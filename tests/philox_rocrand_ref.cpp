// Independent Philox-4x32-10 for pinning the oracle's generator: AMD's
// rocRAND device/host header implementation, compiled as a plain host
// program.  Each stdin line "seed c0 c1 c2 c3" (decimal) prints the four
// output words of counter (c0, c1, c2, c3) under key (seed mod 2^32,
// seed >> 32).
//
// rocRAND addresses its 128-bit counter through (subsequence, offset):
// the subsequence is the upper 64 bits (words 2 and 3) and the offset counts
// 32-bit outputs, four per counter value, so counter words 0 and 1 are
// reached with offset = 4 * (c0 + 2^32 c1).
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed, c0, c1, c2, c3;
  while (std::scanf("%llu %llu %llu %llu %llu", &seed, &c0, &c1, &c2, &c3) == 5) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, c2 | (c3 << 32), 4ull * (c0 | (c1 << 32)), &st);
    const uint4 v = rocrand4(&st);
    std::printf("%u %u %u %u\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
