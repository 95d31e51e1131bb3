// Reference Philox4x32-10 outputs from rocRAND's engine (its public header, run on the host):
// reads "seed x y z w" lines and prints the four 32-bit words for counter (x, y, z, w).
// rocRAND's engine takes the 64-bit seed as its key and places `offset / 4` in counter words
// 0-1 and `subsequence` in words 2-3, so any counter can be addressed.
#include <hip/hip_runtime.h>
#include <rocrand/rocrand_kernel.h>

#include <cstdio>

int main() {
  unsigned long long seed;
  unsigned x, y, z, w;
  while (std::scanf("%llu %u %u %u %u", &seed, &x, &y, &z, &w) == 5) {
    rocrand_state_philox4x32_10 st;
    const unsigned long long subsequence = ((unsigned long long)w << 32) | z;
    const unsigned long long offset = 4ull * (((unsigned long long)y << 32) | x);
    rocrand_init(seed, subsequence, offset, &st);
    const unsigned a = rocrand(&st), b = rocrand(&st), c = rocrand(&st), d = rocrand(&st);
    std::printf("%u %u %u %u\n", a, b, c, d);
  }
  return 0;
}
