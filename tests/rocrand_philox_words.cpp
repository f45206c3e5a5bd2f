// Host-only helper for the oracle's Philox pin: prints rocRAND's Philox-4x32-10
// output for (seed, counter) pairs read from stdin, one pair per line, as four hex
// words.  rocRAND's state for (seed, subsequence 0, offset 4*n) is key =
// (low, high word of seed) and counter = (low, high word of n, 0, 0), so its first
// four outputs are the generator applied to exactly that key and counter.
// Built with hipcc for the host only; it launches nothing on a GPU.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
  unsigned long long seed = 0, ctr = 0;
  while (std::scanf("%llu %llu", &seed, &ctr) == 2) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, 0ULL, 4ULL * ctr, &st);
    uint4 r = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", r.x, r.y, r.z, r.w);
  }
  return 0;
}
