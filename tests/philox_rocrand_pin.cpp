// Test helper (host only): prints rocRAND's Philox4x32-10 blocks for the
// (seed, row, position, offset) tuples read from stdin, one per line, so the
// oracle's Philox can be checked against an independent library routine.
// rocRAND keys the engine with (seed_lo, seed_hi), puts the subsequence in
// counter words 2-3 and advances words 0-1 by offset/4.
#include <cstdio>
#include <rocrand/rocrand_kernel.h>

int main() {
  unsigned long long seed, row, pos, off;
  while (std::scanf("%llu %llu %llu %llu", &seed, &row, &pos, &off) == 4) {
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, off, 4ull * (pos + (row << 32)), &st);
    uint4 b = rocrand4(&st);
    std::printf("%u %u %u %u\n", b.x, b.y, b.z, b.w);
  }
  return 0;
}
