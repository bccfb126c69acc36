// Reference Philox4x32-10 blocks from rocRAND's host-callable engine.
// Reads "seed counter" pairs (decimal or 0x hex) from stdin, one per line, and
// prints the four 32-bit words of the block at that counter, as 8-digit hex.
// rocrand_init(seed, subsequence = 0, offset = 4 * counter) positions the engine at
// the first word of block `counter`; rocrand4 then returns that whole block.
// Built with hipcc as plain host code: no device is touched.
#include <rocrand/rocrand_kernel.h>
#include <cstdio>
#include <cstdlib>

int main() {
  char a[64], b[64];
  while (std::scanf("%63s %63s", a, b) == 2) {
    unsigned long long seed = std::strtoull(a, nullptr, 0);
    unsigned long long ctr = std::strtoull(b, nullptr, 0);
    rocrand_state_philox4x32_10 st;
    rocrand_init(seed, 0ull, 4ull * ctr, &st);
    uint4 v = rocrand4(&st);
    std::printf("%08x %08x %08x %08x\n", v.x, v.y, v.z, v.w);
  }
  return 0;
}
