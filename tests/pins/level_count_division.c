/* Checks the quotient form the QSGD dequantization kernels use for fl(t / s), s a level
 * count in [1, 127]:  q0 = fl(t * ys) with ys = fl(1/s),  q = fma(fma(-q0, s, t), ys, q0),
 * against the IEEE binary32 division, for every t whose bit pattern lies in [lo, hi)
 * (non-negative t: 0 .. 0x7F800000 is every finite value) and every s in [s0, s1].
 * t = +Inf is excluded: there the kernels take q0 itself.
 * Usage: level_count_division s0 s1 lo hi   (prints the number of mismatches) */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

static float from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t to_bits(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

int main(int argc, char** argv) {
  if (argc != 5) return 2;
  const int s0 = atoi(argv[1]), s1 = atoi(argv[2]);
  const uint64_t lo = strtoull(argv[3], NULL, 0), hi = strtoull(argv[4], NULL, 0);
  unsigned long long bad = 0;
  for (int si = s0; si <= s1; ++si) {
    const float s = (float)si;
    const float ys = 1.0f / s;
    for (uint64_t u = lo; u < hi; ++u) {
      const float t = from_bits((uint32_t)u);
      const float q0 = t * ys;
      const float q = fmaf(fmaf(-q0, s, t), ys, q0);
      const float want = t / s;
      if (to_bits(q) != to_bits(want)) {
        if (bad < 4) fprintf(stderr, "s=%d t=%a: %a, division %a\n", si, t, q, want);
        ++bad;
      }
    }
  }
  printf("%llu\n", bad);
  return 0;
}
