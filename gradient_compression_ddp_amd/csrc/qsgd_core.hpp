// Per-quad QSGD arithmetic shared by the stand-alone QSGD kernel and the QSGD stage of
// the Top-K pipeline.  One binary32 operation per step, in this order:
//   a = fl(|v|/nu), u = fl(a*s), l = floor(u), p = u - l (exact), level = min(l + (U<p), s),
//   g_hat = sign * fl(fl(nu*level)/s), code = sign * level; nu == 0 gives level 0.
#pragma once

#include "common.hpp"

namespace gc {

// ys = fl(1/s); the division by s goes through div_level_count (the same quotient).
__device__ __forceinline__ void qsgd_quad(const float v[4], float nu, float s, float ys, const float u[4],
                                          int lev[4], float gh[4]) {
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    float level = 0.f;
    if (nu > 0.f) {
      const float a = fabsf(v[m]) / nu;
      const float uu = a * s;
      const float l = floorf(uu);
      const float p = uu - l;
      level = fminf(l + (u[m] < p ? 1.f : 0.f), s);
    }
    lev[m] = v[m] < 0.f ? -(int)level : (int)level;
    gh[m] = nu * level;   // t, divided below
  }
  // with nu >= 2^-100 every t = fl(nu * level) is 0 or >= 2^-100: div_level_count's domain
  float mag[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) mag[m] = div_level_count(gh[m], s, ys);
  if (!(nu >= 0x1p-100f)) {
#pragma unroll
    for (int m = 0; m < 4; ++m) mag[m] = gh[m] / s;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) gh[m] = v[m] < 0.f ? -mag[m] : mag[m];
}

__device__ __forceinline__ uint32_t pack_codes4(const int lev[4]) {
  return (uint32_t)(uint8_t)lev[0] | ((uint32_t)(uint8_t)lev[1] << 8) |
         ((uint32_t)(uint8_t)lev[2] << 16) | ((uint32_t)(uint8_t)lev[3] << 24);
}

// Sum of squares of a quad as the two lowest levels of the pairwise tree.
__device__ __forceinline__ float quad_sumsq(const float v[4]) {
  return (v[0] * v[0] + v[1] * v[1]) + (v[2] * v[2] + v[3] * v[3]);
}

}  // namespace gc
