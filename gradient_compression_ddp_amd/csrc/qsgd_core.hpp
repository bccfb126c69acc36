// Per-quad QSGD arithmetic shared by the stand-alone QSGD kernel and the QSGD stage of
// the Top-K pipeline.  One binary32 operation per step, in this order:
//   a = fl(|v|/nu), u = fl(a*s), l = floor(u), p = u - l (exact), level = min(l + (U<p), s),
//   g_hat = sign * fl(fl(nu*level)/s), code = sign * level; nu == 0 gives level 0.
#pragma once

#include "common.hpp"

namespace gc {

// ys = fl(1/s); the division by s goes through div_level_count (the same quotient).
//
// The level needs floor(u) and the decision U < p of u = fl(fl(|v| / nu) * s).  An
// estimate u' = fl(|v| * fl(rnu * s)) with rnu = v_rcp_f32(nu) (within 1 ulp of 1/nu, for
// nu in [2^-126, 2^126)) carries three relative errors (2^-23, 2^-24, 2^-24) against the
// two roundings of u (2^-24 each), so it lies within (|v| / nu) * s * (2^-22 + 2^-23) <
// 2^-14 of u, since s <= 127 and |v| <= nu up to a few ulps.  So when p' = u' - floor(u') is at least 2^-13 from 0, from 1 and from U,
// floor(u) = floor(u') and (U < p) = (U < p'); a quad with any element outside that band
// (or nu outside the range, or nu = 0) divides.  One reciprocal per quad replaces four
// IEEE divisions on almost every quad.
//
// When the estimate is taken, nu lies in that range (so nu > 0), and the level needs no
// clamp to s: |v| <= nu up to a few ulps, so u' <= s * (1 + 2^-21), and floor(u') = s
// would leave p' < 2^-13, which divides.  A taken element is also nonzero and not NaN
// (p' >= 2^-13), so its sign bit is the sign test v < 0; the divided path keeps both the
// nu > 0 test and the clamp (a NaN or zero element, or nu = 0, gives level 0, and -0 as
// well as 0 converts to code 0; -Inf gives -s through the sign bit, as v < 0 does).
__device__ __forceinline__ void qsgd_quad(const float v[4], float nu, float s, float ys, const float u[4],
                                          int lev[4], float gh[4]) {
  const float rnus = __builtin_amdgcn_rcpf(nu) * s;
  bool slow = !(nu >= 0x1p-126f && nu < 0x1p126f);
  float level[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float uu = fabsf(v[m]) * rnus;
    const float l = floorf(uu);
    const float p = uu - l;
    slow |= !(p >= 0x1p-13f && p <= 1.0f - 0x1p-13f && fabsf(u[m] - p) >= 0x1p-13f);
    level[m] = l + (u[m] < p ? 1.f : 0.f);
  }
  if (slow) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float l = 0.f, up1 = 0.f;
      if (nu > 0.f) {
        const float a = fabsf(v[m]) / nu;
        const float uu = a * s;
        l = floorf(uu);
        up1 = u[m] < (uu - l) ? 1.f : 0.f;
      }
      level[m] = nu > 0.f ? fminf(l + up1, s) : 0.f;
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    lev[m] = (int)__builtin_copysignf(level[m], v[m]);   // level 0 gives 0 for either sign
    gh[m] = nu * level[m];   // t, divided below
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
