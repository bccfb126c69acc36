// Per-quad QSGD arithmetic shared by the stand-alone QSGD kernel and the QSGD stage of
// the Top-K pipeline.  One binary32 operation per step, in this order:
//   a = fl(|v|/nu), u = fl(a*s), l = floor(u), p = u - l (exact), level = min(l + (U<p), s),
//   g_hat = sign * fl(fl(nu*level)/s), code = sign * level; nu == 0 gives level 0.
#pragma once

#include "common.hpp"

namespace gc {

// ys = fl(1/s); the division by s goes through div_level_count (the same quotient).
//
// The level l + (U < p), with u = fl(fl(|v| / nu) * s), l = floor(u) and p = u - l, equals
// ceil(u - U) for U in [0, 1): U < p puts u - U in (l, l + 1), U >= p puts it in (l - 1, l].
// An estimate u' = fl(|v| * fl(rnu * s)) with rnu = v_rcp_f32(nu) (within 1 ulp of 1/nu,
// for nu in [2^-126, 2^126)) carries three relative errors (2^-23, 2^-24, 2^-24) against
// the two roundings of u (2^-24 each), so it lies within (|v| / nu) * s * (2^-22 + 2^-23)
// < 2^-14 of u, since s <= 127 and |v| <= nu up to a few ulps; d' = fl(u' - U) adds at most
// 2^-18.  So when ceil(d') - d' is at least 2^-13 from 0 and from 1, ceil(u - U) =
// ceil(d'); a quad with any element outside that band (or nu outside the range, or nu =
// 0) divides.  One reciprocal per quad replaces four IEEE divisions on almost every quad.
//
// When the estimate is taken, nu lies in that range (so nu > 0), and the level needs no
// clamp to s: u' <= s * (1 + 2^-21), and d' above s would leave ceil(d') - d' within 2^-14
// of 1, which divides.  A NaN element fails the band and divides.  A zero element (and
// any d' in (-1, 0)) takes the level -0, which converts to code 0 and enters the
// dequantization as +0; the divided path keeps both the nu > 0 test and the clamp (a NaN
// or zero element, or nu = 0, gives level 0; -Inf gives -s through the sign bit, as v < 0
// does).
__device__ __forceinline__ void qsgd_quad(const float v[4], float nu, float s, float ys, const float u[4],
                                          int lev[4], float gh[4]) {
  const float rnus = __builtin_amdgcn_rcpf(nu) * s;
  bool slow = !(nu >= 0x1p-126f && nu < 0x1p126f);
  float level[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const float d = fabsf(v[m]) * rnus - u[m];
    const float c = ceilf(d);
    const float e = c - d;
    slow |= !(e >= 0x1p-13f && e <= 1.0f - 0x1p-13f);
    level[m] = c;
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
    gh[m] = nu * fabsf(level[m]);   // t, divided below (|.| turns an estimated -0 level into +0)
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
