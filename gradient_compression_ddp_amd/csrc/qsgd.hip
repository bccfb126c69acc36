// QSGD: stochastic rounding onto s levels of the group L2 norm, gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", section 1.1
// (stochastic rounding between levels, unbiased, run with error feedback) and section
// 1.2 (grouping); the per-group L2-norm levels of the QSGD paper the page cites.
//
// Layout: each lane owns an aligned quad of 4 consecutive elements; a group of G
// elements (power of two, 4..256) spans G/4 lanes.  The group's sum of squares is a
// balanced pairwise tree in index order: inside the lane ((x0^2+x1^2)+(x2^2+x3^2)), then
// a lane butterfly with offsets 1, 2, 4, ... (each step adds exactly one tree pair).
// The random draw of element e is word (e&3) of the Philox block at counter e>>2, so an
// aligned quad costs one Philox call.  One pass: 4 B read, 1 B code written per element
// (+4 B read and written for the residual), 4 B per group for the norm.
#include "common.hpp"
#include "internal.hpp"
#include "qsgd_core.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;

template <bool EF>
__global__ __launch_bounds__(kBlock) void k_qsgd(const float* __restrict__ x, float* __restrict__ res,
                                                 int64_t n, int lpg_log2, float s, uint64_t seed,
                                                 int64_t index_base, int8_t* __restrict__ codes,
                                                 float* __restrict__ norms) {
  const int64_t nquads = (n + 3) >> 2;
  const int lpg = 1 << lpg_log2;
  const int lane = lane_id();
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t base = (int64_t)blockIdx.x * kBlock; base < nquads; base += stride) {
    const int64_t q = base + threadIdx.x;
    const int64_t e0 = q << 2;
    const bool live = q < nquads;
    const bool full = e0 + 4 <= n;
    float v[4];
    if (live && full) {
      const float4 a = *reinterpret_cast<const float4*>(x + e0);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      if (EF) {
        const float4 b = *reinterpret_cast<const float4*>(res + e0);
        v[0] = v[0] + b.x; v[1] = v[1] + b.y; v[2] = v[2] + b.z; v[3] = v[3] + b.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float t = 0.f;
        if (live && e0 + m < n) {
          t = x[e0 + m];
          if (EF) t = t + res[e0 + m];
        }
        v[m] = t;
      }
    }
    // pairwise tree: lane-local levels, then the lane butterfly
    float ss = quad_sumsq(v);
    ss = seg_tree_sum(ss, lpg);
    if (!live) continue;
    const float nu = sqrtf(ss);
    float u[4];
    uniforms4(seed, (uint64_t)(index_base + e0), u);
    int lev[4];
    float gh[4];
    qsgd_quad(v, nu, s, u, lev, gh);
    if (full) {
      *reinterpret_cast<uint32_t*>(codes + e0) = pack_codes4(lev);
      if (EF) {
        float4 r;
        r.x = v[0] - gh[0]; r.y = v[1] - gh[1]; r.z = v[2] - gh[2]; r.w = v[3] - gh[3];
        *reinterpret_cast<float4*>(res + e0) = r;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (e0 + m < n) {
          codes[e0 + m] = (int8_t)lev[m];
          if (EF) res[e0 + m] = v[m] - gh[m];
        }
    }
    if ((lane & (lpg - 1)) == 0) norms[e0 >> (lpg_log2 + 2)] = nu;
  }
}

}  // namespace

hipError_t launch_qsgd(const float* x, float* res, int64_t n, int64_t group, int levels,
                       uint64_t seed, int64_t index_base, int8_t* codes, float* norms,
                       hipStream_t s) {
  if (n == 0) return hipSuccess;
  int lpg_log2 = 0;
  while ((int64_t(4) << lpg_log2) < group) ++lpg_log2;
  const int64_t nquads = (n + 3) / 4;
  int64_t blocks = (nquads + kBlock - 1) / kBlock;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  const float sf = (float)levels;
  if (res)
    hipLaunchKernelGGL((k_qsgd<true>), (int)blocks, kBlock, 0, s, x, res, n, lpg_log2, sf, seed, index_base, codes, norms);
  else
    hipLaunchKernelGGL((k_qsgd<false>), (int)blocks, kBlock, 0, s, x, res, n, lpg_log2, sf, seed, index_base, codes, norms);
  return hipGetLastError();
}

}  // namespace gc
