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
// (+4 B read and written for the residual), 4 B per group for the norm.  The pass is
// bound by VALU work more than by HBM: a Philox4x32-10 block per quad (19 64-bit integer
// multiply-adds, each issued at the full rate on gfx950) and the level decision, taken from
// a reciprocal estimate except near its boundaries (qsgd_core.hpp); the group's butterfly
// is compile-time (DPP steps for up to 16 lanes).  On a 25 MiB bucket two quads per lane
// measured fastest (9.88 us against 9.94 with one and 11.1 with four); a tile wholly
// inside the input computes both rounds before its first store (10.42 -> 9.88 us).
#include "common.hpp"
#include "internal.hpp"
#include "qsgd_core.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kRounds = 2;                                 // quads per thread per tile
constexpr int64_t kTile = (int64_t)kBlock * 4 * kRounds;   // 2048 elements

// One 2048-element tile per block: 2 rounds of 1024 elements, each starting at a multiple
// of 1024 so that every group (G <= 256) lies inside one wave of one round.  All loads
// of the tile are issued before any arithmetic (non-temporal 16-byte loads and stores).
template <bool EF, int LPG_LOG2, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_qsgd(const float* __restrict__ x, float* __restrict__ res,
                                                 int64_t n, float s, float ys, uint64_t seed,
                                                 int64_t index_base, int8_t* __restrict__ codes,
                                                 float* __restrict__ norms) {
  constexpr int lpg_log2 = LPG_LOG2;
  constexpr int lpg = 1 << LPG_LOG2;
  const int lane = lane_id();
  const int64_t base = (int64_t)blockIdx.x * kTile;
  float v[kRounds][4];
  if (base + kTile <= n) {
    // the whole tile is in range (a block-uniform branch): straight-line code, no
    // per-element masks
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + e0));
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      if (EF) {
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(res + e0));
        v[j][0] = v[j][0] + b.x; v[j][1] = v[j][1] + b.y; v[j][2] = v[j][2] + b.z; v[j][3] = v[j][3] + b.w;
      }
    }
    // the draws need no loaded data: they run while the loads are in flight
    float u[kRounds][4];
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
      uniforms4_t<ALIGNED>(seed, (uint64_t)(index_base + base + j * (kBlock * 4) + threadIdx.x * 4), u[j]);
    // keep the compiler from sinking the second round's draw into the code after the
    // first round's wait (an empty asm that takes the draws as operands pins them here)
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(u[j][m]));
    // every round's results before the first store: the wait for a later round's load
    // would otherwise also wait for the earlier stores (the counter retires in order)
    uint32_t cw[kRounds];
    float nus[kRounds];
    f32x4 rr[kRounds];
    {
      float ss[kRounds];
#pragma unroll
      for (int j = 0; j < kRounds; ++j) ss[j] = seg_tree_sum_c<LPG_LOG2>(quad_sumsq(v[j]));
      if constexpr (LPG_LOG2 >= 1 && kRounds == 2) {
        // both lanes of a pair hold both rounds' group sums: each takes one root, and the
        // pair swaps them (one correctly rounded square root per lane instead of two)
        const bool odd = (lane & 1) != 0;
        const float mine = sqrtf(odd ? ss[1] : ss[0]);
        const float other = __uint_as_float(bfly_u32<0>(__float_as_uint(mine)));
        nus[0] = odd ? other : mine;
        nus[1] = odd ? mine : other;
      } else {
#pragma unroll
        for (int j = 0; j < kRounds; ++j) nus[j] = sqrtf(ss[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      int lev[4];
      float gh[4];
      qsgd_quad(v[j], nus[j], s, ys, u[j], lev, gh);
      cw[j] = pack_codes4(lev);
      if (EF) {
        rr[j].x = v[j][0] - gh[0]; rr[j].y = v[j][1] - gh[1];
        rr[j].z = v[j][2] - gh[2]; rr[j].w = v[j][3] - gh[3];
      }
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
      __builtin_nontemporal_store(cw[j], reinterpret_cast<uint32_t*>(codes + e0));
      if (EF) __builtin_nontemporal_store(rr[j], reinterpret_cast<f32x4*>(res + e0));
      if ((lane & (lpg - 1)) == 0) norms[e0 >> (lpg_log2 + 2)] = nus[j];
    }
    return;
  }
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    if (e0 + 4 <= n) {
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + e0));
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      if (EF) {
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(res + e0));
        v[j][0] = v[j][0] + b.x; v[j][1] = v[j][1] + b.y; v[j][2] = v[j][2] + b.z; v[j][3] = v[j][3] + b.w;
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        float t = 0.f;
        if (e0 + m < n) {
          t = x[e0 + m];
          if (EF) t = t + res[e0 + m];
        }
        v[j][m] = t;
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    // pairwise tree: lane-local levels, then the lane butterfly (every lane takes part;
    // lanes past the end hold +0.0)
    float ss = quad_sumsq(v[j]);
    ss = seg_tree_sum_c<LPG_LOG2>(ss);
    if (e0 >= n) continue;
    const bool full = e0 + 4 <= n;
    const float nu = sqrtf(ss);
    float u[4];
    uniforms4_t<ALIGNED>(seed, (uint64_t)(index_base + e0), u);
    int lev[4];
    float gh[4];
    qsgd_quad(v[j], nu, s, ys, u, lev, gh);
    if (full) {
      __builtin_nontemporal_store(pack_codes4(lev), reinterpret_cast<uint32_t*>(codes + e0));
      if (EF) {
        f32x4 r;
        r.x = v[j][0] - gh[0]; r.y = v[j][1] - gh[1]; r.z = v[j][2] - gh[2]; r.w = v[j][3] - gh[3];
        __builtin_nontemporal_store(r, reinterpret_cast<f32x4*>(res + e0));
      }
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (e0 + m < n) {
          codes[e0 + m] = (int8_t)lev[m];
          if (EF) res[e0 + m] = v[j][m] - gh[m];
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
  const int64_t blocks = (n + kTile - 1) / kTile;
  const float sf = (float)levels;
  const float ys = 1.0f / sf;
  // element e0 of a lane is a multiple of 4: its draw is one Philox block exactly when
  // index_base is a multiple of 4
  const bool aligned = (index_base & 3) == 0;
#define GC_QSGD(E, W)                                                                                        \
  do {                                                                                                      \
    if (aligned) hipLaunchKernelGGL((k_qsgd<E, W, true>), (int)blocks, kBlock, 0, s, x, res, n, sf, ys, seed,  \
                                    index_base, codes, norms);                                              \
    else hipLaunchKernelGGL((k_qsgd<E, W, false>), (int)blocks, kBlock, 0, s, x, res, n, sf, ys, seed,         \
                            index_base, codes, norms);                                                      \
  } while (0)
#define GC_QSGD_WIDTH(E)                  \
  switch (lpg_log2) {                     \
    case 0: GC_QSGD(E, 0); break;         \
    case 1: GC_QSGD(E, 1); break;         \
    case 2: GC_QSGD(E, 2); break;         \
    case 3: GC_QSGD(E, 3); break;         \
    case 4: GC_QSGD(E, 4); break;         \
    case 5: GC_QSGD(E, 5); break;         \
    default: GC_QSGD(E, 6); break;        \
  }
  if (res) { GC_QSGD_WIDTH(true) } else { GC_QSGD_WIDTH(false) }
#undef GC_QSGD_WIDTH
#undef GC_QSGD
  return hipGetLastError();
}

}  // namespace gc
