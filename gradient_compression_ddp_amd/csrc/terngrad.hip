// TernGrad: stochastic ternary codes with one scale per segment (layer), gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", section 1.1
// (codes in {-1,0,+1}, layer-wise normalization), with the per-layer scheme of the
// TernGrad paper the page cites: s = max|x|, code = sign(x) * Bernoulli(|x|/s).
//
// Two passes per batch of segments: (A) max|x'| per segment with one ordered atomic per
// block (|x'| >= 0, so its bit pattern orders like the value); (B) codes.  Pass B works in
// global quad space: lane L owns the aligned quad Q = qs + b0 + L, so loads are 16-byte
// vector loads and the Philox block of the quad is shared by its 4 elements.  A segment
// may start mid-quad (offset d = start & 3); its packed byte b then takes the top 4-d
// codes of quad qs+b and the bottom d codes of quad qs+b+1, which the wave stitches with
// one lane shuffle.  With d != 0 a run of 64 lanes emits 63 bytes and lane 63 only
// supplies the neighbour codes.
//
// Both passes keep kUnroll independent 16-byte loads in flight per lane.  All segments
// (up to 32 per launch) share one launch of each pass: grouping them so that pass B would
// re-read from the 256 MB memory-side cache measured slower on MI355X (launches of
// 60-170 MB each cost more than the cache saves).  Pass B is bound by its VALU work, a
// Philox4x32-10 block per quad, rather than by HBM.
#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kSegBatch = 32;
constexpr int kUnroll = 4;

struct SegBatch {
  int count;
  int index[kSegBatch];       // segment number (into scales)
  int64_t start[kSegBatch];   // first global position
  int64_t end[kSegBatch];     // one past the last position
  int64_t out_byte[kSegBatch];
};

__global__ void k_zero_f32(float* __restrict__ p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0.f;
}

template <bool EF>
__device__ __forceinline__ void load_quad_masked(const float* __restrict__ x,
                                                 const float* __restrict__ res, int64_t Q,
                                                 int64_t lo, int64_t hi, int64_t n, float v[4],
                                                 bool ok[4]) {
  const int64_t p0 = Q << 2;
  if (p0 + 4 <= n) {
    const float4 a = *reinterpret_cast<const float4*>(x + p0);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    if (EF) {
      const float4 b = *reinterpret_cast<const float4*>(res + p0);
      v[0] = v[0] + b.x; v[1] = v[1] + b.y; v[2] = v[2] + b.z; v[3] = v[3] + b.w;
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      float t = 0.f;
      if (p0 + m < n) {
        t = x[p0 + m];
        if (EF) t = t + res[p0 + m];
      }
      v[m] = t;
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) ok[m] = (p0 + m >= lo) && (p0 + m < hi);
}

template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_max(const float* __restrict__ x,
                                                     const float* __restrict__ res, int64_t n,
                                                     SegBatch sb, float* __restrict__ scales) {
  __shared__ uint32_t s_max[kBlock / kWave];
  const int si = blockIdx.y;
  const int64_t lo = sb.start[si], hi = sb.end[si];
  const int64_t q0 = lo >> 2, q1 = (hi + 3) >> 2;
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  uint32_t mx = 0u;
  for (int64_t Q = q0 + (int64_t)blockIdx.x * kBlock + threadIdx.x; Q < q1; Q += kUnroll * stride) {
    float v[kUnroll][4];
    bool ok[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t Qu = Q + u * stride;
      if (Qu < q1) {
        load_quad_masked<EF>(x, res, Qu, lo, hi, n, v[u], ok[u]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) { v[u][m] = 0.f; ok[u][m] = false; }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u)
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (ok[u][m]) mx = max(mx, fbits(fabsf(v[u][m])));
  }
  mx = seg_max_u32(mx, kWave);
  const int w = threadIdx.x / kWave;
  if (lane_id() == 0) s_max[w] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_max[0];
    for (int i = 1; i < kBlock / kWave; ++i) m = max(m, s_max[i]);
    if (m) atomicMax(reinterpret_cast<uint32_t*>(scales) + sb.index[si], m);
  }
}

template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_codes(const float* __restrict__ x,
                                                       float* __restrict__ res, int64_t n,
                                                       SegBatch sb, const float* __restrict__ scales,
                                                       uint64_t seed, int64_t index_base,
                                                       uint8_t* __restrict__ packed) {
  const int si = blockIdx.y;
  const int64_t lo = sb.start[si], hi = sb.end[si];
  const int64_t len = hi - lo;
  if (len <= 0) return;
  const int64_t nb = (len + 3) >> 2;                  // output bytes of the segment
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;        // bytes per wave run
  const int64_t qs = lo >> 2;
  const int64_t nq = ((hi + 3) >> 2) - qs;             // quads touched by the segment
  const int64_t runs = (nq + step - 1) / step;         // every touched quad has one owner
  const float sc = scales[sb.index[si]];
  const int lane = lane_id();
  uint8_t* __restrict__ out = packed + sb.out_byte[si];
  const int64_t waves = ((int64_t)gridDim.x * kBlock) >> 6;
  // The loop bound is uniform per wave, so every lane takes part in the shuffle.
  for (int64_t run = ((int64_t)blockIdx.x * kBlock + threadIdx.x) >> 6; run < runs; run += kUnroll * waves) {
    float v[kUnroll][4];
    bool ok[kUnroll][4];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t ru = run + u * waves;
      if (ru < runs) {
        load_quad_masked<EF>(x, res, qs + ru * step + lane, lo, hi, n, v[u], ok[u]);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) { v[u][m] = 0.f; ok[u][m] = false; }
      }
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int64_t ru = run + u * waves;
      if (ru >= runs) break;   // uniform across the wave
      const int64_t b0 = ru * step;
      const int64_t Q = qs + b0 + lane;
      float uu[4];
      uniforms4(seed, (uint64_t)(index_base + (Q << 2)), uu);
      uint32_t c8 = 0u;
      float gh[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        uint32_t bits = 0u;
        float g = 0.f;
        if (ok[u][m] && sc > 0.f) {
          const float p = fabsf(v[u][m]) / sc;
          if (uu[m] < p) {
            const bool neg = v[u][m] < 0.f;
            bits = neg ? 3u : 1u;
            g = neg ? -sc : sc;
          }
        }
        gh[m] = g;
        c8 |= bits << (2 * m);
      }
      const uint32_t nxt = (uint32_t)__shfl_down((int)c8, 1, kWave);
      const uint32_t byte = d == 0 ? c8 : (((c8 >> (2 * d)) | (nxt << (8 - 2 * d))) & 0xFFu);
      const bool owner = lane < step;
      if (owner && b0 + lane < nb) out[b0 + lane] = (uint8_t)byte;
      if (EF && owner) {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (ok[u][m]) res[(Q << 2) + m] = v[u][m] - gh[m];
      }
    }
  }
}

}  // namespace

size_t terngrad_workspace(int64_t, int) { return 0; }

hipError_t launch_terngrad(const float* x, float* res, int nseg, const int64_t* off,
                           uint64_t seed, int64_t index_base, uint8_t* packed, float* scales,
                           void*, hipStream_t s) {
  if (nseg == 0) return hipSuccess;
  hipLaunchKernelGGL(k_zero_f32, (nseg + 255) / 256, 256, 0, s, scales, nseg);
  const int64_t n = off[nseg];
  const int cus = device_cu_count();
  int64_t out_byte = 0;
  for (int b0 = 0; b0 < nseg;) {
    SegBatch sb{};
    const int cnt = nseg - b0 < kSegBatch ? nseg - b0 : kSegBatch;
    sb.count = cnt;
    int64_t maxlen = 0;
    for (int i = 0; i < sb.count; ++i) {
      sb.index[i] = b0 + i;
      sb.start[i] = off[b0 + i];
      sb.end[i] = off[b0 + i + 1];
      sb.out_byte[i] = out_byte;
      const int64_t len = sb.end[i] - sb.start[i];
      out_byte += (len + 3) / 4;
      if (len > maxlen) maxlen = len;
    }
    b0 += cnt;
    if (maxlen == 0) continue;
    // spread roughly 8 blocks per CU over the batch
    int64_t per_seg = ((int64_t)cus * 8 + sb.count - 1) / sb.count;
    const int64_t qmax = (maxlen + 7) / 4;
    int64_t gx = (qmax + kBlock - 1) / kBlock;
    if (gx > per_seg) gx = per_seg;
    if (gx < 1) gx = 1;
    const dim3 grid((unsigned)gx, (unsigned)sb.count);
    if (res) hipLaunchKernelGGL((k_tern_max<true>), grid, kBlock, 0, s, x, res, n, sb, scales);
    else hipLaunchKernelGGL((k_tern_max<false>), grid, kBlock, 0, s, x, res, n, sb, scales);
    const int64_t runs = (maxlen + 3) / 4 / (kWave - 1) + 1;
    int64_t gx2 = (runs + (kBlock / kWave) - 1) / (kBlock / kWave);
    if (gx2 > per_seg) gx2 = per_seg;
    if (gx2 < 1) gx2 = 1;
    const dim3 grid2((unsigned)gx2, (unsigned)sb.count);
    if (res) hipLaunchKernelGGL((k_tern_codes<true>), grid2, kBlock, 0, s, x, res, n, sb, scales, seed, index_base, packed);
    else hipLaunchKernelGGL((k_tern_codes<false>), grid2, kBlock, 0, s, x, res, n, sb, scales, seed, index_base, packed);
  }
  return hipGetLastError();
}

}  // namespace gc
