// TernGrad: stochastic ternary codes with one scale per segment (layer), gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", section 1.1
// (codes in {-1,0,+1}, layer-wise normalization), with the per-layer scheme of the
// TernGrad paper the page cites: s = max|x|, code = sign(x) * Bernoulli(|x|/s).
//
// Two passes over every segment: (A) max|x'| per segment, one ordered atomic per tile
// (|x'| >= 0, so its bit pattern orders like the value); (B) the codes.  Pass A is bound by
// HBM and pass B by its VALU work (a Philox4x32-10 block per quad and the decision
// U < fl(|x|/s), from a product estimate or the IEEE division), so they are pipelined over batches of segments: launch j runs the codes of
// batch j-1 and the maxima of batch j, their tiles interleaved in dispatch order, so that
// every CU mixes streaming tiles with arithmetic tiles.  Codes of batch j-1 only need
// the scales that launch j-1 finished; the first launch only takes maxima and the last only
// codes.  Both roles take one tile per block on a non-persistent grid (8192 elements for
// a max tile, 4096 for a code tile).
//
// Pass B works in global quad space: lane L owns the aligned quad Q = qs + b0 + L, so loads
// are 16-byte vector loads and the Philox block of the quad is shared by its 4 elements.
// A segment may start mid-quad (offset d = start & 3); its packed byte b then takes the
// top 4-d codes of quad qs+b and the bottom d codes of quad qs+b+1, which the wave
// stitches with one lane shuffle.  With d != 0 a run of 64 lanes emits 63 bytes and lane
// 63 only supplies the neighbour codes.  Tiles (pass A) and runs (pass B) that lie wholly
// inside their segment skip the per-element range masks.
//
// Pass A spreads each segment's atomics over 64 workspace slots, and pass B reduces the
// slots when it reads the scale: with one address per segment the tiles' atomics
// serialised (the max pass of 350M elements took 0.85 ms with 4096-element tiles; about
// 0.25 ms now).  Pass A loads through the caches, pass B with non-temporal loads, so that pass B
// does not evict the batch that pass A has just read (0.52 against 0.56 ms).
#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;                  // 4
constexpr int kSegBatch = 32;                           // segments per batch at most
constexpr int kQuadsA = 8;                              // pass A: quads per thread per tile
constexpr int64_t kTileQuadsA = (int64_t)kBlock * kQuadsA;   // 2048 quads = 8192 elements
// Pass A spreads the atomics of a segment over this many slots (tile index mod kSlots);
// pass B takes the max of the slots.
constexpr int kSlots = kWave;
constexpr int kRunsB = 4;                               // pass B: wave runs per wave per tile
constexpr int kRunsPerBlock = kWaves * kRunsB;          // 16 runs of 64 quads
// A batch is closed once it holds this many elements (or kSegBatch segments).  On the
// 24 x 14,583,333 workload, batches of two layers (117 MB) measured fastest on MI355X:
// 0.52 ms per call against 0.57-0.64 ms with 1, 3 or 5 layers and 0.62 ms with one batch
// (no overlap); the previous two-kernel form took 0.73 ms.
constexpr int64_t kBatchElems = int64_t(1) << 24;

struct SegList {
  int count;
  uint32_t blk[kSegBatch + 1];  // exclusive prefix of this role's tiles over the segments
  int index[kSegBatch];         // segment number (into scales)
  int64_t start[kSegBatch];     // first global position
  int64_t end[kSegBatch];       // one past the last position
  int64_t out_byte[kSegBatch];  // first packed byte
};

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

__global__ void k_zero2(float* __restrict__ a, int64_t na, float* __restrict__ b, int64_t nb) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < na) a[i] = 0.f;
  if (i < nb) b[i] = 0.f;
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

// The segment of a role's tile t: the largest si with blk[si] <= t (uniform per block).
__device__ __forceinline__ int seg_of(const SegList& L, uint32_t t) {
  int si = 0;
  while (si + 1 < L.count && L.blk[si + 1] <= t) ++si;
  return si;
}

// Pass A: max |x'| over the tile bi of segment si, then one atomic on the segment's slot
// bi mod kSlots.
template <bool EF>
__device__ __forceinline__ void max_tile(const float* __restrict__ x, const float* __restrict__ res,
                                         int64_t n, const SegList& A, int si, int64_t bi,
                                         uint32_t* __restrict__ slots, uint32_t* s_max) {
  const int64_t lo = A.start[si], hi = A.end[si];
  const int64_t qa = (lo >> 2) + bi * kTileQuadsA;
  const int64_t q1 = (hi + 3) >> 2;
  uint32_t mx = 0u;
  if ((qa << 2) >= lo && ((qa + kTileQuadsA) << 2) <= hi) {
    float4 v[kQuadsA], r[kQuadsA];
#pragma unroll
    for (int u = 0; u < kQuadsA; ++u) {
      const int64_t p0 = (qa + u * kBlock + threadIdx.x) << 2;
      v[u] = *reinterpret_cast<const float4*>(x + p0);
      if (EF) r[u] = *reinterpret_cast<const float4*>(res + p0);
    }
#pragma unroll
    for (int u = 0; u < kQuadsA; ++u) {
      if (EF) { v[u].x = v[u].x + r[u].x; v[u].y = v[u].y + r[u].y; v[u].z = v[u].z + r[u].z; v[u].w = v[u].w + r[u].w; }
      mx = max(mx, max(max(fbits(fabsf(v[u].x)), fbits(fabsf(v[u].y))),
                       max(fbits(fabsf(v[u].z)), fbits(fabsf(v[u].w)))));
    }
  } else {
#pragma unroll
    for (int u = 0; u < kQuadsA; ++u) {
      const int64_t Q = qa + u * kBlock + threadIdx.x;
      if (Q < q1) {
        float v[4];
        bool ok[4];
        load_quad_masked<EF>(x, res, Q, lo, hi, n, v, ok);
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (ok[m]) mx = max(mx, fbits(fabsf(v[m])));
      }
    }
  }
  mx = seg_max_u32(mx, kWave);
  if (lane_id() == 0) s_max[threadIdx.x / kWave] = mx;
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t m = s_max[0];
    for (int i = 1; i < kWaves; ++i) m = max(m, s_max[i]);
    if (m) atomicMax(slots + (int64_t)A.index[si] * kSlots + (bi & (kSlots - 1)), m);
  }
}

// Pass B: codes (and the residual) of the kRunsB wave runs of this wave in tile bi of
// segment si.  FULL: every quad of the runs lies inside the segment.
template <bool EF, bool FULL>
__device__ __forceinline__ void codes_runs(const float* __restrict__ x, float* __restrict__ res,
                                           int64_t n, int64_t lo, int64_t hi, int64_t r0,
                                           int64_t runs, float sc, float rsc, uint64_t seed,
                                           int64_t index_base, uint8_t* __restrict__ out) {
  const int64_t nb = (hi - lo + 3) >> 2;              // output bytes of the segment
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;        // bytes per wave run
  const int64_t qs = lo >> 2;
  const int lane = lane_id();
  float v[kRunsB][4];
  bool ok[kRunsB][4];
#pragma unroll
  for (int u = 0; u < kRunsB; ++u) {
    const int64_t Q = qs + (r0 + u) * step + lane;
    if (FULL) {
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + (Q << 2)));
      v[u][0] = a.x; v[u][1] = a.y; v[u][2] = a.z; v[u][3] = a.w;
      if (EF) {
        const f32x4 b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(res + (Q << 2)));
        v[u][0] = v[u][0] + b.x; v[u][1] = v[u][1] + b.y; v[u][2] = v[u][2] + b.z; v[u][3] = v[u][3] + b.w;
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) ok[u][m] = true;
    } else if (r0 + u < runs) {
      load_quad_masked<EF>(x, res, Q, lo, hi, n, v[u], ok[u]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) { v[u][m] = 0.f; ok[u][m] = false; }
    }
  }
#pragma unroll
  for (int u = 0; u < kRunsB; ++u) {
    const int64_t ru = r0 + u;
    if (!FULL && ru >= runs) break;   // uniform across the wave
    const int64_t b0 = ru * step;
    const int64_t Q = qs + b0 + lane;
    float uu[4];
    uniforms4(seed, (uint64_t)(index_base + (Q << 2)), uu);
    // U < p, p = fl(|x'| / sc) <= 1: d = fl(fl(|x'| * rsc) - U), rsc = fl(1/sc), lies within
    // 2^-22 + 2^-25 + 2^-25 < 2^-21 of p - U (rsc's relative error 2^-24, two roundings
    // below 1 and p's own), so d's sign decides when 2^-21 <= |d| <= 2; otherwise (and for
    // NaN or infinite d) the quad divides
    bool take[4];
    bool slow = false;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float d = fabsf(v[u][m]) * rsc - uu[m];
      take[m] = d > 0.f;
      slow |= !(fabsf(d) >= 0x1p-21f && fabsf(d) <= 2.0f);
    }
    if (slow) {
#pragma unroll
      for (int m = 0; m < 4; ++m) take[m] = uu[m] < fabsf(v[u][m]) / sc;
    }
    uint32_t c8 = 0u;
    float gh[4];
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      uint32_t bits = 0u;
      float g = 0.f;
      if (ok[u][m] && sc > 0.f) {
        if (take[m]) {
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
    if (owner && (FULL || b0 + lane < nb)) out[b0 + lane] = (uint8_t)byte;
    if (EF) {
      // Element m of this lane's quad goes to byte lane (m >= d) or byte lane-1 (m < d), and
      // the lane whose byte takes it is the one that writes its residual: lanes 0..62
      // write m >= d, lanes 1..63 write m < d.  A quad shared by two runs (lane 63 of one,
      // lane 0 of the next, possibly in another wave) is then split between them, so no
      // lane uses an element that another lane writes.
      if (FULL && (d == 0 || (lane >= 1 && lane <= kWave - 2))) {
        float4 r;
        r.x = v[u][0] - gh[0]; r.y = v[u][1] - gh[1]; r.z = v[u][2] - gh[2]; r.w = v[u][3] - gh[3];
        *reinterpret_cast<float4*>(res + (Q << 2)) = r;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bool mine = d == 0 || (m >= d ? lane <= kWave - 2 : lane >= 1);
          if (ok[u][m] && mine) res[(Q << 2) + m] = v[u][m] - gh[m];
        }
      }
    }
  }
}

template <bool EF>
__device__ __forceinline__ void codes_tile(const float* __restrict__ x, float* __restrict__ res,
                                           int64_t n, const SegList& B, int si, int64_t bi,
                                           const uint32_t* __restrict__ slots,
                                           float* __restrict__ scales, uint64_t seed,
                                           int64_t index_base, uint8_t* __restrict__ packed) {
  const int64_t lo = B.start[si], hi = B.end[si];
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;
  const int64_t qs = lo >> 2;
  const int64_t nq = ((hi + 3) >> 2) - qs;            // quads touched by the segment
  const int64_t runs = cdiv64(nq, step);              // every touched quad has one owner
  // the segment's scale: the max of its slots (every wave takes it; tile 0 stores it)
  const uint32_t sb = seg_max_u32(slots[(int64_t)B.index[si] * kSlots + lane_id()], kWave);
  const float sc = bitsf(sb);
  if (bi == 0 && threadIdx.x == 0) scales[B.index[si]] = sc;
  const float rsc = 1.0f / sc;
  uint8_t* __restrict__ out = packed + B.out_byte[si];
  const int64_t r0 = bi * kRunsPerBlock + (threadIdx.x / kWave) * kRunsB;
  if (r0 >= runs) return;
  // the wave's runs read quads [qs + r0*step, qs + (r0 + kRunsB - 1)*step + 64)
  const int64_t qlast = qs + (r0 + kRunsB - 1) * step + kWave;
  if (((qs + r0 * step) << 2) >= lo && (qlast << 2) <= hi)
    codes_runs<EF, true>(x, res, n, lo, hi, r0, runs, sc, rsc, seed, index_base, out);
  else
    codes_runs<EF, false>(x, res, n, lo, hi, r0, runs, sc, rsc, seed, index_base, out);
}

// One pipelined launch: the codes tiles of batch B and the max tiles of batch A, mixed in
// dispatch order in proportion to their counts.
template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_step(const float* __restrict__ x,
                                                      float* __restrict__ res, int64_t n,
                                                      SegList A, SegList B,
                                                      uint32_t* __restrict__ slots,
                                                      float* __restrict__ scales, uint64_t seed,
                                                      int64_t index_base,
                                                      uint8_t* __restrict__ packed) {
  __shared__ uint32_t s_max[kWaves];
  const uint64_t nA = A.blk[A.count], nB = B.blk[B.count];
  const uint64_t b = blockIdx.x, N = nA + nB;
  // tiles of A before block b: floor(b * nA / N); block b is an A tile iff that count
  // grows at b, so the A tiles and the B tiles each come in their own order.
  const uint64_t a0 = b * nA / N, a1 = (b + 1) * nA / N;
  if (a1 > a0) {
    const int si = seg_of(A, (uint32_t)a0);
    max_tile<EF>(x, res, n, A, si, (int64_t)(a0 - A.blk[si]), slots, s_max);
  } else {
    const uint32_t t = (uint32_t)(b - a0);
    const int si = seg_of(B, t);
    codes_tile<EF>(x, res, n, B, si, (int64_t)(t - B.blk[si]), slots, scales, seed, index_base, packed);
  }
}

void launch_step(const float* x, float* res, int64_t n, const SegList& A, const SegList& B,
                 uint32_t* slots, float* scales, uint64_t seed, int64_t index_base, uint8_t* packed,
                 hipStream_t s) {
  const uint64_t N = (uint64_t)A.blk[A.count] + B.blk[B.count];
  if (N == 0) return;
  if (res) hipLaunchKernelGGL((k_tern_step<true>), dim3((unsigned)N), kBlock, 0, s, x, res, n, A, B, slots, scales, seed, index_base, packed);
  else hipLaunchKernelGGL((k_tern_step<false>), dim3((unsigned)N), kBlock, 0, s, x, res, n, A, B, slots, scales, seed, index_base, packed);
}

}  // namespace

size_t terngrad_workspace(int64_t n, int nseg) {
  return (n > 0 && nseg > 0) ? align256((size_t)nseg * kSlots * sizeof(uint32_t)) : 0;
}

hipError_t launch_terngrad(const float* x, float* res, int nseg, const int64_t* off,
                           uint64_t seed, int64_t index_base, uint8_t* packed, float* scales,
                           void* ws, hipStream_t s) {
  if (nseg == 0) return hipSuccess;
  const int64_t n = off[nseg];
  uint32_t* slots = static_cast<uint32_t*>(ws);
  const int64_t nslots = n > 0 ? (int64_t)nseg * kSlots : 0;
  hipLaunchKernelGGL(k_zero2, (unsigned)((nslots + 255) / 256 + (nseg + 255) / 256), 256, 0, s, scales,
                     (int64_t)nseg, reinterpret_cast<float*>(slots), nslots);
  if (n == 0) return hipGetLastError();
  SegList prev{}, curA{}, curB{};   // count 0, blk[0] 0: no tiles
  int64_t out_byte = 0;
  for (int b0 = 0; b0 < nseg;) {
    curA = SegList{};
    curB = SegList{};
    int64_t elems = 0;
    int cnt = 0;
    while (b0 + cnt < nseg && cnt < kSegBatch && (cnt == 0 || elems < kBatchElems)) {
      const int i = b0 + cnt;
      const int64_t lo = off[i], hi = off[i + 1], len = hi - lo;
      for (SegList* L : {&curA, &curB}) {
        L->index[cnt] = i;
        L->start[cnt] = lo;
        L->end[cnt] = hi;
        L->out_byte[cnt] = out_byte;
      }
      int64_t ta = 0, tb = 0;
      if (len > 0) {
        const int64_t nq = ((hi + 3) >> 2) - (lo >> 2);
        ta = cdiv64(nq, kTileQuadsA);
        tb = cdiv64(cdiv64(nq, (lo & 3) ? kWave - 1 : kWave), kRunsPerBlock);
      }
      curA.blk[cnt + 1] = curA.blk[cnt] + (uint32_t)ta;
      curB.blk[cnt + 1] = curB.blk[cnt] + (uint32_t)tb;
      out_byte += (len + 3) / 4;
      elems += len;
      ++cnt;
    }
    curA.count = cnt;
    curB.count = cnt;
    b0 += cnt;
    launch_step(x, res, n, curA, prev, slots, scales, seed, index_base, packed, s);
    prev = curB;
  }
  launch_step(x, res, n, SegList{}, prev, slots, scales, seed, index_base, packed, s);
  return hipGetLastError();
}

}  // namespace gc
