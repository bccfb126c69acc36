// TernGrad: stochastic ternary codes with one scale per segment (layer), gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", section 1.1
// (codes in {-1,0,+1}, layer-wise normalization), with the per-layer scheme of the
// TernGrad paper the page cites: s = max|x|, code = sign(x) * Bernoulli(|x|/s).
//
// The code of an element needs its layer's scale s, which is only known once the whole
// layer has been read; a second pass over the layer would read it twice (measured on
// MI355X: a second read of a 117 MB batch right after the first streams at 6.6-6.8 TB/s,
// the HBM rate, so the memory-side cache does not serve it).  Instead the input is read
// once:
//  1. sample   every 32nd 1 KB chunk of each segment raises the segment's maximum slots
//              (a lower bound of s: these are elements of the segment);
//  2. pass     one read of every element.  A block takes s_lo = max(its own maximum, the
//              sampled maxima) <= s, and adds it to the pass's maximum slots (apart from
//              the sampled ones: slots that every block both reads and updates serialise
//              the blocks, 2.4 ms against 0.3 ms for this pass on 350M elements).  An element whose
//              uniform U is at least fl(|x| / s_lo) has code 0 for the true s as well
//              (fl(|x|/s) <= fl(|x|/s_lo) <= U), and so does x = 0.  A code byte whose 4
//              elements are all settled is 0; any other byte is listed (its position and
//              its 4 values) in the tile's list.  The pass writes every code byte as 0
//              and, with error feedback, r = x + r everywhere (the settled elements'
//              final residual).
//  3. fix-up   with the final s (the maximum of both sets of slots), every listed byte is decided
//              exactly (U < fl(|x| / s), the IEEE division) and written, and the residual
//              of each +-1 element becomes x - sign(x) * s.  A tile whose list overflowed
//              is redone byte by byte from x (plain) or from the residual, which holds x
//              after step 2 (error feedback).
// With the sampled bound about 1% of the elements (4% of the bytes) of a t(3) layer are
// listed, so the traffic is one read of x (and r), the codes, and a few percent more.
//
// Layout (as before): lane L of a wave run owns the aligned global quad Q = qs + b0 + L,
// so loads are 16-byte vector loads and a quad's 4 elements share one Philox block.  A
// segment may start mid-quad (d = start & 3); its packed byte b then takes the top 4-d
// elements of quad qs+b and the bottom d of quad qs+b+1, which the wave stitches with
// lane shuffles; with d != 0 a run of 64 lanes owns 63 bytes.  Every byte of a segment
// and every element has exactly one owning lane in the pass and in the fix-up.
#include <vector>

#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;                  // 4
constexpr int kSegBatch = 32;                           // segments per launch at most
constexpr int kSlots = kWave;                           // maximum slots per segment
constexpr int kRunsB = 4;                               // wave runs per wave per tile
constexpr int kRunsPerBlock = kWaves * kRunsB;          // 16 runs of 64 quads per tile
constexpr int kCap = 128;                               // listed bytes per tile
constexpr int kSampleChunkQuads = kWave;                // a sampled chunk: 64 quads = 1 KB
constexpr int kSampleEvery = 32;                        // one chunk in 32

struct SegList {
  int count;
  uint32_t blk[kSegBatch + 1];  // exclusive prefix of this launch's blocks (or waves) per segment
  int index[kSegBatch];         // segment number (into scales and the slots)
  int64_t start[kSegBatch];     // first global position
  int64_t end[kSegBatch];       // one past the last position
  int64_t out_byte[kSegBatch];  // first packed byte
  int64_t tile0[kSegBatch];     // the segment's first tile in the workspace's tile arrays
};

__host__ __device__ inline int64_t cdiv64(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Tiles of a segment [lo, hi): runs of 64 quads (63 bytes when the start is not
// quad-aligned), 16 runs per tile.
__host__ __device__ inline int64_t seg_runs(int64_t lo, int64_t hi) {
  const int64_t nq = ((hi + 3) >> 2) - (lo >> 2);
  return hi > lo ? cdiv64(nq, (lo & 3) ? kWave - 1 : kWave) : 0;
}
__host__ __device__ inline int64_t seg_tiles(int64_t lo, int64_t hi) { return cdiv64(seg_runs(lo, hi), kRunsPerBlock); }

// Upper bound of the tiles of nseg segments holding n elements in all.
int64_t tiles_bound(int64_t n, int nseg) {
  return cdiv64(n / 4 + 2 * (int64_t)nseg, (int64_t)(kWave - 1) * kRunsPerBlock) + 2 * (int64_t)nseg + 1;
}

struct Work {
  uint32_t* samp;     // [nseg * kSlots] sampled maxima (|x| bits), written before the pass
  uint32_t* slots;    // [nseg * kSlots] the pass's maxima (|x| bits)
  uint32_t* tile_cnt; // [tiles] listed bytes of each tile (> kCap: overflowed)
  uint32_t* lst_b;    // [tiles * kCap] byte within its segment
  f32x4* lst_x;       // [tiles * kCap] the byte's 4 values (x + r), byte order
  size_t bytes;
};

Work work_layout(void* base, int64_t n, int nseg) {
  Work w{};
  const int64_t tiles = tiles_bound(n, nseg);
  char* b = reinterpret_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  w.samp = (uint32_t*)take((size_t)nseg * kSlots * sizeof(uint32_t));
  w.slots = (uint32_t*)take((size_t)nseg * kSlots * sizeof(uint32_t));
  w.tile_cnt = (uint32_t*)take((size_t)tiles * sizeof(uint32_t));
  w.lst_b = (uint32_t*)take((size_t)tiles * kCap * sizeof(uint32_t));
  w.lst_x = (f32x4*)take((size_t)tiles * kCap * sizeof(f32x4));
  w.bytes = off;
  return w;
}

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

// The segment of a launch's block (or wave) t: the largest si with blk[si] <= t.
__device__ __forceinline__ int seg_of(const SegList& L, uint32_t t) {
  int si = 0;
  while (si + 1 < L.count && L.blk[si + 1] <= t) ++si;
  return si;
}

// The 4 elements of packed byte b of a segment starting at lo: element j is position
// lo + 4b + j.  Its ternary code bits (00, 01, 11) under scale sc > 0 from the IEEE
// decision U < fl(|x| / sc), and the new residuals (x - code * sc).
__device__ __forceinline__ uint32_t byte_codes(const float xs[4], int nvalid, float sc, uint64_t seed,
                                               uint64_t e0, float rnew[4], bool take[4]) {
  float u[4];
  uniforms4(seed, e0, u);
  uint32_t byte = 0u;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    take[j] = false;
    rnew[j] = xs[j];
    if (j < nvalid && sc > 0.f && u[j] < fabsf(xs[j]) / sc) {
      const bool neg = xs[j] < 0.f;
      byte |= (neg ? 3u : 1u) << (2 * j);
      rnew[j] = xs[j] - (neg ? -sc : sc);
      take[j] = true;
    }
  }
  return byte;
}

// ---- 1: sampled maxima --------------------------------------------------------------
// Sampled chunk c of a segment: quads qs + c * 32 * 64 .. + 64, masked to the segment.
// Wave w of the launch takes chunks 4w' .. 4w' + 3 of its segment (w' its rank in the
// segment); their maximum |x| goes to sampled slot w' mod kSlots.
constexpr int kSampleChunksPerWave = 4;
template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_sample(const float* __restrict__ x, const float* __restrict__ res,
                                                        int64_t n, SegList S, uint32_t* __restrict__ samp) {
  const uint32_t wv = (uint32_t)((blockIdx.x * kBlock + threadIdx.x) / kWave);
  if (wv >= S.blk[S.count]) return;
  const int si = seg_of(S, wv);
  const int64_t lo = S.start[si], hi = S.end[si];
  const int64_t wr = (int64_t)(wv - S.blk[si]);
  uint32_t mx = 0u;
  float v[kSampleChunksPerWave][4];
  bool ok[kSampleChunksPerWave][4];
#pragma unroll
  for (int c = 0; c < kSampleChunksPerWave; ++c) {
    const int64_t Q = (lo >> 2) + (wr * kSampleChunksPerWave + c) * kSampleEvery * kSampleChunkQuads + lane_id();
#pragma unroll
    for (int m = 0; m < 4; ++m) { v[c][m] = 0.f; ok[c][m] = false; }
    if ((Q << 2) < hi) load_quad_masked<EF>(x, res, Q, lo, hi, n, v[c], ok[c]);
  }
#pragma unroll
  for (int c = 0; c < kSampleChunksPerWave; ++c)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (ok[c][m]) mx = max(mx, fbits(fabsf(v[c][m])));
  mx = seg_max_c<6>(mx);
  if (lane_id() == 0 && mx) atomicMax(samp + (int64_t)S.index[si] * kSlots + (wr & (kSlots - 1)), mx);
}

// ---- 2: the pass --------------------------------------------------------------------
// One wave's 4 runs.  FULL: every quad of the runs lies inside the segment (no masks, no
// bounds).  Every wave of the block calls this once and meets its one barrier, where the
// block's maximum is combined into the bound s_lo.
template <bool EF, bool ALIGNED, bool FULL>
__device__ __forceinline__ void pass_wave(const float* __restrict__ x, float* __restrict__ res, int64_t n,
                                          int64_t lo, int64_t hi, int64_t r0, int64_t runs, uint32_t sampled,
                                          uint32_t* __restrict__ slot, uint32_t* s_max, uint32_t* s_n,
                                          uint64_t seed, int64_t index_base, uint8_t* __restrict__ out,
                                          int64_t tile, uint32_t* __restrict__ lst_b, f32x4* __restrict__ lst_x) {
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;   // bytes per wave run
  const int64_t qs = lo >> 2;
  const int64_t nb = (hi - lo + 3) >> 2;         // output bytes of the segment
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
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
  // the block's maximum (with the sampled maxima, one slot per lane) into the pass's
  // slots, and the bound s_lo
  uint32_t mx = sampled;
#pragma unroll
  for (int u = 0; u < kRunsB; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (ok[u][m]) mx = max(mx, fbits(fabsf(v[u][m])));
  mx = seg_max_c<6>(mx);
  if (lane == 0) s_max[w] = mx;
  __syncthreads();
  const uint32_t lo_bits = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  if (threadIdx.x == 0 && lo_bits) atomicMax(slot + (blockIdx.x & (kSlots - 1)), lo_bits);
  const float rsc = 1.0f / bitsf(lo_bits);
#pragma unroll
  for (int u = 0; u < kRunsB; ++u) {
    const int64_t ru = r0 + u;
    if (!FULL && ru >= runs) break;   // uniform across the wave
    const int64_t b0 = ru * step;
    const int64_t Q = qs + b0 + lane;
    float uu[4];
    uniforms4_t<ALIGNED>(seed, (uint64_t)(index_base + (Q << 2)), uu);
    // settled: x = 0, or U >= fl(|x| / s_lo) (so code 0 under every s >= s_lo).
    // d = fl(fl(|x| * rsc) - U) lies within 2^-21 of fl(|x|/s_lo) - U (rsc's relative
    // error 2^-24, two roundings below 1 and the quotient's own), so d <= -2^-21 settles it
    uint32_t open = 0u;   // bit m: element m of the quad is not settled
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const float ax = fabsf(v[u][m]);
      const float dd = ax * rsc - uu[m];
      const bool settled = !ok[u][m] || ax == 0.f || dd <= -0x1p-21f;
      open |= settled ? 0u : (1u << m);
    }
    // byte b0 + lane: elements m >= d of this quad and m < d of the next
    const uint32_t nxt = (uint32_t)__shfl_down((int)open, 1, kWave);
    const uint32_t bopen = d == 0 ? open : (((open >> d) | (nxt << (4 - d))) & 0xFu);
    const bool owner = lane < step && (FULL || b0 + lane < nb);
    const bool listed = owner && bopen != 0u;
    if (owner) out[b0 + lane] = 0;
    const uint64_t lm = ballot(listed);
    if (lm) {
      // the byte's values: xs[j] = element j + d of this quad (j < 4 - d), else element
      // j + d - 4 of the next lane's quad.  d is uniform, and each case indexes with
      // constants (an index computed from d would put the arrays in scratch memory)
      float xs[4];
      if (d == 0) {
        xs[0] = v[u][0]; xs[1] = v[u][1]; xs[2] = v[u][2]; xs[3] = v[u][3];
      } else {
        float nv[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) nv[m] = __shfl_down(v[u][m], 1, kWave);
        if (d == 1) {
          xs[0] = v[u][1]; xs[1] = v[u][2]; xs[2] = v[u][3]; xs[3] = nv[0];
        } else if (d == 2) {
          xs[0] = v[u][2]; xs[1] = v[u][3]; xs[2] = nv[0]; xs[3] = nv[1];
        } else {
          xs[0] = v[u][3]; xs[1] = nv[0]; xs[2] = nv[1]; xs[3] = nv[2];
        }
      }
      uint32_t base = 0u;
      if (lane == 0) base = atomicAdd(s_n, (uint32_t)__popcll(lm));
      base = (uint32_t)__shfl((int)base, 0, kWave);
      const uint32_t pos = base + mbcnt(lm);
      if (listed && pos < kCap) {
        lst_b[tile * kCap + pos] = (uint32_t)(b0 + lane);
        lst_x[tile * kCap + pos] = f32x4{xs[0], xs[1], xs[2], xs[3]};
      }
    }
    if (EF) {
      // element m of this lane's quad belongs to byte lane (m >= d) or byte lane-1 (m < d);
      // the lane owning that byte writes its residual, so a quad shared by two runs is
      // split between them and no lane writes an element another lane writes
      if (FULL && (d == 0 || (lane >= 1 && lane <= kWave - 2))) {
        __builtin_nontemporal_store(f32x4{v[u][0], v[u][1], v[u][2], v[u][3]},
                                    reinterpret_cast<f32x4*>(res + (Q << 2)));
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const bool mine = d == 0 || (m >= d ? lane <= kWave - 2 : lane >= 1);
          if (ok[u][m] && mine) res[(Q << 2) + m] = v[u][m];
        }
      }
    }
  }
}

// Block t of the launch: tile bi of its segment, 16 runs of 64 quads (4 per wave).
template <bool EF, bool ALIGNED>
__global__ __launch_bounds__(kBlock) void k_tern_pass(const float* __restrict__ x, float* __restrict__ res,
                                                      int64_t n, SegList S, const uint32_t* __restrict__ samp,
                                                      uint32_t* __restrict__ slots, uint64_t seed, int64_t index_base,
                                                      uint8_t* __restrict__ packed, uint32_t* __restrict__ tile_cnt,
                                                      uint32_t* __restrict__ lst_b, f32x4* __restrict__ lst_x) {
  __shared__ uint32_t s_max[kWaves];
  __shared__ uint32_t s_n;
  const int si = seg_of(S, blockIdx.x);
  const int64_t bi = (int64_t)blockIdx.x - S.blk[si];
  const int64_t lo = S.start[si], hi = S.end[si];
  const int step = (lo & 3) == 0 ? kWave : kWave - 1;
  const int64_t qs = lo >> 2;
  const int64_t runs = seg_runs(lo, hi);
  const int64_t r0 = bi * kRunsPerBlock + (threadIdx.x / kWave) * kRunsB;
  const int64_t tile = S.tile0[si] + bi;
  uint32_t* __restrict__ slot = slots + (int64_t)S.index[si] * kSlots;
  // the sampled maxima: written by the sample launch, only read here (the pass's own
  // atomics go to the other slots, so these lines stay cached and uncontended)
  const uint32_t sampled = samp[(int64_t)S.index[si] * kSlots + lane_id()];
  uint8_t* __restrict__ out = packed + S.out_byte[si];
  if (threadIdx.x == 0) s_n = 0u;
  // the wave's runs read quads [qs + r0*step, qs + (r0 + kRunsB - 1)*step + 64)
  const bool full = ((qs + r0 * step) << 2) >= lo && ((qs + (r0 + kRunsB - 1) * step + kWave) << 2) <= hi;
  if (full)
    pass_wave<EF, ALIGNED, true>(x, res, n, lo, hi, r0, runs, sampled, slot, s_max, &s_n, seed, index_base, out,
                                 tile, lst_b, lst_x);
  else
    pass_wave<EF, ALIGNED, false>(x, res, n, lo, hi, r0, runs, sampled, slot, s_max, &s_n, seed, index_base, out,
                                  tile, lst_b, lst_x);
  __syncthreads();
  if (threadIdx.x == 0) tile_cnt[tile] = s_n;
}

// ---- 3: the fix-up ------------------------------------------------------------------
// Wave t of the launch: tile t of the batch.  Listed bytes are decided exactly; an
// overflowed tile is redone byte by byte over the bytes it owns.  Tile 0 of a segment
// also writes the segment's scale.
template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_fix(const float* __restrict__ x, float* __restrict__ res,
                                                     SegList S, const uint32_t* __restrict__ samp,
                                                     const uint32_t* __restrict__ slots,
                                                     float* __restrict__ scales, uint64_t seed, int64_t index_base,
                                                     uint8_t* __restrict__ packed, const uint32_t* __restrict__ tile_cnt,
                                                     const uint32_t* __restrict__ lst_b,
                                                     const f32x4* __restrict__ lst_x) {
  const uint32_t wt = (uint32_t)((blockIdx.x * kBlock + threadIdx.x) / kWave);
  if (wt >= S.blk[S.count]) return;
  const int si = seg_of(S, wt);
  const int64_t bi = (int64_t)(wt - S.blk[si]);
  const int64_t lo = S.start[si], hi = S.end[si];
  const int64_t nb = (hi - lo + 3) >> 2;
  const int lane = lane_id();
  const int64_t sl = (int64_t)S.index[si] * kSlots + lane;
  const float sc = bitsf(seg_max_c<6>(max(slots[sl], samp[sl])));
  if (bi == 0 && lane == 0) scales[S.index[si]] = sc;
  const int64_t tile = S.tile0[si] + bi;
  uint8_t* __restrict__ out = packed + S.out_byte[si];
  const uint32_t cnt = tile_cnt[tile];
  if (cnt <= (uint32_t)kCap) {
    for (uint32_t i = lane; i < cnt; i += kWave) {
      const int64_t b = lst_b[tile * kCap + i];
      const f32x4 q = lst_x[tile * kCap + i];
      const float xs[4] = {q.x, q.y, q.z, q.w};
      const int64_t p0 = lo + 4 * b;
      const int nvalid = (int)(hi - p0 < 4 ? hi - p0 : 4);
      float rnew[4];
      bool take[4];
      out[b] = (uint8_t)byte_codes(xs, nvalid, sc, seed, (uint64_t)(index_base + p0), rnew, take);
      if (EF) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (take[j]) res[p0 + j] = rnew[j];
      }
    }
    return;
  }
  // overflowed: every byte this tile owns, from x (or from the residual, which holds x + r)
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;
  const int64_t b_first = bi * kRunsPerBlock * step;
  int64_t b_last = b_first + (int64_t)kRunsPerBlock * step;
  if (b_last > nb) b_last = nb;
  const float* __restrict__ src = EF ? res : x;
  for (int64_t b = b_first + lane; b < b_last; b += kWave) {
    const int64_t p0 = lo + 4 * b;
    const int nvalid = (int)(hi - p0 < 4 ? hi - p0 : 4);
    float xs[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) xs[j] = j < nvalid ? src[p0 + j] : 0.f;
    float rnew[4];
    bool take[4];
    out[b] = (uint8_t)byte_codes(xs, nvalid, sc, seed, (uint64_t)(index_base + p0), rnew, take);
    if (EF) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        if (take[j]) res[p0 + j] = rnew[j];
    }
  }
}

}  // namespace

size_t terngrad_workspace(int64_t n, int nseg) {
  return (n > 0 && nseg > 0) ? work_layout(nullptr, n, nseg).bytes : 0;
}

hipError_t launch_terngrad(const float* x, float* res, int nseg, const int64_t* off,
                           uint64_t seed, int64_t index_base, uint8_t* packed, float* scales,
                           void* ws, hipStream_t s) {
  if (nseg == 0) return hipSuccess;
  const int64_t n = off[nseg];
  const Work w = work_layout(ws, n, nseg);
  // both slot sets are contiguous: clear them together
  const int64_t nslots = n > 0 ? 2 * (int64_t)nseg * kSlots : 0;
  static_assert(kSlots * sizeof(uint32_t) % 256 == 0, "the slot sets are adjacent");
  hipLaunchKernelGGL(k_zero2, (unsigned)((nslots + 255) / 256 + (nseg + 255) / 256), 256, 0, s, scales,
                     (int64_t)nseg, reinterpret_cast<float*>(w.samp), nslots);
  if (n == 0) return hipGetLastError();
  // the segments in batches of up to 32 per launch: the sample launches of every batch,
  // then the passes, then the fix-ups, so every pass sees every segment's sample
  std::vector<SegList> batches;
  int64_t out_byte = 0, tile = 0;
  for (int b0 = 0; b0 < nseg; b0 += kSegBatch) {
    SegList L{};
    L.count = nseg - b0 < kSegBatch ? nseg - b0 : kSegBatch;
    for (int c = 0; c < L.count; ++c) {
      const int i = b0 + c;
      L.index[c] = i;
      L.start[c] = off[i];
      L.end[c] = off[i + 1];
      L.out_byte[c] = out_byte;
      L.tile0[c] = tile;
      out_byte += (off[i + 1] - off[i] + 3) / 4;
      tile += seg_tiles(off[i], off[i + 1]);
    }
    batches.push_back(L);
  }
  for (SegList L : batches) {
    // one wave per sampled chunk
    L.blk[0] = 0;
    for (int c = 0; c < L.count; ++c) {
      const int64_t nq = L.end[c] > L.start[c] ? ((L.end[c] + 3) >> 2) - (L.start[c] >> 2) : 0;
      const int64_t chunks = cdiv64(nq, (int64_t)kSampleEvery * kSampleChunkQuads);
      L.blk[c + 1] = L.blk[c] + (uint32_t)cdiv64(chunks, kSampleChunksPerWave);
    }
    const int64_t waves = L.blk[L.count];
    if (waves == 0) continue;
    if (res) hipLaunchKernelGGL((k_tern_sample<true>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, n, L, w.samp);
    else hipLaunchKernelGGL((k_tern_sample<false>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, n, L, w.samp);
  }
  for (SegList L : batches) {
    L.blk[0] = 0;
    for (int c = 0; c < L.count; ++c) L.blk[c + 1] = L.blk[c] + (uint32_t)seg_tiles(L.start[c], L.end[c]);
    const int64_t blocks = L.blk[L.count];
    if (blocks == 0) continue;
#define GC_TERN_PASS(E, A)                                                                                    \
  hipLaunchKernelGGL((k_tern_pass<E, A>), (unsigned)blocks, kBlock, 0, s, x, res, n, L, (const uint32_t*)w.samp, \
                     w.slots, seed, index_base, packed, w.tile_cnt, w.lst_b, w.lst_x)
    // a lane's quad starts at a multiple of 4, so its element indices are aligned blocks of
    // the stream exactly when index_base is a multiple of 4
    const bool aligned = (index_base & 3) == 0;
    if (res) { if (aligned) GC_TERN_PASS(true, true); else GC_TERN_PASS(true, false); }
    else { if (aligned) GC_TERN_PASS(false, true); else GC_TERN_PASS(false, false); }
#undef GC_TERN_PASS
  }
  for (SegList L : batches) {
    // one wave per tile; segments without tiles still get their scale (0) from k_zero2
    L.blk[0] = 0;
    for (int c = 0; c < L.count; ++c) L.blk[c + 1] = L.blk[c] + (uint32_t)seg_tiles(L.start[c], L.end[c]);
    const int64_t waves = L.blk[L.count];
    if (waves == 0) continue;
    if (res) hipLaunchKernelGGL((k_tern_fix<true>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, L, (const uint32_t*)w.samp, (const uint32_t*)w.slots, scales, seed, index_base, packed, w.tile_cnt, w.lst_b, w.lst_x);
    else hipLaunchKernelGGL((k_tern_fix<false>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, L, (const uint32_t*)w.samp, (const uint32_t*)w.slots, scales, seed, index_base, packed, w.tile_cnt, w.lst_b, w.lst_x);
  }
  return hipGetLastError();
}

}  // namespace gc
