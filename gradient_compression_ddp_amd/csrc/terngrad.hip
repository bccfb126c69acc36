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
constexpr int kRunsB = 8;                               // wave runs per wave per tile
constexpr int kRunsPerBlock = kWaves * kRunsB;          // 16 runs of 64 quads per tile
constexpr int kCap = 64;                                // listed bytes per wave list
constexpr int kFixLists = 16;                           // wave lists per fix-up wave
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
// quad-aligned), 16 runs per tile, 4 per wave.
__host__ __device__ inline int64_t seg_runs(int64_t lo, int64_t hi) {
  const int64_t nq = ((hi + 3) >> 2) - (lo >> 2);
  return hi > lo ? cdiv64(nq, (lo & 3) ? kWave - 1 : kWave) : 0;
}
__host__ __device__ inline int64_t seg_tiles(int64_t lo, int64_t hi) { return cdiv64(seg_runs(lo, hi), kRunsPerBlock); }

// Upper bound of the tiles of nseg segments holding n elements in all.
int64_t tiles_bound(int64_t n, int nseg) {
  return cdiv64(n / 4 + 2 * (int64_t)nseg, (int64_t)(kWave - 1) * kRunsPerBlock) + 2 * (int64_t)nseg + 1;
}

// One list per wave of the pass: wave w of tile t owns list t * kWaves + w.
struct Work {
  uint32_t* samp;     // [nseg * kSlots] sampled maxima (|x| bits), written before the pass
  uint32_t* slots;    // [nseg * kSlots] the pass's maxima (|x| bits)
  uint32_t* cnt;      // [lists] listed bytes of each wave list (> kCap: overflowed)
  uint32_t* lst_b;    // [lists * kCap] byte within its segment
  f32x4* lst_x;       // [lists * kCap] the byte's 4 values (x + r), byte order
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
  const size_t lists = (size_t)tiles * kWaves;
  w.cnt = (uint32_t*)take(lists * sizeof(uint32_t));
  w.lst_b = (uint32_t*)take(lists * kCap * sizeof(uint32_t));
  w.lst_x = (f32x4*)take(lists * kCap * sizeof(f32x4));
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

// The segment of a launch's block (or wave) t: the largest si < count with blk[si] <= t
// (blk is nondecreasing, blk[0] = 0), by bisection: at most 5 dependent reads of the
// kernel argument instead of one per segment.
__device__ __forceinline__ int seg_of(const SegList& L, uint32_t t) {
  int a = 0, b = L.count - 1;
  while (a < b) {
    const int mid = (a + b + 1) >> 1;
    if (L.blk[mid] <= t) a = mid; else b = mid - 1;
  }
  return a;
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

// The value of the next lane (lane 63 gets 0): a DPP wave shift by one lane.
__device__ __forceinline__ float next_lane(float v) {
  return bitsf((uint32_t)__builtin_amdgcn_update_dpp(0, (int)fbits(v), 0x130, 0xF, 0xF, false));
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
// Segments whose start is D elements past a multiple of 4 (D is a template argument: the
// byte stitching and the masks below are then fixed at compile time).

// The block's bound s_lo: the maximum of fm over the block (fm holds a wave's |x| maximum
// and the sampled maxima) goes to the pass's slots; returns fl(1/s_lo) * 2^32 (inf when
// s_lo is 0 or below 2^-96).  Every wave of the block calls this once.
__device__ __forceinline__ float block_bound(float fm, uint32_t* __restrict__ slot, uint32_t* s_max) {
  // |x| >= 0, so the order of the bit patterns is the order of the values
  const uint32_t mx = seg_max_c<6>(fbits(fm));
  if (lane_id() == 0) s_max[threadIdx.x / kWave] = mx;
  __syncthreads();
  const uint32_t lo_bits = max(max(s_max[0], s_max[1]), max(s_max[2], s_max[3]));
  if (threadIdx.x == 0 && lo_bits) atomicMax(slot + (blockIdx.x & (kSlots - 1)), lo_bits);
  return (1.0f / bitsf(lo_bits)) * 0x1p32f;
}

// One wave run: bytes b0 .. b0 + 62 (or 63) of the segment from the lane's quad q0 + lane
// (values vq, ok: inside the segment).  Writes the bytes as 0, lists the unsettled ones
// (nl: the wave's count so far, uniform) and, with error feedback, r = x + r.
template <bool EF, bool ALIGNED, int D, bool FULL>
__device__ __forceinline__ void run_pass(f32x4 vq, const bool ok[4], int64_t b0, int64_t q0, int64_t nb,
                                         float rsc32, uint64_t seed, int64_t index_base, uint8_t* __restrict__ out,
                                         float* __restrict__ res, uint32_t& nl, uint32_t* __restrict__ lst_b,
                                         f32x4* __restrict__ lst_x) {
  constexpr int step = D == 0 ? kWave : kWave - 1;
  const int lane = lane_id();
  uint32_t wd[4];
  if constexpr (ALIGNED) {
    // index_base % 4 == 0: the lane's quad is Philox block index_base / 4 + q0 + lane
    const Words4 a = philox_block(seed, (uint64_t)((index_base >> 2) + q0) + (uint32_t)lane);
#pragma unroll
    for (int m = 0; m < 4; ++m) wd[m] = a.w[m];
  } else {
    words4_t<false>(seed, (uint64_t)(index_base + ((q0 + lane) << 2)), wd);
  }
  // Settled: U >= q = fl(|x| / s_lo), U = (w >> 8) * 2^-24; then the code is 0 under
  // every scale s >= s_lo, since fl(|x| / s) <= q.  Let Q = |x| / s_lo <= 1 (s_lo is at
  // least this block's own maximum).  rsc32 is within 2^-24 relative (or 2^-118
  // absolute, in the subnormal range) of 2^32 / s_lo, the fused add rounds once, and q
  // is within 2^-24 relative of Q, so F = fl(|x| * rsc32 + 8192) >= q * 2^32 + 6000.
  // fl(w) is within 128 of w and (w >> 8) * 2^8 >= w - 255, so fl(w) > F gives U > q.
  // An element is open (unsettled) when F >= fl(w); x = 0 with rsc32 = inf gives
  // F = NaN: settled, correctly (its code is 0).  Each element's test is a lane mask,
  // and a byte's mask is stitched from them with scalar operations.
  uint64_t om[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) om[m] = ballot(ok[m] && fmaf(fabsf(vq[m]), rsc32, 8192.0f) >= (float)wd[m]);
  // byte b0 + lane: elements m >= D of this lane's quad and m < D of the next lane's
  uint64_t hi_m = 0ull, lo_m = 0ull;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    if (m >= D) hi_m |= om[m]; else lo_m |= om[m];
  }
  const uint64_t own = FULL ? (D == 0 ? ~0ull : (~0ull >> 1)) : ballot(lane < step && b0 + lane < nb);
  const uint64_t lm = (hi_m | (lo_m >> 1)) & own;
  if (__builtin_amdgcn_inverse_ballot_w64(own)) (out + b0)[lane] = 0;
  if (lm) {
    // the byte's values: elements D.. of this quad, then elements ..D-1 of the next
    // lane's quad (a wave shift by one lane)
    f32x4 xs;
    if constexpr (D == 0) {
      xs = vq;
    } else if constexpr (D == 1) {
      xs = f32x4{vq.y, vq.z, vq.w, next_lane(vq.x)};
    } else if constexpr (D == 2) {
      xs = f32x4{vq.z, vq.w, next_lane(vq.x), next_lane(vq.y)};
    } else {
      xs = f32x4{vq.w, next_lane(vq.x), next_lane(vq.y), next_lane(vq.z)};
    }
    const uint32_t pos = __builtin_amdgcn_mbcnt_hi((uint32_t)(lm >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)lm, nl));
    if (__builtin_amdgcn_inverse_ballot_w64(lm) && pos < kCap) {
      lst_b[pos] = (uint32_t)b0 + (uint32_t)lane;
      lst_x[pos] = xs;
    }
    nl += (uint32_t)__popcll(lm);
  }
  if (EF) {
    // element m of this lane's quad belongs to byte lane (m >= D) or byte lane-1 (m < D);
    // the lane owning that byte writes its residual, so a quad shared by two runs is
    // split between them and no lane writes an element another lane writes
    float* __restrict__ rq = res + (q0 << 2);
    if (FULL && (D == 0 || (lane >= 1 && lane <= kWave - 2))) {
      __builtin_nontemporal_store(vq, reinterpret_cast<f32x4*>(rq) + lane);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bool mine = D == 0 || (m >= D ? lane <= kWave - 2 : lane >= 1);
        if (ok[m] && mine) rq[4 * lane + m] = vq[m];
      }
    }
  }
}

// A wave's 4 runs when every quad of them lies inside the segment: loaded once, kept in
// registers across the block's barrier.
template <bool EF, bool ALIGNED, int D>
__device__ __forceinline__ void pass_wave_full(const float* __restrict__ x, float* __restrict__ res, int64_t lo,
                                               int64_t hi, int64_t r0, uint32_t sampled, uint32_t* __restrict__ slot,
                                               uint32_t* s_max, uint64_t seed, int64_t index_base,
                                               uint8_t* __restrict__ out, uint32_t* __restrict__ cnt_out,
                                               uint32_t* __restrict__ lst_b, f32x4* __restrict__ lst_x) {
  constexpr int step = D == 0 ? kWave : kWave - 1;
  const int64_t qs = lo >> 2;
  const int64_t nb = (hi - lo + 3) >> 2;
  const int lane = lane_id();
  f32x4 v[kRunsB];
#pragma unroll
  for (int u = 0; u < kRunsB; ++u) {
    const int64_t q0 = qs + (r0 + u) * step;   // the run's first quad (uniform)
    v[u] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(x + (q0 << 2)) + lane);
    if (EF) v[u] = v[u] + __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(res + (q0 << 2)) + lane);
  }
  float fm = bitsf(sampled);
#pragma unroll
  for (int u = 0; u < kRunsB; ++u)
#pragma unroll
    for (int m = 0; m < 4; ++m) fm = fmaxf(fm, fabsf(v[u][m]));
  const float rsc32 = block_bound(fm, slot, s_max);
  const bool all[4] = {true, true, true, true};
  uint32_t nl = 0u;
#pragma unroll
  for (int u = 0; u < kRunsB; ++u) {
    const int64_t b0 = (r0 + u) * step;
    run_pass<EF, ALIGNED, D, true>(v[u], all, b0, qs + b0, nb, rsc32, seed, index_base, out, res, nl, lst_b, lst_x);
  }
  if (lane == 0) *cnt_out = nl;
}

// A wave's runs at a segment's edges (masked to the segment, possibly fewer than 4): the
// values are loaded for the maximum, then again run by run after the barrier, so that few
// registers stay live (the kernel's register count, and so its occupancy, is the larger
// of this path's and the full path's).
template <bool EF, bool ALIGNED, int D>
__device__ __forceinline__ void pass_wave_edge(const float* __restrict__ x, float* __restrict__ res, int64_t n,
                                            int64_t lo, int64_t hi, int64_t r0, int64_t runs, uint32_t sampled,
                                            uint32_t* __restrict__ slot, uint32_t* s_max, uint64_t seed,
                                            int64_t index_base, uint8_t* __restrict__ out,
                                            uint32_t* __restrict__ cnt_out, uint32_t* __restrict__ lst_b,
                                            f32x4* __restrict__ lst_x) {
  constexpr int step = D == 0 ? kWave : kWave - 1;
  const int64_t qs = lo >> 2;
  const int64_t nb = (hi - lo + 3) >> 2;
  const int lane = lane_id();
  const int nr = (int)(runs - r0 < kRunsB ? (runs - r0 > 0 ? runs - r0 : 0) : kRunsB);
  float fm = bitsf(sampled);
#pragma unroll 1
  for (int u = 0; u < nr; ++u) {
    float t[4];
    bool ok[4];
    load_quad_masked<EF>(x, res, qs + (r0 + u) * step + lane, lo, hi, n, t, ok);
#pragma unroll
    for (int m = 0; m < 4; ++m) fm = fmaxf(fm, ok[m] ? fabsf(t[m]) : 0.f);
  }
  const float rsc32 = block_bound(fm, slot, s_max);
  uint32_t nl = 0u;
#pragma unroll 1
  for (int u = 0; u < nr; ++u) {
    const int64_t b0 = (r0 + u) * step;
    float t[4];
    bool ok[4];
    load_quad_masked<EF>(x, res, qs + b0 + lane, lo, hi, n, t, ok);
    run_pass<EF, ALIGNED, D, false>(f32x4{t[0], t[1], t[2], t[3]}, ok, b0, qs + b0, nb, rsc32, seed, index_base,
                                    out, res, nl, lst_b, lst_x);
  }
  if (lane == 0) *cnt_out = nl;
}

// Block t of the launch: tile bi of its segment, 16 runs of 64 quads (4 per wave).  Every
// segment of the launch starts D elements past a multiple of 4.
template <bool EF, bool ALIGNED, int D>
__global__ __launch_bounds__(kBlock) void k_tern_pass(const float* __restrict__ x, float* __restrict__ res,
                                                      int64_t n, SegList S, const uint32_t* __restrict__ samp,
                                                      uint32_t* __restrict__ slots, uint64_t seed, int64_t index_base,
                                                      uint8_t* __restrict__ packed, uint32_t* __restrict__ cnt,
                                                      uint32_t* __restrict__ lst_b, f32x4* __restrict__ lst_x) {
  constexpr int step = D == 0 ? kWave : kWave - 1;
  __shared__ uint32_t s_max[kWaves];
  const int si = seg_of(S, blockIdx.x);
  const int64_t bi = (int64_t)blockIdx.x - S.blk[si];
  const int64_t lo = S.start[si], hi = S.end[si];
  const int64_t qs = lo >> 2;
  const int64_t runs = seg_runs(lo, hi);
  const int w = threadIdx.x / kWave;
  const int64_t r0 = bi * kRunsPerBlock + w * kRunsB;
  const int64_t list = (S.tile0[si] + bi) * kWaves + w;
  uint32_t* __restrict__ slot = slots + (int64_t)S.index[si] * kSlots;
  // the sampled maxima: written by the sample launch, only read here (the pass's own
  // atomics go to the other slots, so these lines stay cached and uncontended)
  const uint32_t sampled = samp[(int64_t)S.index[si] * kSlots + lane_id()];
  uint8_t* __restrict__ out = packed + S.out_byte[si];
  // the wave's runs read quads [qs + r0*step, qs + (r0 + kRunsB - 1)*step + 64)
  const bool full = ((qs + r0 * step) << 2) >= lo && ((qs + (r0 + kRunsB - 1) * step + kWave) << 2) <= hi;
  if (full)
    pass_wave_full<EF, ALIGNED, D>(x, res, lo, hi, r0, sampled, slot, s_max, seed, index_base, out, cnt + list,
                                   lst_b + list * kCap, lst_x + list * kCap);
  else
    pass_wave_edge<EF, ALIGNED, D>(x, res, n, lo, hi, r0, runs, sampled, slot, s_max, seed, index_base, out,
                                   cnt + list, lst_b + list * kCap, lst_x + list * kCap);
}

// ---- 3: the fix-up ------------------------------------------------------------------
// Wave t of the launch: kFixLists consecutive wave lists of one segment.  Their entries
// are laid out densely over the lanes (an LDS table maps entry f to its list and slot),
// decided exactly and written.  A list that overflowed is redone byte by byte over the
// bytes of its wave's runs.  The first wave of a segment also writes the segment's scale.
template <bool EF>
__global__ __launch_bounds__(kBlock) void k_tern_fix(const float* __restrict__ x, float* __restrict__ res,
                                                     SegList S, const uint32_t* __restrict__ samp,
                                                     const uint32_t* __restrict__ slots,
                                                     float* __restrict__ scales, uint64_t seed, int64_t index_base,
                                                     uint8_t* __restrict__ packed, const uint32_t* __restrict__ cnt,
                                                     const uint32_t* __restrict__ lst_b,
                                                     const f32x4* __restrict__ lst_x) {
  static_assert(kFixLists * kCap <= 65536, "table entries fit 16 bits");
  __shared__ uint16_t s_tab[kWaves][kFixLists * kCap];
  const uint32_t wt = (uint32_t)((blockIdx.x * kBlock + threadIdx.x) / kWave);
  if (wt >= S.blk[S.count]) return;
  const int si = seg_of(S, wt);
  const int64_t fw = (int64_t)(wt - S.blk[si]);
  const int64_t lo = S.start[si], hi = S.end[si];
  const int64_t nb = (hi - lo + 3) >> 2;
  const int lane = lane_id();
  uint16_t* tab = s_tab[threadIdx.x / kWave];
  // lists [L0, L0 + ng) of the segment's [tile0 * kWaves, (tile0 + tiles) * kWaves)
  const int64_t L0 = S.tile0[si] * kWaves + fw * kFixLists;
  const int64_t Lend = (S.tile0[si] + seg_tiles(lo, hi)) * kWaves;
  const int ng = (int)(Lend - L0 < kFixLists ? Lend - L0 : kFixLists);
  const uint32_t craw = lane < ng ? cnt[L0 + lane] : 0u;
  const int64_t sl = (int64_t)S.index[si] * kSlots + lane;
  const float sc = bitsf(seg_max_c<6>(max(slots[sl], samp[sl])));
  if (fw == 0 && lane == 0) scales[S.index[si]] = sc;
  uint8_t* __restrict__ out = packed + S.out_byte[si];
  // the table: entry pre_g + i of the wave's entries is slot i of list g.  An overflowed
  // list takes no entries: it is redone below from x (or the residual, which its entries
  // would otherwise have changed first)
  const uint32_t c = craw <= (uint32_t)kCap ? craw : 0u;
  uint32_t total = 0u;
#pragma unroll
  for (int g = 0; g < kFixLists; ++g) {
    const uint32_t cg = (uint32_t)__builtin_amdgcn_readlane((int)c, g);
    for (uint32_t i = (uint32_t)lane; i < cg; i += kWave) tab[total + i] = (uint16_t)(g * kCap + i);
    total += cg;
  }
  // the table is read by other lanes of the same wave
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  for (uint32_t f0 = 0; f0 < total; f0 += kWave) {
    const uint32_t f = f0 + (uint32_t)lane;
    if (f < total) {
      const int64_t e = L0 * kCap + tab[f];   // list L0 + g, slot i
      const int64_t b = lst_b[e];
      const f32x4 q = lst_x[e];
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
  }
  // overflowed lists: every byte of the wave's runs, from x (or from the residual, which
  // holds x + r after the pass)
  uint64_t ovf = ballot(craw > (uint32_t)kCap);
  if (!ovf) return;
  const int d = (int)(lo & 3);
  const int step = d == 0 ? kWave : kWave - 1;
  const float* __restrict__ src = EF ? res : x;
  while (ovf) {
    const int g = __builtin_ctzll(ovf);
    ovf &= ovf - 1;
    const int64_t lr = L0 + g - S.tile0[si] * kWaves;   // the list's wave within the segment
    const int64_t r0 = (lr / kWaves) * kRunsPerBlock + (lr % kWaves) * kRunsB;
    const int64_t b_first = r0 * step;
    int64_t b_last = b_first + (int64_t)kRunsB * step;
    if (b_last > nb) b_last = nb;
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
  // the passes: one launch per batch and start phase d = start % 4 (the pass kernel is
  // compiled for each d)
  for (const SegList& B : batches) {
    for (int d = 0; d < 4; ++d) {
      SegList L{};
      for (int c = 0; c < B.count; ++c) {
        if ((B.start[c] & 3) != d) continue;
        const int k = L.count++;
        L.index[k] = B.index[c];
        L.start[k] = B.start[c];
        L.end[k] = B.end[c];
        L.out_byte[k] = B.out_byte[c];
        L.tile0[k] = B.tile0[c];
        L.blk[k + 1] = L.blk[k] + (uint32_t)seg_tiles(B.start[c], B.end[c]);
      }
      const int64_t blocks = L.blk[L.count];
      if (blocks == 0) continue;
      // a lane's quad starts at a multiple of 4, so its element indices are aligned blocks
      // of the stream exactly when index_base is a multiple of 4
      const bool aligned = (index_base & 3) == 0;
#define GC_TERN_PASS(E, A, D)                                                                                    \
  hipLaunchKernelGGL((k_tern_pass<E, A, D>), (unsigned)blocks, kBlock, 0, s, x, res, n, L,                       \
                     (const uint32_t*)w.samp, w.slots, seed, index_base, packed, w.cnt, w.lst_b, w.lst_x)
#define GC_TERN_PASS_D(E, A) \
  switch (d) { case 0: GC_TERN_PASS(E, A, 0); break; case 1: GC_TERN_PASS(E, A, 1); break; \
               case 2: GC_TERN_PASS(E, A, 2); break; default: GC_TERN_PASS(E, A, 3); break; }
      if (res) { if (aligned) { GC_TERN_PASS_D(true, true) } else { GC_TERN_PASS_D(true, false) } }
      else { if (aligned) { GC_TERN_PASS_D(false, true) } else { GC_TERN_PASS_D(false, false) } }
#undef GC_TERN_PASS_D
#undef GC_TERN_PASS
    }
  }
  for (SegList L : batches) {
    // one wave per kFixLists wave lists of a segment; segments without tiles still get
    // their scale (0) from k_zero2
    L.blk[0] = 0;
    for (int c = 0; c < L.count; ++c)
      L.blk[c + 1] = L.blk[c] + (uint32_t)cdiv64(seg_tiles(L.start[c], L.end[c]) * kWaves, kFixLists);
    const int64_t waves = L.blk[L.count];
    if (waves == 0) continue;
    if (res) hipLaunchKernelGGL((k_tern_fix<true>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, L, (const uint32_t*)w.samp, (const uint32_t*)w.slots, scales, seed, index_base, packed, w.cnt, w.lst_b, w.lst_x);
    else hipLaunchKernelGGL((k_tern_fix<false>), (unsigned)cdiv64(waves, kWaves), kBlock, 0, s, x, res, L, (const uint32_t*)w.samp, (const uint32_t*)w.slots, scales, seed, index_base, packed, w.cnt, w.lst_b, w.lst_x);
  }
  return hipGetLastError();
}

}  // namespace gc
