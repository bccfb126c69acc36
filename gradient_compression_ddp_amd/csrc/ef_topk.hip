// Error-feedback Top-K sparsification (optionally followed by QSGD on the kept values),
// gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", sections 2
// and 2.1 (keep the K largest magnitudes, feed the dropped part back next round);
// 5688vip.com "梯度累积与梯度压缩", section 4.2.1 (int64 indices plus values) and 4.3
// (Top-1% combined with 8-bit quantization); aiqz.cc "梯度聚合通信优化实战方案",
// section "Python 演示" (error_feedback_compress).  Exactly k entries are kept, the lower
// index wins among equal magnitudes, and the indices come out ascending.
//
// Pipeline (all on the caller's stream, no host synchronization):
//  1. sample   key(g+r) at m <= 2^20 jittered positions;
//  2. select   a conservative lower bound L on the k-th largest key from the sample
//              (exact when the sample is the whole input);
//  3. K1       the one full streaming pass: c = g + r written over r, and every element
//              with key >= L appended to per-block pages of a candidate pool (a wave
//              ballot and mbcnt give each candidate its slot; no inter-block waiting);
//  4. scan     per-tile candidate counts -> per-tile offsets in index order;
//              the device then picks the source: the candidates if they surely hold the
//              answer (no pool overflow, count >= k), else the full c (exact fallback);
//  5. reorder  candidates into one array in ascending index order;
//  6. select   the exact k-th largest key T by three radix passes (11, 11, 9 bits) with
//              LDS histograms, and `need`, the number of entries with key == T to keep;
//  7. count + scan + emit: ordered compaction of {key > T} plus the first `need` entries
//              with key == T, writing idx (+index_base) and values; pure Top-K also sets
//              the residual at kept positions to +0.0;
//  8. QSGD     (optional) on the kept values, groups in kept order, RNG index = kept
//              position, and residual[idx] = v - g_hat.
// HBM traffic is 12 B per element in K1 (read g and r, write c) plus O(candidates).
#include "common.hpp"
#include "internal.hpp"
#include "qsgd_core.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;       // 4
constexpr int kRounds = 8;                   // quads per thread per tile
constexpr int64_t kTile = (int64_t)kBlock * 4 * kRounds;   // 8192 elements
constexpr uint32_t kPage = 8192;             // pool page, >= the largest tile count
constexpr int kMaxGrid = 2048;               // K1 blocks (each owns at most one open page)
constexpr int kSampleMax = 1 << 20;
constexpr int kScanChunk = 1024;             // items per block in the multi-block scan
constexpr int kBins = 2048;
constexpr uint32_t kInvalid = 0xFFFFFFFFu;

enum : uint32_t { MODE_CAND = 0, MODE_FULL = 1 };

struct TopkCtrl {
  uint32_t L;              // candidate lower bound on the key
  uint32_t page_next;      // next free pool page
  uint32_t overflow;       // set when a block found no free page
  uint32_t mode;           // MODE_CAND or MODE_FULL
  unsigned long long ncand;   // candidates found by K1
  unsigned long long krem;    // rank still to locate inside the current prefix (1-based)
  uint32_t prefix;         // key bits fixed so far by the radix passes
  uint32_t T;              // the k-th largest key
  unsigned long long need;    // entries with key == T to keep
  unsigned long long nchunks; // compaction chunks of the selected source
  unsigned long long hist[kBins];
};

struct Layout {
  TopkCtrl* ctrl;
  uint32_t* sample;        // [kSampleMax]
  uint32_t* tile_start;    // [ntiles] pool position of the tile's candidates
  uint32_t* tile_count;    // [ntiles]
  unsigned long long* tile_excl;  // [ntiles] exclusive prefix of tile counts
  unsigned long long* scan_up;    // [2 * scan blocks] block sums, then their exclusive scan
  uint32_t* page_fill;     // [cap_pages]
  float* pool_val;         // [cap_pages * kPage]
  uint16_t* pool_off;      // [cap_pages * kPage]
  float* cand_val;         // [cap_pages * kPage] candidates in index order
  int64_t* cand_idx;       // [cap_pages * kPage]
  uint32_t* chunk_gt;      // [max_chunks]
  uint32_t* chunk_eq;      // [max_chunks]
  unsigned long long* chunk_gt_excl;  // [max_chunks]
  unsigned long long* chunk_eq_excl;  // [max_chunks]
  float* staging;          // [k] kept values (QSGD mode without out_val)
  int64_t ntiles, cap_pages, max_chunks, scan_blocks;
  size_t bytes;
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

Layout make_layout(void* base, int64_t n, int64_t k, bool staging) {
  Layout l{};
  l.ntiles = cdiv(n, kTile);
  const int64_t grid = l.ntiles < kMaxGrid ? l.ntiles : kMaxGrid;
  int64_t cap = cdiv(2 * k, (int64_t)kPage) + grid + 1;
  if (cap > l.ntiles) cap = l.ntiles;
  const int64_t pool_max = (int64_t)0xFFFFFFFFu / kPage;   // pool positions fit in uint32
  if (cap > pool_max) cap = pool_max;
  l.cap_pages = cap;
  l.max_chunks = l.ntiles > cap ? l.ntiles : cap;
  const int64_t scan_items = l.max_chunks;
  l.scan_blocks = cdiv(scan_items, kScanChunk);
  size_t off = 0;
  char* b = reinterpret_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  l.ctrl = (TopkCtrl*)take(sizeof(TopkCtrl));
  l.sample = (uint32_t*)take(sizeof(uint32_t) * kSampleMax);
  l.tile_start = (uint32_t*)take(sizeof(uint32_t) * l.ntiles);
  l.tile_count = (uint32_t*)take(sizeof(uint32_t) * l.ntiles);
  l.tile_excl = (unsigned long long*)take(sizeof(unsigned long long) * l.ntiles);
  l.scan_up = (unsigned long long*)take(sizeof(unsigned long long) * 4 * (l.scan_blocks + 1));
  l.page_fill = (uint32_t*)take(sizeof(uint32_t) * cap);
  const int64_t pool = cap * (int64_t)kPage;
  l.pool_val = (float*)take(sizeof(float) * pool);
  l.pool_off = (uint16_t*)take(sizeof(uint16_t) * pool);
  l.cand_val = (float*)take(sizeof(float) * pool);
  l.cand_idx = (int64_t*)take(sizeof(int64_t) * pool);
  l.chunk_gt = (uint32_t*)take(sizeof(uint32_t) * l.max_chunks);
  l.chunk_eq = (uint32_t*)take(sizeof(uint32_t) * l.max_chunks);
  l.chunk_gt_excl = (unsigned long long*)take(sizeof(unsigned long long) * l.max_chunks);
  l.chunk_eq_excl = (unsigned long long*)take(sizeof(unsigned long long) * l.max_chunks);
  l.staging = staging ? (float*)take(sizeof(float) * (k > 0 ? k : 1)) : nullptr;
  l.bytes = off;
  return l;
}

// ---------------------------------------------------------------------------------
// Block-level ordered ranking.  A block handles 8192 entries as 8 rounds x 4 waves x
// 64 lanes x 4 entries; entry (j, w, lane, m) has index j*1024 + w*256 + lane*4 + m.
// For a predicate held as one 4-bit mask per lane and round, rank_round() returns the
// entry's rank among the lane's earlier set bits plus the earlier lanes of the wave, and
// stores the wave's count; block_scan32() then turns the per-(round, wave) counts into
// exclusive offsets in index order.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t rank_round(uint32_t nib, uint32_t* wave_count) {
  const uint64_t b0 = ballot(nib & 1u), b1 = ballot(nib & 2u), b2 = ballot(nib & 4u), b3 = ballot(nib & 8u);
  *wave_count = (uint32_t)(__popcll(b0) + __popcll(b1) + __popcll(b2) + __popcll(b3));
  return mbcnt(b0) + mbcnt(b1) + mbcnt(b2) + mbcnt(b3);
}

// s_cnt / s_off: [kRounds * kWaves] in (round, wave) order.  Called by all threads,
// between barriers.  Returns the block total (valid in every thread after the barrier
// that follows; the value is also stored to *s_total).
__device__ __forceinline__ void block_scan32(const uint32_t* s_cnt, uint32_t* s_off, uint32_t* s_total) {
  if (threadIdx.x < kWave) {
    const int t = threadIdx.x;
    uint32_t v = t < kRounds * kWaves ? s_cnt[t] : 0u;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < 32; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
      if (t >= d) inc += o;
    }
    if (t < kRounds * kWaves) s_off[t] = inc - v;
    if (t == kRounds * kWaves - 1) *s_total = inc;
  }
}

// ---------------------------------------------------------------------------------
// Kernels
// ---------------------------------------------------------------------------------
__global__ void k_init(TopkCtrl* __restrict__ ctrl, unsigned long long krem) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) ctrl->hist[i] = 0ull;
  if (threadIdx.x == 0) {
    ctrl->L = 0u;
    ctrl->page_next = 0u;
    ctrl->overflow = 0u;
    ctrl->mode = MODE_CAND;
    ctrl->ncand = 0ull;
    ctrl->krem = krem;
    ctrl->prefix = 0u;
    ctrl->T = 0u;
    ctrl->need = 0ull;
    ctrl->nchunks = 0ull;
  }
}

// Integer hash for the sample jitter (splitmix64 finalizer); not part of the method's
// arithmetic, only of where the threshold estimate looks.
__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z += 0x9E3779B97F4A7C15ull;
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__global__ void k_sample(const float* __restrict__ g, const float* __restrict__ r, int64_t n, int64_t m,
                         uint32_t* __restrict__ keys) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m;
       i += (int64_t)gridDim.x * blockDim.x) {
    // i < 2^20 and n <= 2^40, so the products stay below 2^61
    const int64_t lo = (int64_t)(((uint64_t)i * (uint64_t)n) / (uint64_t)m);
    const int64_t hi = (int64_t)(((uint64_t)(i + 1) * (uint64_t)n) / (uint64_t)m);
    const int64_t p = lo + (int64_t)(mix64((uint64_t)i) % (uint64_t)(hi - lo));
    keys[i] = mag_key(g[p] + r[p]);
  }
}

// Radix histogram pass over the key bits [shift, shift+bits) of the entries whose higher
// bits equal the prefix fixed so far.  SRC 0: sample keys; SRC 1: candidates or full c.
template <int SRC>
__global__ __launch_bounds__(kBlock) void k_hist(TopkCtrl* __restrict__ ctrl,
                                                 const uint32_t* __restrict__ sample_keys,
                                                 int64_t sample_n, const float* __restrict__ cand,
                                                 const float* __restrict__ full, int64_t n,
                                                 int shift, int bits) {
  __shared__ uint32_t lh[kWaves][kBins];
  for (int i = threadIdx.x; i < kWaves * kBins; i += kBlock) (&lh[0][0])[i] = 0u;
  __syncthreads();
  const uint32_t hshift = (uint32_t)(shift + bits);
  const uint32_t want = ctrl->prefix >> hshift;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t* my = lh[threadIdx.x / kWave];
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  if (SRC == 0) {
    for (int64_t i = (int64_t)blockIdx.x * kBlock + threadIdx.x; i < sample_n; i += stride) {
      const uint32_t key = sample_keys[i];
      if ((key >> hshift) == want) atomicAdd(&my[(key >> shift) & mask], 1u);
    }
  } else {
    const bool use_cand = ctrl->mode == MODE_CAND;
    const float* __restrict__ src = use_cand ? cand : full;
    const int64_t cnt = use_cand ? (int64_t)ctrl->ncand : n;
    const int64_t nq = cnt >> 2;
    for (int64_t q = (int64_t)blockIdx.x * kBlock + threadIdx.x; q < nq; q += stride) {
      const float4 v = *reinterpret_cast<const float4*>(src + (q << 2));
      const float vv[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t key = mag_key(vv[m]);
        if ((key >> hshift) == want) atomicAdd(&my[(key >> shift) & mask], 1u);
      }
    }
    if (blockIdx.x == 0 && threadIdx.x < (cnt & 3)) {
      const uint32_t key = mag_key(src[(nq << 2) + threadIdx.x]);
      if ((key >> hshift) == want) atomicAdd(&my[(key >> shift) & mask], 1u);
    }
  }
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kBlock) {
    const uint32_t c = lh[0][b] + lh[1][b] + lh[2][b] + lh[3][b];
    if (c) atomicAdd(&ctrl->hist[b], (unsigned long long)c);
  }
}

// Locate the bin holding rank `krem` (counted from the largest key) and fix its bits.
// final_op: 0 = intermediate pass; 1 = last pass of the sample select (set L, reset for
// the main select with rank k); 2 = last pass of the main select (set T and need).
__global__ __launch_bounds__(kBlock) void k_pick(TopkCtrl* __restrict__ ctrl, int shift, int final_op,
                                                 unsigned long long k_main) {
  __shared__ unsigned long long s_sum[kBlock];
  constexpr int per = kBins / kBlock;   // 8 bins per thread, highest bins first
  const int t = threadIdx.x;
  const int hi_bin = kBins - 1 - per * t;
  unsigned long long c[per];
  unsigned long long local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    c[i] = ctrl->hist[hi_bin - i];
    local += c[i];
  }
  s_sum[t] = local;
  __syncthreads();
  // exclusive prefix of the chunk sums in thread order (= descending bins)
  for (int d = 1; d < kBlock; d <<= 1) {
    const unsigned long long o = t >= d ? s_sum[t - d] : 0ull;
    __syncthreads();
    s_sum[t] += o;
    __syncthreads();
  }
  unsigned long long before = s_sum[t] - local;
  const unsigned long long krem = ctrl->krem;
  __syncthreads();
#pragma unroll
  for (int i = 0; i < per; ++i) {
    if (before < krem && before + c[i] >= krem) {
      ctrl->prefix |= (uint32_t)(hi_bin - i) << shift;
      ctrl->krem = krem - before;
    }
    before += c[i];
  }
  for (int i = 0; i < per; ++i) ctrl->hist[hi_bin - i] = 0ull;
  __syncthreads();
  if (t == 0 && final_op != 0) {
    const uint32_t T = ctrl->prefix;
    if (final_op == 1) {
      ctrl->L = T;
      ctrl->prefix = 0u;
      ctrl->krem = k_main;
    } else {
      ctrl->T = T;
      ctrl->need = ctrl->krem;
    }
  }
}

// K1: the fused error-feedback add and candidate extraction.  Tiles are assigned
// statically (tile = blockIdx.x + i*gridDim.x); each block appends its candidates to
// its own open page and takes a new page with one atomic when the tile does not fit.
__global__ __launch_bounds__(kBlock) void k_ef_cand(const float* __restrict__ g, float* __restrict__ r,
                                                    int64_t n, int64_t ntiles, TopkCtrl* __restrict__ ctrl,
                                                    uint32_t* __restrict__ tile_start,
                                                    uint32_t* __restrict__ tile_count,
                                                    uint32_t* __restrict__ page_fill,
                                                    float* __restrict__ pool_val,
                                                    uint16_t* __restrict__ pool_off,
                                                    uint32_t cap_pages) {
  __shared__ uint32_t s_cnt[kRounds * kWaves];
  __shared__ uint32_t s_off[kRounds * kWaves];
  __shared__ uint32_t s_total;
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_ok;
  const uint32_t L = ctrl->L;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  uint32_t page = kInvalid, fill = kPage;   // meaningful in thread 0 only
  unsigned long long found = 0ull;          // thread 0 only
  for (int64_t tile = blockIdx.x; tile < ntiles; tile += gridDim.x) {
    const int64_t base = tile * kTile;
    float c[kRounds][4];
    if (base + kTile <= n) {
      f32x4 gv[kRounds], rv[kRounds];
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
        gv[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + e));
        rv[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + e));
      }
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
        f32x4 cv;
        cv.x = gv[j].x + rv[j].x; cv.y = gv[j].y + rv[j].y;
        cv.z = gv[j].z + rv[j].z; cv.w = gv[j].w + rv[j].w;
        __builtin_nontemporal_store(cv, reinterpret_cast<f32x4*>(r + e));
        c[j][0] = cv.x; c[j][1] = cv.y; c[j][2] = cv.z; c[j][3] = cv.w;
      }
    } else {
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
          float v = 0.f;
          if (e < n) {
            v = g[e] + r[e];
            r[e] = v;
          }
          c[j][m] = v;
        }
      }
    }
    uint32_t nib[kRounds], pre[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t b = 0u;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
        b |= ((mag_key(c[j][m]) >= L) && e < n) ? (1u << m) : 0u;
      }
      nib[j] = b;
      uint32_t wc;
      pre[j] = rank_round(b, &wc);
      if (lane == 0) s_cnt[j * kWaves + w] = wc;
    }
    __syncthreads();
    block_scan32(s_cnt, s_off, &s_total);
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t total = s_total;
      uint32_t start = 0u, ok = 1u;
      if (total) {
        if (fill + total > kPage) {
          if (page < cap_pages) page_fill[page] = fill;
          page = atomicAdd(&ctrl->page_next, 1u);
          fill = 0u;
          if (page >= cap_pages) atomicOr(&ctrl->overflow, 1u);
        }
        ok = page < cap_pages ? 1u : 0u;
        start = ok ? page * kPage + fill : 0u;
        fill += total;
      }
      tile_start[tile] = start;
      tile_count[tile] = total;
      found += total;
      s_base = start;
      s_ok = ok;
    }
    __syncthreads();
    if (s_ok) {
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        if (nib[j]) {
          uint32_t pos = s_base + s_off[j * kWaves + w] + pre[j];
#pragma unroll
          for (int m = 0; m < 4; ++m) {
            if (nib[j] & (1u << m)) {
              pool_val[pos] = c[j][m];
              pool_off[pos] = (uint16_t)(j * (kBlock * 4) + threadIdx.x * 4 + m);
              ++pos;
            }
          }
        }
      }
    }
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (page < cap_pages) page_fill[page] = fill;
    atomicAdd(&ctrl->ncand, found);
  }
}

// Plain error-feedback add for k == 0: r = g + r.
__global__ void k_ef_add(const float* __restrict__ g, float* __restrict__ r, int64_t n) {
  const int64_t nq = n >> 2;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t q = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; q < nq; q += stride) {
    const float4 a = *reinterpret_cast<const float4*>(g + 4 * q);
    float4 b = *reinterpret_cast<const float4*>(r + 4 * q);
    b.x = a.x + b.x; b.y = a.y + b.y; b.z = a.z + b.z; b.w = a.w + b.w;
    *reinterpret_cast<float4*>(r + 4 * q) = b;
  }
  if (blockIdx.x == 0 && threadIdx.x < (n & 3)) {
    const int64_t e = 4 * nq + threadIdx.x;
    r[e] = g[e] + r[e];
  }
}

// ---- multi-block exclusive scan of up to two uint32 count arrays ---------------------
// Items are a[i] (and b[i] when b != nullptr); results are 64-bit exclusive prefixes.
// The item count is read from *count_dev when given, else `count`.
__device__ __forceinline__ int64_t scan_count(const unsigned long long* count_dev, int64_t count) {
  return count_dev ? (int64_t)*count_dev : count;
}

__global__ __launch_bounds__(kBlock) void k_scan_up(const uint32_t* __restrict__ a,
                                                    const uint32_t* __restrict__ b,
                                                    const unsigned long long* count_dev, int64_t count,
                                                    unsigned long long* __restrict__ up) {
  __shared__ unsigned long long s[2][kWaves];
  const int64_t cnt = scan_count(count_dev, count);
  const int64_t nb = cdiv(cnt, kScanChunk);
  for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
    unsigned long long sa = 0, sb = 0;
    for (int i = threadIdx.x; i < kScanChunk; i += kBlock) {
      const int64_t it = blk * kScanChunk + i;
      if (it < cnt) {
        sa += a[it];
        if (b) sb += b[it];
      }
    }
    sa = wave_sum_u64(sa);
    sb = wave_sum_u64(sb);
    if (lane_id() == 0) { s[0][threadIdx.x / kWave] = sa; s[1][threadIdx.x / kWave] = sb; }
    __syncthreads();
    if (threadIdx.x == 0) {
      up[2 * blk] = s[0][0] + s[0][1] + s[0][2] + s[0][3];
      up[2 * blk + 1] = s[1][0] + s[1][1] + s[1][2] + s[1][3];
    }
    __syncthreads();
  }
}

// One block: exclusive scan of the block sums in place.
__global__ __launch_bounds__(kBlock) void k_scan_mid(const unsigned long long* count_dev, int64_t count,
                                                     unsigned long long* __restrict__ up) {
  __shared__ unsigned long long s_carry[2];
  const int64_t nb = cdiv(scan_count(count_dev, count), kScanChunk);
  if (threadIdx.x == 0) { s_carry[0] = 0; s_carry[1] = 0; }
  __syncthreads();
  for (int64_t b0 = 0; b0 < nb; b0 += kWave) {
    if (threadIdx.x < kWave) {
      const int64_t i = b0 + threadIdx.x;
      const unsigned long long va = i < nb ? up[2 * i] : 0ull;
      const unsigned long long vb = i < nb ? up[2 * i + 1] : 0ull;
      const unsigned long long ia = wave_incl_scan_u64(va);
      const unsigned long long ib = wave_incl_scan_u64(vb);
      const unsigned long long ca = s_carry[0], cb = s_carry[1];
      if (i < nb) { up[2 * i] = ca + ia - va; up[2 * i + 1] = cb + ib - vb; }
      const unsigned long long ta = __shfl(ia, kWave - 1, kWave);
      const unsigned long long tb = __shfl(ib, kWave - 1, kWave);
      if (threadIdx.x == 0) { s_carry[0] = ca + ta; s_carry[1] = cb + tb; }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(kBlock) void k_scan_down(const uint32_t* __restrict__ a,
                                                      const uint32_t* __restrict__ b,
                                                      const unsigned long long* count_dev, int64_t count,
                                                      const unsigned long long* __restrict__ up,
                                                      unsigned long long* __restrict__ oa,
                                                      unsigned long long* __restrict__ ob) {
  __shared__ unsigned long long s_w[2][kWaves];
  __shared__ unsigned long long s_carry[2];
  const int64_t cnt = scan_count(count_dev, count);
  const int64_t nb = cdiv(cnt, kScanChunk);
  const int w = threadIdx.x / kWave;
  for (int64_t blk = blockIdx.x; blk < nb; blk += gridDim.x) {
    if (threadIdx.x == 0) { s_carry[0] = up[2 * blk]; s_carry[1] = up[2 * blk + 1]; }
    __syncthreads();
    for (int r0 = 0; r0 < kScanChunk; r0 += kBlock) {
      const int64_t it = blk * kScanChunk + r0 + threadIdx.x;
      const unsigned long long va = it < cnt ? a[it] : 0ull;
      const unsigned long long vb = (b && it < cnt) ? b[it] : 0ull;
      const unsigned long long ia = wave_incl_scan_u64(va);
      const unsigned long long ib = wave_incl_scan_u64(vb);
      if (lane_id() == kWave - 1) { s_w[0][w] = ia; s_w[1][w] = ib; }
      __syncthreads();
      unsigned long long pa = s_carry[0], pb = s_carry[1];
      for (int i = 0; i < w; ++i) { pa += s_w[0][i]; pb += s_w[1][i]; }
      if (it < cnt) {
        oa[it] = pa + ia - va;
        if (ob) ob[it] = pb + ib - vb;
      }
      __syncthreads();
      if (threadIdx.x == 0) {
        s_carry[0] += s_w[0][0] + s_w[0][1] + s_w[0][2] + s_w[0][3];
        s_carry[1] += s_w[1][0] + s_w[1][1] + s_w[1][2] + s_w[1][3];
      }
      __syncthreads();
    }
  }
}

// Choose the source of the exact selection.  Candidates hold the answer iff the pool did
// not overflow and at least k entries reached the bound L (then T >= L).
__global__ void k_decide(TopkCtrl* __restrict__ ctrl, unsigned long long k, int64_t n) {
  if (threadIdx.x == 0) {
    const bool full = ctrl->overflow != 0u || ctrl->ncand < k;
    ctrl->mode = full ? MODE_FULL : MODE_CAND;
    const unsigned long long cnt = full ? (unsigned long long)n : ctrl->ncand;
    ctrl->nchunks = (cnt + kTile - 1) / kTile;
  }
}

// Copy each tile's candidates from the pool into one array in index order.  Block b
// handles the tiles it produced in K1 (b, b+G, ...); within a batch of up to 1024 such
// tiles the entries are spread over threads and mapped back to (tile, offset) by binary
// search over the batch's in-block prefix.
__global__ __launch_bounds__(kBlock) void k_reorder(const TopkCtrl* __restrict__ ctrl, int64_t ntiles, int grid1,
                                                    const uint32_t* __restrict__ tile_start,
                                                    const uint32_t* __restrict__ tile_count,
                                                    const unsigned long long* __restrict__ tile_excl,
                                                    const float* __restrict__ pool_val,
                                                    const uint16_t* __restrict__ pool_off,
                                                    float* __restrict__ cand_val,
                                                    int64_t* __restrict__ cand_idx) {
  constexpr int kB = 1024;
  __shared__ uint32_t s_pre[kB + 1];
  __shared__ uint32_t s_start[kB];
  __shared__ unsigned long long s_excl[kB];
  __shared__ uint32_t s_w[kWaves];
  if (ctrl->mode != MODE_CAND) return;
  const int w = threadIdx.x / kWave;
  for (int b = blockIdx.x; b < grid1; b += gridDim.x) {
    const int64_t my_tiles = b < ntiles ? cdiv(ntiles - b, grid1) : 0;
    for (int64_t t0 = 0; t0 < my_tiles; t0 += kB) {
      const int nt = (int)(my_tiles - t0 < kB ? my_tiles - t0 : kB);
      // per-tile data and the in-batch exclusive prefix of the counts
      uint32_t cnt4[4];
      uint32_t local = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int li = threadIdx.x * 4 + i;
        uint32_t cn = 0;
        if (li < nt) {
          const int64_t tile = b + (t0 + li) * (int64_t)grid1;
          cn = tile_count[tile];
          s_start[li] = tile_start[tile];
          s_excl[li] = tile_excl[tile];
        }
        cnt4[i] = cn;
        local += cn;
      }
      uint32_t inc = local;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
        if (lane_id() >= d) inc += o;
      }
      if (lane_id() == kWave - 1) s_w[w] = inc;
      __syncthreads();
      uint32_t p = inc - local;
      for (int i = 0; i < w; ++i) p += s_w[i];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int li = threadIdx.x * 4 + i;
        if (li < nt) s_pre[li] = p;
        p += cnt4[i];
      }
      const uint32_t total = s_w[0] + s_w[1] + s_w[2] + s_w[3];
      if (threadIdx.x == 0) s_pre[nt] = total;
      __syncthreads();
      for (uint32_t j = threadIdx.x; j < total; j += kBlock) {
        // last tile whose prefix is <= j
        int lo = 0, hi = nt;   // invariant: s_pre[lo] <= j < s_pre[hi]
        while (hi - lo > 1) {
          const int mid = (lo + hi) >> 1;
          if (s_pre[mid] <= j) lo = mid; else hi = mid;
        }
        const uint32_t o = j - s_pre[lo];
        const uint32_t src = s_start[lo] + o;
        const unsigned long long dst = s_excl[lo] + o;
        const int64_t tile = b + (t0 + lo) * (int64_t)grid1;
        cand_val[dst] = pool_val[src];
        cand_idx[dst] = tile * kTile + pool_off[src];
      }
      __syncthreads();
    }
  }
}

// Per-chunk counts of key > T and key == T over the selected source.
__global__ __launch_bounds__(kBlock) void k_count(const TopkCtrl* __restrict__ ctrl,
                                                  const float* __restrict__ cand,
                                                  const float* __restrict__ full, int64_t n,
                                                  uint32_t* __restrict__ chunk_gt,
                                                  uint32_t* __restrict__ chunk_eq) {
  __shared__ uint32_t s[2][kWaves];
  const bool use_cand = ctrl->mode == MODE_CAND;
  const float* __restrict__ src = use_cand ? cand : full;
  const int64_t cnt = use_cand ? (int64_t)ctrl->ncand : n;
  const int64_t nch = (int64_t)ctrl->nchunks;
  const uint32_t T = ctrl->T;
  for (int64_t ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const int64_t base = ch * kTile;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
      float v[4];
      if (e + 4 <= cnt) {
        const float4 a = *reinterpret_cast<const float4*>(src + e);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const uint32_t key = mag_key(v[m]);
          gt += key > T;
          eq += key == T;
        }
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (e + m < cnt) {
            const uint32_t key = mag_key(src[e + m]);
            gt += key > T;
            eq += key == T;
          }
      }
    }
    gt = (uint32_t)wave_sum_u64(gt);
    eq = (uint32_t)wave_sum_u64(eq);
    if (lane_id() == 0) { s[0][threadIdx.x / kWave] = gt; s[1][threadIdx.x / kWave] = eq; }
    __syncthreads();
    if (threadIdx.x == 0) {
      chunk_gt[ch] = s[0][0] + s[0][1] + s[0][2] + s[0][3];
      chunk_eq[ch] = s[1][0] + s[1][1] + s[1][2] + s[1][3];
    }
    __syncthreads();
  }
}

// Ordered compaction: keep key > T, and the first `need` entries with key == T.
__global__ __launch_bounds__(kBlock) void k_emit(const TopkCtrl* __restrict__ ctrl,
                                                 const float* __restrict__ cand_val,
                                                 const int64_t* __restrict__ cand_idx,
                                                 float* __restrict__ r, int64_t n,
                                                 const unsigned long long* __restrict__ gt_excl,
                                                 const unsigned long long* __restrict__ eq_excl,
                                                 int64_t index_base, int64_t* __restrict__ out_idx,
                                                 float* __restrict__ out_val, int zero_residual,
                                                 int64_t k) {
  __shared__ uint32_t s_cnt[kRounds * kWaves];
  __shared__ uint32_t s_off[kRounds * kWaves];
  __shared__ uint32_t s_total;
  const bool use_cand = ctrl->mode == MODE_CAND;
  const float* __restrict__ src = use_cand ? cand_val : r;
  const int64_t cnt = use_cand ? (int64_t)ctrl->ncand : n;
  const int64_t nch = (int64_t)ctrl->nchunks;
  const uint32_t T = ctrl->T;
  const unsigned long long need = ctrl->need;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int64_t ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const int64_t base = ch * kTile;
    float v[kRounds][4];
    uint32_t gtn[kRounds], eqn[kRounds], pre[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
      if (e + 4 <= cnt) {
        const float4 a = *reinterpret_cast<const float4*>(src + e);
        v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) v[j][m] = e + m < cnt ? src[e + m] : 0.f;
      }
      uint32_t gb = 0, qb = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const uint32_t key = mag_key(v[j][m]);
        const bool in = e + m < cnt;
        gb |= (in && key > T) ? (1u << m) : 0u;
        qb |= (in && key == T) ? (1u << m) : 0u;
      }
      gtn[j] = gb;
      eqn[j] = qb;
      uint32_t wc;
      pre[j] = rank_round(qb, &wc);
      if (lane == 0) s_cnt[j * kWaves + w] = wc;
    }
    __syncthreads();
    block_scan32(s_cnt, s_off, &s_total);
    __syncthreads();
    // ties: entry is kept iff its global rank among key == T is below need
    const unsigned long long eq0 = eq_excl[ch];
    uint32_t keep[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t kb = gtn[j];
      uint32_t r0 = s_off[j * kWaves + w] + pre[j];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (eqn[j] & (1u << m)) {
          if (eq0 + r0 < need) kb |= 1u << m;
          ++r0;
        }
      keep[j] = kb;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t wc;
      pre[j] = rank_round(keep[j], &wc);
      if (lane == 0) s_cnt[j * kWaves + w] = wc;
    }
    __syncthreads();
    block_scan32(s_cnt, s_off, &s_total);
    __syncthreads();
    const unsigned long long kept0 = gt_excl[ch] + (eq0 < need ? eq0 : need);
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (keep[j]) {
        unsigned long long pos = kept0 + s_off[j * kWaves + w] + pre[j];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (keep[j] & (1u << m)) {
            const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
            const int64_t idx = use_cand ? cand_idx[e] : e;
            if (pos < (unsigned long long)k) {   // exactly k are kept; the guard only bounds stores
              out_idx[pos] = idx + index_base;
              out_val[pos] = v[j][m];
            }
            if (zero_residual) r[idx] = 0.f;
            ++pos;
          }
      }
    }
    __syncthreads();
  }
}

// QSGD over the kept values (groups in kept order, RNG index = kept position) and the
// residual fix-up r[idx] = v - g_hat.
__global__ __launch_bounds__(kBlock) void k_qsgd_kept(const float* __restrict__ vals, int64_t k,
                                                      int lpg_log2, float s, uint64_t seed,
                                                      int8_t* __restrict__ codes, float* __restrict__ norms,
                                                      const int64_t* __restrict__ idx, int64_t index_base,
                                                      float* __restrict__ r, int64_t n) {
  const int64_t nquads = (k + 3) >> 2;
  const int lpg = 1 << lpg_log2;
  const int lane = lane_id();
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t base = (int64_t)blockIdx.x * kBlock; base < nquads; base += stride) {
    const int64_t q = base + threadIdx.x;
    const int64_t e0 = q << 2;
    const bool live = q < nquads;
    const bool full = e0 + 4 <= k;
    float v[4];
    if (live && full) {
      const float4 a = *reinterpret_cast<const float4*>(vals + e0);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) v[m] = (live && e0 + m < k) ? vals[e0 + m] : 0.f;
    }
    float ss = quad_sumsq(v);
    ss = seg_tree_sum(ss, lpg);
    if (!live) continue;
    const float nu = sqrtf(ss);
    float u[4];
    uniforms4(seed, (uint64_t)e0, u);
    int lev[4];
    float gh[4];
    qsgd_quad(v, nu, s, u, lev, gh);
    if (full) {
      *reinterpret_cast<uint32_t*>(codes + e0) = pack_codes4(lev);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (e0 + m < k) codes[e0 + m] = (int8_t)lev[m];
    }
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (e0 + m < k) {
        const int64_t p = idx[e0 + m] - index_base;
        if (p >= 0 && p < n) r[p] = v[m] - gh[m];
      }
    if ((lane & (lpg - 1)) == 0) norms[e0 >> (lpg_log2 + 2)] = nu;
  }
}

int clamp_grid(int64_t want, int64_t cap) {
  if (want < 1) want = 1;
  return (int)(want > cap ? cap : want);
}

}  // namespace

size_t ef_topk_workspace(int64_t n, int64_t k, int qsgd_levels) {
  return make_layout(nullptr, n, k, qsgd_levels > 0).bytes;
}

hipError_t launch_ef_topk(const float* grad, float* res, int64_t n, int64_t k, int64_t index_base,
                          int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group,
                          uint64_t qsgd_seed, int8_t* out_codes, float* out_norms, void* ws,
                          size_t, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const int cus = device_cu_count();
  if (k == 0) {
    hipLaunchKernelGGL(k_ef_add, clamp_grid(cdiv(n, 4 * 256), cus * 16), 256, 0, s, grad, res, n);
    return hipGetLastError();
  }
  prof_mark(s, 0);
  const bool quant = qsgd_levels > 0;
  const Layout l = make_layout(ws, n, k, quant && out_val == nullptr);
  TopkCtrl* ctrl = l.ctrl;

  // 1-2: sample and conservative bound L on the k-th largest key
  const int64_t m = n < kSampleMax ? n : kSampleMax;
  int64_t j;
  if (m == n) {
    j = k;
  } else {
    const double expect = (double)k * (double)m / (double)n;
    j = (int64_t)(1.25 * expect + 8.0 * __builtin_sqrt(expect) + 16.0) + 1;
    if (j > m) j = m;
  }
  hipLaunchKernelGGL(k_init, 1, 256, 0, s, ctrl, (unsigned long long)j);
  hipLaunchKernelGGL(k_sample, clamp_grid(cdiv(m, 256), cus * 8), 256, 0, s, grad, res, n, m, l.sample);
  const int shifts[3] = {20, 9, 0}, widths[3] = {11, 11, 9};
  const int sgrid = clamp_grid(cdiv(m, 256 * 8), cus * 2);
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL((k_hist<0>), sgrid, kBlock, 0, s, ctrl, l.sample, m, (const float*)nullptr,
                       (const float*)nullptr, n, shifts[p], widths[p]);
    hipLaunchKernelGGL(k_pick, 1, kBlock, 0, s, ctrl, shifts[p], p == 2 ? 1 : 0, (unsigned long long)k);
  }

  // 3: the streaming pass
  const int grid1 = (int)(l.ntiles < kMaxGrid ? l.ntiles : kMaxGrid);
  prof_mark(s, 1);
  hipLaunchKernelGGL(k_ef_cand, grid1, kBlock, 0, s, grad, res, n, l.ntiles, ctrl, l.tile_start,
                     l.tile_count, l.page_fill, l.pool_val, l.pool_off, (uint32_t)l.cap_pages);
  prof_mark(s, 2);

  // 4: tile offsets, source decision
  const int scan_grid = clamp_grid(cdiv(l.ntiles, kScanChunk), cus * 4);
  hipLaunchKernelGGL(k_scan_up, scan_grid, kBlock, 0, s, l.tile_count, (const uint32_t*)nullptr,
                     (const unsigned long long*)nullptr, l.ntiles, l.scan_up);
  hipLaunchKernelGGL(k_scan_mid, 1, kBlock, 0, s, (const unsigned long long*)nullptr, l.ntiles, l.scan_up);
  hipLaunchKernelGGL(k_scan_down, scan_grid, kBlock, 0, s, l.tile_count, (const uint32_t*)nullptr,
                     (const unsigned long long*)nullptr, l.ntiles, (const unsigned long long*)l.scan_up,
                     l.tile_excl, (unsigned long long*)nullptr);
  hipLaunchKernelGGL(k_decide, 1, 64, 0, s, ctrl, (unsigned long long)k, n);

  // 5: candidates in index order
  hipLaunchKernelGGL(k_reorder, clamp_grid(grid1, cus * 8), kBlock, 0, s, ctrl, l.ntiles, grid1,
                     l.tile_start, l.tile_count, l.tile_excl, l.pool_val, l.pool_off, l.cand_val,
                     l.cand_idx);

  // 6: exact k-th key over the selected source
  const int hgrid = cus * 4;
  for (int p = 0; p < 3; ++p) {
    hipLaunchKernelGGL((k_hist<1>), hgrid, kBlock, 0, s, ctrl, (const uint32_t*)nullptr, (int64_t)0,
                       l.cand_val, res, n, shifts[p], widths[p]);
    hipLaunchKernelGGL(k_pick, 1, kBlock, 0, s, ctrl, shifts[p], p == 2 ? 2 : 0, (unsigned long long)k);
  }

  // 7: ordered compaction
  const int cgrid = clamp_grid(l.max_chunks, cus * 8);
  hipLaunchKernelGGL(k_count, cgrid, kBlock, 0, s, ctrl, l.cand_val, res, n, l.chunk_gt, l.chunk_eq);
  const unsigned long long* nch_dev = &ctrl->nchunks;
  const int cscan = clamp_grid(cdiv(l.max_chunks, kScanChunk), cus * 4);
  hipLaunchKernelGGL(k_scan_up, cscan, kBlock, 0, s, l.chunk_gt, l.chunk_eq, nch_dev, (int64_t)0, l.scan_up);
  hipLaunchKernelGGL(k_scan_mid, 1, kBlock, 0, s, nch_dev, (int64_t)0, l.scan_up);
  hipLaunchKernelGGL(k_scan_down, cscan, kBlock, 0, s, l.chunk_gt, l.chunk_eq, nch_dev, (int64_t)0,
                     (const unsigned long long*)l.scan_up, l.chunk_gt_excl, l.chunk_eq_excl);
  float* vals = quant ? (out_val ? out_val : l.staging) : out_val;
  hipLaunchKernelGGL(k_emit, cgrid, kBlock, 0, s, ctrl, l.cand_val, l.cand_idx, res, n, l.chunk_gt_excl,
                     l.chunk_eq_excl, index_base, out_idx, vals, quant ? 0 : 1, k);

  // 8: QSGD on the kept values
  if (quant) {
    int lpg_log2 = 0;
    while ((int64_t(4) << lpg_log2) < qsgd_group) ++lpg_log2;
    const int qgrid = clamp_grid(cdiv(cdiv(k, 4), kBlock), cus * 16);
    hipLaunchKernelGGL(k_qsgd_kept, qgrid, kBlock, 0, s, vals, k, lpg_log2, (float)qsgd_levels, qsgd_seed,
                       out_codes, out_norms, out_idx, index_base, res, n);
  }
  prof_mark(s, 3);
  return hipGetLastError();
}

}  // namespace gc
