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
//  1. sample   key(g+r) at m <= 2^19 jittered positions;
//  2. select   a conservative lower bound L on the k-th largest key from the sample.
//              When n <= 2^15 the sample is the whole input and this select is already
//              exact (T and need); the pool then has room for all n elements and steps
//              4-5 and the fallback are skipped, which halves the kernel count of a
//              small call;
//  3. K1       the one full streaming pass, one 4096-element tile per block: c = g + r
//              written over r, and every element with key >= L appended to a candidate
//              pool (a wave ballot and mbcnt give each candidate its slot; the tile claims
//              its pool segment with one atomic on one of 32 interleaved region counters,
//              so no block ever waits for another);
//  4. decide   the candidates are used if they surely hold the answer (no pool overflow,
//              count >= k); otherwise the exact fallback selects over the full c;
//  5. select   the exact k-th largest key T by three radix passes (11, 11, 9 bits) with
//              LDS histograms, and `need`, the number of entries with key == T to keep;
//  6. count    per unit of 16 tiles, the candidates with key > T and key == T, and an
//              exclusive scan of both over the units;
//  7. emit     ordered compaction straight from the pool, by batches of 128 tiles (8
//              units) from a device-side work queue: a batch's candidates are taken
//              in (tile, offset) order, which is index order, and entry e goes to
//              position gt_before(e) + min(eq_before(e), need) when key > T, or when
//              key == T and eq_before(e) < need (so the lower index wins the ties); pure
//              Top-K also sets the residual at kept positions to +0.0.  The fallback
//              runs the same count / scan / emit over tiles of the full c;
//  8. QSGD     (optional) on the kept values, groups in kept order, RNG index = kept
//              position, and the new residual v - g_hat scattered to the kept positions.
// HBM traffic is 12 B per element in K1 (read g and r, write c) plus O(candidates) plus
// the scattered residual update of the kept set (one 64-byte sector per isolated entry).
//
// Error-feedback Random-K (hotdry.top, section 2.2; zyxy.net/archives/25733, section
// 二.2) runs the same pipeline with another key: the Philox word of the element's global
// index under the selection seed, shifted right by one (31 bits, like the magnitude key).
// Its instantiations (RAND = true) draw the sample from the generator, store each
// candidate's key bits in pool_val and its value in pool_c, and compute keys from the
// index in the fallback; the k largest keys, lower index first among equal keys, are a
// uniform choice of k entries without replacement.
#include "common.hpp"
#include "internal.hpp"
#include "qsgd_core.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kWaves = kBlock / kWave;       // 4
constexpr int kRounds = 4;                   // quads per thread per tile
constexpr int64_t kTile = (int64_t)kBlock * 4 * kRounds;   // 4096 elements
constexpr int kRegions = 32;                 // candidate-pool regions (tile % 32)
// At 7e9 elements a draw of 2^20 points (about ten random 64-byte sectors each, with the
// record lookup) took 0.10 ms; 2^19 points took the sample and its select 0.145 -> 0.100 ms
// while the looser bound grew the pool passes and the emit by about 0.015 ms.  2^18 points
// took it to 0.06 ms, but the after-pass grew by 0.04 ms and the streaming pass, writing
// more candidates, by 0.1-0.2 ms (step medians 15.18-15.20 against 15.02-15.13 ms).
constexpr int kSampleMax = 1 << 19;
constexpr int kScanChunk = 1024;             // items per block in the multi-block scan
constexpr int kBins = 2048;
constexpr int kUnit = 16;                    // tiles per unit of the candidate count and scan
constexpr int kBatch = 128;                  // tiles per batch of the emit (8 units)
constexpr int kBatchSmall = kUnit;           // the emit's batch when 128-tile batches are too few
constexpr int kKeptChunk = kBlock * 4;       // kept entries per norm-monitor partial
constexpr int kSumChunk = 4096;              // partials per block of the monitor's second level
constexpr int kFusePickGrid = 256;           // radix pass grids up to this fold the pick in
constexpr int kQueues = 32;                  // sub-queues of the batch emit's work queue
// The emit's look-back words hold counts in 31-bit fields, so it serves k below 2^31.
constexpr unsigned long long kLbField = (1ull << 31) - 1ull;
// The smallest sample: inputs up to this size are sampled whole (the select is exact).
constexpr int kSampleMin = 1 << 15;
static_assert(kBatch % kUnit == 0 && kBatch <= 2 * kWave && kUnit <= kWave, "batch tables");
static_assert(kBatchSmall % kUnit == 0 && kBatchSmall <= kWave, "small batch tables");

enum : uint32_t { MODE_CAND = 0, MODE_FULL = 1 };

struct TopkCtrl {
  uint32_t L;              // candidate lower bound on the key
  uint32_t overflow;       // set when a region of the pool is full
  uint32_t mode;           // MODE_CAND or MODE_FULL
  uint32_t prefix;         // key bits fixed so far by the radix passes
  uint32_t T;              // the k-th largest key
  uint32_t ticket;         // last-block hand-off counter (zero between kernels)
  unsigned long long ncand;   // candidates found by K1
  unsigned long long krem;    // rank still to locate inside the current prefix (1-based)
  unsigned long long need;    // entries with key == T to keep
  unsigned long long nchunks; // tiles of the full fallback source
  unsigned long long hist[kBins];
  // per region: candidates appended (low 32 bits) and, of those, keys whose first radix
  // digit (bits 20..30) is above L's (high 32 bits)
  unsigned long long region_fill[kRegions];
  // per region, when the streaming pass is asked for it, keys whose first digit is at
  // least two above L's: region r's count at [16 r], each on a 64-byte line of its own
  // (atomics on one line serialize whatever their addresses; the region fills above keep
  // 8 to a line, which measured faster at 7e9 than one line each)
  alignas(64) uint32_t region_above2[kRegions * 16];
  uint32_t emit_next;         // work queue of the look-back emits (claims in increasing order)
  uint32_t pass;              // the main select's next digit (0, 1, 2; 3: T found)
  uint32_t emit_sub[kQueues * 16];   // the batch emit's sub-queues, one per 64-byte line
};

struct Layout {
  TopkCtrl* ctrl;
  uint32_t* sample;        // [kSampleMax]
  uint32_t* tile_start;    // [ntiles] pool position of the tile's candidates
  uint32_t* tile_count;    // [ntiles] candidates of the tile
  unsigned long long* scan_up;    // [2 * scan blocks] block sums, then their exclusive scan
  float* pool_val;         // [pool] candidate values, region by region (Random-K: the
                           //   selection key bits, whose magnitude key is the key itself)
  float* pool_c;           // [pool] Random-K only: the candidate values
  uint16_t* pool_off;      // [pool] offset of the candidate inside its tile
  uint32_t* chunk_gt;      // [max_chunks] entries with key > T per batch (candidates) or
                           //   per tile (fallback)
  uint32_t* chunk_eq;      // [max_chunks] entries with key == T
  unsigned long long* gt_excl;    // [max_chunks] exclusive prefixes
  unsigned long long* eq_excl;    // [max_chunks]
  float* staging;          // [k] kept values (QSGD mode without out_val)
  double* mon_c;           // [ntiles] norm monitor: sum of c^2 per tile
  double* mon_g;           // [kchunks] sum of g_hat^2 per 1024 kept entries
  double* mon_c2;          // [cdiv(ntiles, kSumChunk)] second level
  double* mon_g2;          // [cdiv(kchunks, kSumChunk)]
  int64_t ntiles, region_cap, pool, max_chunks, scan_blocks, kchunks;
  size_t bytes;
};

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Sample size and the sample rank whose key is taken as the candidate bound L.
// The rank sits 2% above the expected sample rank plus 8 standard deviations, so the
// candidates hold the k largest unless the sample is off by far more than sampling error.
// Up to 2^15 elements the sample is the whole input, which gives the exact k-th key.
// Above, one element in 64 is drawn, between 2^15 and 2^19 points: the draw costs two
// random sectors per point, and a whole-input select of a million keys costs more than
// the small candidate pool a sample leaves (1e6 elements: 1.7% of them at k = 1%).
int64_t sample_size(int64_t n) {
  if (n <= kSampleMin) return n;
  const int64_t m = n >> 6;
  return m < kSampleMin ? kSampleMin : (m > kSampleMax ? kSampleMax : m);
}
int64_t sample_rank(int64_t n, int64_t k) {
  const int64_t m = sample_size(n);
  if (m == n) return k;
  const double expect = (double)k * (double)m / (double)n;
  int64_t j = (int64_t)(1.02 * expect + 8.0 * __builtin_sqrt(expect) + 64.0) + 1;
  return j > m ? m : j;
}

Layout make_layout(void* base, int64_t n, int64_t k, bool staging, bool rand) {
  Layout l{};
  l.ntiles = cdiv(n, kTile);
  // Room for twice the expected candidates (at least 2k) plus one full tile per region;
  // positions stay in uint32.
  const int64_t m = sample_size(n);
  const double expect_cand = (double)sample_rank(n, k) * (double)n / (double)(m > 0 ? m : 1);
  const int64_t want = expect_cand > (double)k ? (int64_t)expect_cand : k;
  int64_t cap = 2 * want + (int64_t)kRegions * kTile;
  // A whole-input sample gives the exact k-th key, and every element may tie with it:
  // room for all n.  Region r then receives at most ceil(ntiles / 32) tiles of 4096,
  // which is within its share cap / 32.
  if (m == n) cap = n + (int64_t)kRegions * kTile;
  const int64_t cap_max = (int64_t)0xFFFFFFFFu - (int64_t)kRegions * (kTile + 4);
  if (cap > cap_max) cap = cap_max;
  l.region_cap = cdiv(cdiv(cap, kRegions), 4) * 4;   // regions start 16-byte aligned
  l.pool = l.region_cap * kRegions;
  l.max_chunks = l.ntiles;   // >= the batches of kBatch tiles
  l.scan_blocks = cdiv(l.max_chunks, kScanChunk);
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
  l.scan_up = (unsigned long long*)take(sizeof(unsigned long long) * 4 * (l.scan_blocks + 1));
  l.pool_val = (float*)take(sizeof(float) * l.pool);
  l.pool_off = (uint16_t*)take(sizeof(uint16_t) * l.pool);
  l.pool_c = rand ? (float*)take(sizeof(float) * l.pool) : nullptr;
  l.chunk_gt = (uint32_t*)take(sizeof(uint32_t) * l.max_chunks);
  l.chunk_eq = (uint32_t*)take(sizeof(uint32_t) * l.max_chunks);
  l.gt_excl = (unsigned long long*)take(sizeof(unsigned long long) * l.max_chunks);
  l.eq_excl = (unsigned long long*)take(sizeof(unsigned long long) * l.max_chunks);
  l.staging = staging ? (float*)take(sizeof(float) * (k > 0 ? k : 1)) : nullptr;
  l.kchunks = cdiv(k > 0 ? k : 1, kKeptChunk);
  l.mon_c = (double*)take(sizeof(double) * l.ntiles);
  l.mon_g = (double*)take(sizeof(double) * l.kchunks);
  l.mon_c2 = (double*)take(sizeof(double) * cdiv(l.ntiles, kSumChunk));
  l.mon_g2 = (double*)take(sizeof(double) * cdiv(l.kchunks, kSumChunk));
  l.bytes = off;
  return l;
}

// ---------------------------------------------------------------------------------
// Pending kept-set corrections (the deferred residual update).  A deferred call leaves
// c = g + r in the residual everywhere and records, for each kept entry, its offset in
// its 4096-element tile and the residual value it should hold (+0.0 for pure Top-K,
// v - g_hat with QSGD).  The next call's streaming pass applies them to r as it reads
// it, so the kept set's residual is written by a coalesced pass instead of a scatter.
// Record layout (caller-owned, zero-filled before first use = empty):
//   PendHdr | tile_first u64[ntiles] | tile_cnt u32[ntiles] | chunks of 64 entries
// Entry j lives in chunk j / 64: 64 uint32 offsets, then 64 float values, so 64
// consecutive entries fill two whole 256-byte runs.  The layout depends only on n.
// ---------------------------------------------------------------------------------
struct PendHdr {
  unsigned long long n;       // elements of the residual the corrections belong to (0: none)
  unsigned long long count;   // corrections recorded
  uint32_t has_vals;          // values recorded (QSGD); otherwise every correction is +0.0
  uint32_t pad[59];
};
static_assert(sizeof(PendHdr) == 256, "pending header is 256 bytes");

struct Pending {
  PendHdr* hdr;
  unsigned long long* tile_first;   // kept-order index of the tile's first correction
  uint32_t* tile_cnt;               // corrections in the tile
  uint32_t* chunks;                 // entry storage
  int64_t ntiles;
  size_t bytes;
};

Pending pending_layout(void* base, int64_t n, int64_t kmax) {
  Pending p{};
  p.ntiles = cdiv(n, kTile);
  char* b = reinterpret_cast<char*>(base);
  size_t off = 0;
  auto take = [&](size_t bytes) -> void* {
    void* q = b ? b + off : nullptr;
    off += align256(bytes);
    return q;
  };
  p.hdr = (PendHdr*)take(sizeof(PendHdr));
  p.tile_first = (unsigned long long*)take(sizeof(unsigned long long) * p.ntiles);
  p.tile_cnt = (uint32_t*)take(sizeof(uint32_t) * p.ntiles);
  p.chunks = (uint32_t*)take((size_t)cdiv(kmax > 0 ? kmax : 1, 64) * 512);
  p.bytes = off;
  return p;
}

__device__ __forceinline__ uint32_t* pend_off(uint32_t* chunks, unsigned long long j) {
  return chunks + (j >> 6) * 128 + (j & 63);
}
__device__ __forceinline__ float* pend_val(uint32_t* chunks, unsigned long long j) {
  return reinterpret_cast<float*>(chunks + (j >> 6) * 128 + 64 + (j & 63));
}

// The recorded corrections of tile t, clamped to the record's capacity (so that even a
// record that was never zero-filled is read in bounds).
__device__ __forceinline__ void pend_range(const Pending& pd, unsigned long long cap, int64_t t,
                                           unsigned long long* first, uint32_t* cnt) {
  unsigned long long f = pd.tile_first[t];
  unsigned long long c = pd.tile_cnt[t];
  if (f > cap) f = cap;
  if (c > cap - f) c = cap - f;
  *first = f;
  *cnt = (uint32_t)c;
}

// The residual of element p: its recorded correction if it has one, else rv.
__device__ __forceinline__ float pend_lookup(const Pending& pd, unsigned long long cap, int64_t p,
                                             uint32_t has_vals, float rv) {
  unsigned long long f;
  uint32_t cnt;
  pend_range(pd, cap, p / kTile, &f, &cnt);
  const uint32_t o = (uint32_t)(p % kTile);
  uint32_t a = 0, b = cnt;   // first entry with offset >= o (offsets ascend in a tile)
  while (a < b) {
    const uint32_t mid = (a + b) >> 1;
    if (*pend_off(pd.chunks, f + mid) < o) a = mid + 1; else b = mid;
  }
  if (a < cnt && *pend_off(pd.chunks, f + a) == o) return has_vals ? *pend_val(pd.chunks, f + a) : 0.f;
  return rv;
}

// Spreads a tile's corrections into LDS: s_cv[o] = value, bit o of s_cf set.  Called by
// every thread of the block (it holds two barriers).
__device__ __forceinline__ void pend_overlay(const Pending& pd, unsigned long long f, uint32_t cnt,
                                             uint32_t has_vals, float* s_cv, uint32_t* s_cf) {
  for (int i = threadIdx.x; i < kTile / 32; i += kBlock) s_cf[i] = 0u;
  __syncthreads();
  for (uint32_t i = threadIdx.x; i < cnt; i += kBlock) {
    const uint32_t o = *pend_off(pd.chunks, f + i) & (uint32_t)(kTile - 1);
    s_cv[o] = has_vals ? *pend_val(pd.chunks, f + i) : 0.f;
    atomicOr(&s_cf[o >> 5], 1u << (o & 31));
  }
  __syncthreads();
}

// ---------------------------------------------------------------------------------
// Block-level ordered ranking.  A block handles 4096 entries as 4 rounds x 4 waves x
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
    for (int d = 1; d < kRounds * kWaves; d <<= 1) {
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
// Resets the control block for a call (block 0 of the sample kernel runs it).
__device__ __forceinline__ void init_ctrl(TopkCtrl* __restrict__ ctrl, unsigned long long krem,
                                          unsigned long long nchunks) {
  for (int i = threadIdx.x; i < kBins; i += blockDim.x) ctrl->hist[i] = 0ull;
  for (int i = threadIdx.x; i < kRegions; i += blockDim.x) {
    ctrl->region_fill[i] = 0ull;
    ctrl->region_above2[i * 16] = 0u;
  }
  if (threadIdx.x == 0) ctrl->emit_next = 0u;
  for (int i = threadIdx.x; i < kQueues; i += blockDim.x) ctrl->emit_sub[i * 16] = 0u;
  if (threadIdx.x == 0) ctrl->pass = 0u;
  if (threadIdx.x == 0) {
    ctrl->L = 0u;
    ctrl->overflow = 0u;
    ctrl->mode = MODE_CAND;
    ctrl->prefix = 0u;
    ctrl->T = 0u;
    ctrl->ticket = 0u;
    ctrl->ncand = 0ull;
    ctrl->krem = krem;
    ctrl->need = 0ull;
    ctrl->nchunks = nchunks;
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

// Selection key of element e.  Top-K: the magnitude key of c = g + r.  Random-K: the
// Philox word of the global index index_base + e under the selection seed, shifted right
// by one (a 31-bit key, like the magnitude key, so the radix passes are shared).
__device__ __forceinline__ uint32_t rand_key(uint32_t word) { return word >> 1; }

// DEFER: r is corrected by the recorded corrections of the previous call first.
// Block 0 also resets the control block (no kernel before this one reads it).
template <bool RAND, bool DEFER>
__global__ void k_sample(const float* __restrict__ g, const float* __restrict__ r, int64_t n, int64_t m,
                         uint32_t* __restrict__ keys, uint64_t seed, int64_t index_base, Pending pd,
                         unsigned long long cap, TopkCtrl* __restrict__ ctrl, unsigned long long krem,
                         unsigned long long nchunks) {
  if (blockIdx.x == 0) init_ctrl(ctrl, krem, nchunks);
  bool apply = false;
  uint32_t has_vals = 0u;
  if (DEFER && !RAND) {
    apply = pd.hdr->n == (unsigned long long)n;
    has_vals = pd.hdr->has_vals;
  }
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < m;
       i += (int64_t)gridDim.x * blockDim.x) {
    // i < 2^20 and n <= 2^40, so the products stay below 2^61, and hi - lo <= 2^20
    const int64_t lo = (int64_t)(((uint64_t)i * (uint64_t)n) / (uint64_t)m);
    const int64_t hi = (int64_t)(((uint64_t)(i + 1) * (uint64_t)n) / (uint64_t)m);
    const uint64_t h = mix64((uint64_t)i) >> 32;
    const int64_t p = lo + (int64_t)((h * (uint64_t)(hi - lo)) >> 32);
    if (RAND) {
      keys[i] = rand_key(philox_word(seed, (uint64_t)(index_base + p)));
    } else {
      float rv = r[p];
      if (DEFER && apply) rv = pend_lookup(pd, cap, p, has_vals, rv);
      keys[i] = mag_key(g[p] + rv);
    }
  }
}


// Histogram counts go to LDS per run: a thread keeps the bin it last added to and a
// count, and adds to LDS only when the bin changes.  The keys of the candidate pool
// crowd into a few bins, so this removes most of the same-address LDS atomics.
struct BinRun {
  uint32_t bin, cnt;
};

__device__ __forceinline__ void run_flush(uint32_t* my, BinRun& r) {
  if (r.cnt) atomicAdd(&my[r.bin], r.cnt);
  r.cnt = 0u;
}

__device__ __forceinline__ void hist_add(uint32_t* my, BinRun& r, uint32_t key, uint32_t hshift, uint32_t want,
                                         int shift, uint32_t mask) {
  if ((key >> hshift) == want) {
    const uint32_t b = (key >> shift) & mask;
    if (b != r.bin) {
      run_flush(my, r);
      r.bin = b;
    }
    ++r.cnt;
  }
}

// Histogram of nq quads plus a scalar tail of `count` floats starting at src (16-byte
// aligned); four quads per thread are loaded before any is counted.
__device__ __forceinline__ void hist_span(const float* __restrict__ src, int64_t count, int64_t first,
                                          int64_t stride, bool tail_owner, uint32_t* my, BinRun& r,
                                          uint32_t hshift, uint32_t want, int shift, uint32_t mask) {
  constexpr int kAhead = 4;
  const int64_t nq = count >> 2;
  for (int64_t q = first; q < nq; q += kAhead * stride) {
    f32x4 v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int64_t qq = q + u * stride;
      v[u] = qq < nq ? *reinterpret_cast<const f32x4*>(src + (qq << 2)) : f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      if (q + u * stride >= nq) break;
      hist_add(my, r, mag_key(v[u].x), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].y), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].z), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].w), hshift, want, shift, mask);
    }
  }
  if (tail_owner && threadIdx.x < (count & 3))
    hist_add(my, r, mag_key(src[(nq << 2) + threadIdx.x]), hshift, want, shift, mask);
}

// Histogram of the candidate pool with its 32 regions taken as one sequence of quads:
// s_rq[r] is the number of whole quads in regions below r, so every thread issues all of
// its loads at once however the candidates are spread over the regions.  The 0-3
// trailing candidates of region r are counted by block r % gridDim.x.
__device__ __forceinline__ void hist_pool(const float* __restrict__ pool, int64_t region_cap,
                                          const unsigned long long* __restrict__ region_fill, const uint32_t* s_rq,
                                          int64_t first, int64_t stride, uint32_t* my, BinRun& r,
                                          uint32_t hshift, uint32_t want, int shift, uint32_t mask) {
  constexpr int kAhead = 4;
  const int64_t total = s_rq[kRegions];
  for (int64_t q = first; q < total; q += kAhead * stride) {
    f32x4 v[kAhead];
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      const int64_t qq = q + u * stride;
      if (qq < total) {
        int rg = 0;   // the region holding quad qq: the largest rg with s_rq[rg] <= qq
#pragma unroll
        for (int st = kRegions / 2; st > 0; st >>= 1)
          if ((int64_t)s_rq[rg + st] <= qq) rg += st;
        v[u] = *reinterpret_cast<const f32x4*>(pool + rg * region_cap + ((qq - s_rq[rg]) << 2));
      } else {
        v[u] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
#pragma unroll
    for (int u = 0; u < kAhead; ++u) {
      if (q + u * stride >= total) break;
      hist_add(my, r, mag_key(v[u].x), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].y), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].z), hshift, want, shift, mask);
      hist_add(my, r, mag_key(v[u].w), hshift, want, shift, mask);
    }
  }
  for (int rg = blockIdx.x; rg < kRegions; rg += gridDim.x) {
    const uint32_t fill = (uint32_t)region_fill[rg];
    if (threadIdx.x < (fill & 3u))
      hist_add(my, r, mag_key(pool[rg * region_cap + (fill & ~3u) + threadIdx.x]), hshift, want, shift, mask);
  }
}

// Random-K keys of the n elements, quad by quad (the fallback's full source).
__device__ __forceinline__ void hist_rand(int64_t n, uint64_t seed, int64_t index_base, int64_t first,
                                          int64_t stride, bool tail_owner, uint32_t* my, BinRun& r,
                                          uint32_t hshift, uint32_t want, int shift, uint32_t mask) {
  const int64_t nq = n >> 2;
  for (int64_t q = first; q < nq; q += stride) {
    uint32_t w[4];
    words4(seed, (uint64_t)(index_base + (q << 2)), w);
#pragma unroll
    for (int m = 0; m < 4; ++m) hist_add(my, r, rand_key(w[m]), hshift, want, shift, mask);
  }
  if (tail_owner && threadIdx.x < (n & 3))
    hist_add(my, r, rand_key(philox_word(seed, (uint64_t)(index_base + (nq << 2) + threadIdx.x))), hshift,
             want, shift, mask);
}

// Choose the source of the exact selection (one thread).  Candidates hold the answer iff
// the pool did not overflow and at least k entries reached the bound L (then T >= L).
// Without overflow the region counters sum to the number of candidates.  `publish`
// stores the decision in the control block for the kernels that follow.
//
// First digit from the counters: every candidate's key is >= L, so when fewer than k of
// them have a first digit (bits 20..30) above L's, the k-th key's first digit is L's,
// and its rank among the candidates of that digit is k minus that count.  With the
// second count (count2: keys whose first digit is at least two above L's), when at least
// k keys have a digit above L's but fewer than k one two above, the k-th key's first
// digit is L's plus one, at rank k minus the second count.  Either way the select then
// starts at the second digit (*skip = true, *prefix = the first digit in place; publish
// also records the prefix, the remaining rank and the next digit for the passes and picks
// that follow).
// ncand, above and above2 are the sums of the region counters.
__device__ __forceinline__ uint32_t decide_mode(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                                unsigned long long k, bool publish, int count2,
                                                unsigned long long ncand, unsigned long long above,
                                                unsigned long long above2, bool* skip, uint32_t* prefix) {
  const bool full = ctrl->overflow != 0u || ncand < k;
  const uint32_t dL = ctrl->L >> 20;
  const bool skip1 = !full && above < k;
  const bool skip2 = !full && !skip1 && count2 != 0 && dL + 1u < (uint32_t)kBins && above2 < k;
  *skip = skip1 || skip2;
  *prefix = skip1 ? (dL << 20) : (skip2 ? ((dL + 1u) << 20) : 0u);
  if (publish) {
    ctrl->ncand = full ? 0ull : ncand;
    ctrl->mode = full ? MODE_FULL : MODE_CAND;
    ctrl->nchunks = (unsigned long long)(full ? ntiles : cdiv(ntiles, kUnit));
    if (*skip) {
      ctrl->prefix = *prefix;
      ctrl->krem = k - (skip1 ? above : above2);
      ctrl->pass = 1u;
    }
  }
  return full ? MODE_FULL : MODE_CAND;
}

// The main select's digits: bits 20..30, 9..19 and 0..8 of the 31-bit key.
__host__ __device__ constexpr int main_shift(uint32_t pass) { return pass == 0u ? 20 : (pass == 1u ? 9 : 0); }
__host__ __device__ constexpr int main_bits(uint32_t pass) { return pass == 2u ? 9 : 11; }

// Locate the bin of the global histogram holding rank krem (counted from the largest
// key), fix its bits in the prefix and clear the histogram (one block; s_sum holds
// kBlock 64-bit words).  final_op: 0 = intermediate pass; 1 = last pass of the sample
// select (set L, reset for the main select with rank k_main); 2 = last pass of the main
// select (set T and need); 3 = last pass of a select over the whole input (L = T too).
// dyn: the main select over the pool or the full c, whose digit (and so shift and
// final_op) is the control block's pass, advanced here; nothing to do once it is 3.
__device__ __forceinline__ void pick_body(TopkCtrl* __restrict__ ctrl, int shift, int final_op,
                                          unsigned long long k_main, unsigned long long* s_sum, int dyn) {
  constexpr int per = kBins / kBlock;   // 8 bins per thread, highest bins first
  uint32_t pass = 0u;
  if (dyn) {
    pass = ctrl->pass;
    if (pass >= 3u) return;   // uniform: every thread read the same word
    shift = main_shift(pass);
    final_op = pass == 2u ? 2 : 0;
  }
  const int t = threadIdx.x;
  const int hi_bin = kBins - 1 - per * t;
  unsigned long long c[per];
  unsigned long long local = 0;
#pragma unroll
  for (int i = 0; i < per; ++i) {
    c[i] = ctrl->hist[hi_bin - i];
    local += c[i];
  }
  // exclusive prefix of the chunk sums in thread order (= descending bins): a wave scan,
  // then the sums of the waves before (two barriers, not two per doubling step)
  const unsigned long long inc = wave_incl_scan_u64(local);
  if (lane_id() == kWave - 1) s_sum[t / kWave] = inc;
  __syncthreads();
  unsigned long long before = inc - local;
  for (int v = 0; v < t / kWave; ++v) before += s_sum[v];
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
  if (t == 0 && dyn) ctrl->pass = pass + 1u;
  if (t == 0 && final_op != 0) {
    const uint32_t T = ctrl->prefix;
    if (final_op == 1) {
      ctrl->L = T;
      ctrl->prefix = 0u;
      ctrl->krem = k_main;
    } else {
      if (final_op == 3) ctrl->L = T;
      ctrl->T = T;
      ctrl->need = ctrl->krem;
    }
  }
}

__global__ __launch_bounds__(kBlock) void k_pick(TopkCtrl* __restrict__ ctrl, int shift, int final_op,
                                                 unsigned long long k_main, int dyn) {
  __shared__ unsigned long long s_sum[kBlock];
  pick_body(ctrl, shift, final_op, k_main, s_sum, dyn);
}

// Radix histogram pass over the key bits [shift, shift+bits) of the entries whose higher
// bits equal the prefix fixed so far.  SRC 0: sample keys; SRC 1: the candidate pool
// (region by region) or, in the fallback, the magnitude keys of the full c; SRC 2: the
// pool or, in the fallback, the Random-K keys of all n indices.  decide_k > 0 (the first
// pass over the pool): every block takes the source decision itself, and block 0 also
// publishes it.  fuse_pick: the last block to finish then locates the rank's bin
// (pick_body); otherwise k_pick follows.  dyn (the main select over the pool or the full
// c): the digit is the control block's pass, not the arguments (the first launch may
// start at the second digit, see decide_mode), and a launch past the last digit returns.
template <int SRC>
__global__ __launch_bounds__(kBlock) void k_hist(TopkCtrl* __restrict__ ctrl,
                                                 const uint32_t* __restrict__ sample_keys,
                                                 int64_t sample_n, const float* __restrict__ pool,
                                                 int64_t region_cap, const float* __restrict__ full,
                                                 int64_t n, int shift, int bits, uint64_t seed,
                                                 int64_t index_base, int64_t ntiles, unsigned long long decide_k,
                                                 int final_op, unsigned long long k_main, int fuse_pick, int dyn,
                                                 int count2) {
  __shared__ __align__(16) uint32_t lh[kWaves][kBins];
  __shared__ uint32_t s_rq[kRegions + 1];
  __shared__ uint32_t s_mode, s_pass, s_prefix;
  for (int i = threadIdx.x; i < kWaves * kBins; i += kBlock) (&lh[0][0])[i] = 0u;
  if (threadIdx.x < kWave) {
    // wave 0: the region counters, one lane each, for the prefix of the regions' whole-quad
    // counts and, in the deciding pass, the decision
    const int lane = (int)threadIdx.x;
    uint32_t pass = 0u, prefix = 0u, mode = MODE_CAND;
    if (SRC != 0) {
      unsigned long long f = 0ull;
      uint32_t a2 = 0u;
      if (lane < kRegions) {
        f = ctrl->region_fill[lane];
        a2 = ctrl->region_above2[lane * 16];
      }
      // exclusive prefix of the regions' whole-quad counts (candidate mode only reads it)
      const uint32_t c = (uint32_t)f >> 2;
      uint32_t inc = c;
#pragma unroll
      for (int d = 1; d < kRegions; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
        if (lane >= d) inc += o;
      }
      if (lane < kRegions) s_rq[lane] = inc - c;
      if (lane == kRegions - 1) s_rq[kRegions] = inc;
      if (decide_k) {
        const unsigned long long ncand = wave_sum_u64(f & 0xFFFFFFFFull);
        const unsigned long long above = wave_sum_u64(f >> 32);
        const unsigned long long above2 = wave_sum_u64((unsigned long long)a2);
        if (lane == 0) {
          // every block decides the same from the counters; block 0 publishes it
          bool skip = false;
          uint32_t skip_prefix = 0u;
          mode = decide_mode(ctrl, ntiles, decide_k, blockIdx.x == 0, count2, ncand, above, above2, &skip,
                             &skip_prefix);
          if (dyn) {
            pass = skip ? 1u : 0u;
            prefix = skip_prefix;
          } else {
            prefix = ctrl->prefix;
          }
        }
      } else if (lane == 0) {
        mode = ctrl->mode;
        prefix = ctrl->prefix;
        if (dyn) pass = ctrl->pass;
      }
    } else if (lane == 0) {
      prefix = ctrl->prefix;
    }
    if (lane == 0) {
      s_mode = mode;
      s_pass = pass;
      s_prefix = prefix;
    }
  }
  __syncthreads();
  if (dyn) {
    if (s_pass >= 3u) return;   // the select ended in an earlier launch (same for every block)
    shift = main_shift(s_pass);
    bits = main_bits(s_pass);
    final_op = s_pass == 2u ? 2 : 0;
  }
  const uint32_t hshift = (uint32_t)(shift + bits);
  const uint32_t want = s_prefix >> hshift;
  const uint32_t mask = (1u << bits) - 1u;
  uint32_t* my = lh[threadIdx.x / kWave];
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  const int64_t first = (int64_t)blockIdx.x * kBlock + threadIdx.x;
  BinRun run{0u, 0u};
  if (SRC == 0) {
    for (int64_t i = first; i < sample_n; i += stride) hist_add(my, run, sample_keys[i], hshift, want, shift, mask);
  } else if (s_mode == MODE_CAND) {
    hist_pool(pool, region_cap, ctrl->region_fill, s_rq, first, stride, my, run, hshift, want, shift, mask);
  } else if (SRC == 1) {
    hist_span(full, n, first, stride, blockIdx.x == 0, my, run, hshift, want, shift, mask);
  } else {
    hist_rand(n, seed, index_base, first, stride, blockIdx.x == 0, my, run, hshift, want, shift, mask);
  }
  run_flush(my, run);
  __syncthreads();
  for (int b = threadIdx.x; b < kBins; b += kBlock) {
    const uint32_t c = lh[0][b] + lh[1][b] + lh[2][b] + lh[3][b];
    if (c) atomicAdd(&ctrl->hist[b], (unsigned long long)c);
  }
  // lh is free once every thread is past the flush (last_block's barrier)
  if (fuse_pick && last_block(&ctrl->ticket))
    pick_body(ctrl, shift, final_op, k_main, reinterpret_cast<unsigned long long*>(&lh[0][0]), dyn);
}


// K1: the fused error-feedback add and candidate extraction, one tile per block.  The
// non-persistent grid with 16-byte non-temporal loads and stores is the fastest
// streaming shape measured on MI355X.  A tile with candidates claims its pool segment
// with one atomic on the counter of region (tile % 32): few enough regions that a run of
// consecutive tiles keeps its segments close together, enough to keep each counter cold.
// RAND: the key is the Random-K key of the index (its Philox block does not depend on
// the loads, so it is computed under their latency); the pool then holds the key bits
// in pool_val and the value in pool_c.
// DEFER: the previous call's recorded corrections of this tile are spread into LDS
// while the loads are in flight and replace r at their positions before the add.
// MON: the tile's sum of c^2 in float64 (exact squares, fixed order) goes to mon_c.
template <bool RAND, bool DEFER, bool MON, bool ALIGNED, bool COUNT2>
__global__ __launch_bounds__(kBlock) void k_ef_cand(const float* __restrict__ g, float* __restrict__ r,
                                                    int64_t n, TopkCtrl* __restrict__ ctrl,
                                                    uint32_t* __restrict__ tile_start,
                                                    uint32_t* __restrict__ tile_count,
                                                    float* __restrict__ pool_val,
                                                    uint16_t* __restrict__ pool_off,
                                                    uint32_t region_cap, float* __restrict__ pool_c,
                                                    uint64_t seed, int64_t index_base, Pending pd,
                                                    unsigned long long cap, double* __restrict__ mon_c,
                                                    unsigned long long* __restrict__ lb_status) {
  __shared__ uint32_t s_cnt[kRounds * kWaves];
  __shared__ uint32_t s_a2[kWaves];
  __shared__ double s_mon[MON ? kWaves : 1];
  __shared__ uint32_t s_off[kRounds * kWaves];
  __shared__ uint32_t s_total;
  __shared__ uint32_t s_base;
  __shared__ uint32_t s_ok;
  __shared__ float s_cv[DEFER ? kTile : 1];
  __shared__ uint32_t s_cf[DEFER ? kTile / 32 : 1];
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t tile = blockIdx.x;
  const int64_t base = tile * kTile;
  const uint32_t L = ctrl->L;
  if (threadIdx.x == 0) lb_status[tile] = 0ull;   // the emit's look-back word of this tile
  unsigned long long pf = 0;
  uint32_t pc = 0u, has_vals = 0u;
  if (DEFER && pd.hdr->n == (unsigned long long)n) {
    pend_range(pd, cap, tile, &pf, &pc);
    has_vals = pd.hdr->has_vals;
  }
  float c[kRounds][4];
  if (base + kTile <= n) {
    f32x4 gv[kRounds], rv[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
      gv[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(g + e));
      rv[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(r + e));
    }
    if (DEFER && pc) {
      pend_overlay(pd, pf, pc, has_vals, s_cv, s_cf);
#pragma unroll
      for (int j = 0; j < kRounds; ++j) {
        const int q = j * (kBlock * 4) + threadIdx.x * 4;
        const uint32_t bits = (s_cf[q >> 5] >> (q & 31)) & 0xFu;
        if (bits) {
          if (bits & 1u) rv[j].x = s_cv[q];
          if (bits & 2u) rv[j].y = s_cv[q + 1];
          if (bits & 4u) rv[j].z = s_cv[q + 2];
          if (bits & 8u) rv[j].w = s_cv[q + 3];
        }
      }
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
    if (DEFER && pc) pend_overlay(pd, pf, pc, has_vals, s_cv, s_cf);
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
        float v = 0.f;
        if (e < n) {
          float rr = r[e];
          if (DEFER && pc) {
            const int q = j * (kBlock * 4) + threadIdx.x * 4 + m;
            if ((s_cf[q >> 5] >> (q & 31)) & 1u) rr = s_cv[q];
          }
          v = g[e] + rr;
          r[e] = v;
        }
        c[j][m] = v;
      }
    }
  }
  if (MON) {
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j)
#pragma unroll
      for (int m = 0; m < 4; ++m) ss += (double)c[j][m] * (double)c[j][m];
    ss = wave_sum_f64(ss);
    if (lane == 0) s_mon[w] = ss;
  }
  uint32_t key[kRounds][4];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    if (RAND) {
      words4_t<ALIGNED>(seed, (uint64_t)(index_base + base + j * (kBlock * 4) + threadIdx.x * 4), key[j]);
#pragma unroll
      for (int m = 0; m < 4; ++m) key[j][m] = rand_key(key[j][m]);
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) key[j][m] = mag_key(c[j][m]);
    }
  }
  // candidates (key >= L) and, in the high 16 bits of each wave's count, those whose first
  // radix digit is above L's (key >= A; counts stay below 2^13 per tile, so the packed
  // scan never carries); COUNT2: also those whose first digit is two or more above L's
  // (key >= A2, with L's digit below 2047 at most 2049 << 20), summed per wave
  const uint32_t A = ((L >> 20) + 1u) << 20;
  const uint32_t A2 = ((L >> 20) + 2u) << 20;
  uint32_t wa2 = 0u;
  uint32_t nib[kRounds], pre[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    uint32_t b = 0u, wa = 0u;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
      const bool in = e < n;
      b |= ((key[j][m] >= L) && in) ? (1u << m) : 0u;
      wa += (uint32_t)__popcll(ballot((key[j][m] >= A) && in));
      if (COUNT2) wa2 += (uint32_t)__popcll(ballot((key[j][m] >= A2) && in));
    }
    nib[j] = b;
    uint32_t wc;
    pre[j] = rank_round(b, &wc);
    if (lane == 0) s_cnt[j * kWaves + w] = wc | (wa << 16);
  }
  if (COUNT2 && lane == 0) s_a2[w] = wa2;
  __syncthreads();
  block_scan32(s_cnt, s_off, &s_total);
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t total = s_total & 0xFFFFu, above = s_total >> 16;
    uint32_t start = 0u, ok = 1u;
    if (total) {
      const uint32_t region = (uint32_t)(tile & (kRegions - 1));
      const uint32_t at = (uint32_t)atomicAdd(&ctrl->region_fill[region],
                                              ((unsigned long long)above << 32) | (unsigned long long)total);
      if (COUNT2) {
        const uint32_t above2 = (s_a2[0] + s_a2[1]) + (s_a2[2] + s_a2[3]);
        if (above2) atomicAdd(&ctrl->region_above2[region * 16], above2);
      }
      if (at + total > region_cap) {
        atomicOr(&ctrl->overflow, 1u);
        ok = 0u;
      } else {
        start = region * region_cap + at;
      }
    }
    tile_start[tile] = start;
    tile_count[tile] = total;
    s_base = start;
    s_ok = ok;
    if (MON) mon_c[tile] = ((s_mon[0] + s_mon[1]) + s_mon[2]) + s_mon[3];
  }
  __syncthreads();
  if (s_ok) {
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (nib[j]) {
        uint32_t pos = s_base + (s_off[j * kWaves + w] & 0xFFFFu) + pre[j];
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          if (nib[j] & (1u << m)) {
            if (RAND) {
              pool_val[pos] = bitsf(key[j][m]);
              pool_c[pos] = c[j][m];
            } else {
              pool_val[pos] = c[j][m];
            }
            pool_off[pos] = (uint16_t)(j * (kBlock * 4) + threadIdx.x * 4 + m);
            ++pos;
          }
        }
      }
    }
  }
}


// Plain error-feedback add for k == 0: r = g + r, in the same tile shape as K1.
__global__ __launch_bounds__(kBlock) void k_ef_add(const float* __restrict__ g, float* __restrict__ r,
                                                   int64_t n) {
  const int64_t base = (int64_t)blockIdx.x * kTile;
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
    }
  } else {
    for (int64_t e = base + threadIdx.x; e < n; e += kBlock) r[e] = g[e] + r[e];
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


// One-block exclusive scan of one or two uint32 count arrays (small counts only; b and
// ob may be null; the count is *count_dev when given).  A thread takes four consecutive
// items per round of 1024.  Runs as the extra job of one block of the kernel that
// follows the one writing the counts.
struct SmallScan {
  const uint32_t* a;
  const uint32_t* b;
  const unsigned long long* count_dev;
  int64_t count_host;
  unsigned long long* oa;
  unsigned long long* ob;
};

__device__ __forceinline__ void scan_small_body(const SmallScan& sc) {
  constexpr int kPer = 4;
  const uint32_t* __restrict__ a = sc.a;
  const uint32_t* __restrict__ b = sc.b;
  unsigned long long* __restrict__ oa = sc.oa;
  unsigned long long* __restrict__ ob = sc.ob;
  const int64_t count = scan_count(sc.count_dev, sc.count_host);
  __shared__ unsigned long long s_w[2][kWaves];
  unsigned long long ca = 0, cb = 0;
  const int w = threadIdx.x / kWave;
  for (int64_t r0 = 0; r0 < count; r0 += (int64_t)kBlock * kPer) {
    const int64_t i0 = r0 + (int64_t)threadIdx.x * kPer;
    unsigned long long va[kPer], vb[kPer], ta = 0, tb = 0;
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      va[m] = i0 + m < count ? a[i0 + m] : 0ull;
      vb[m] = (b && i0 + m < count) ? b[i0 + m] : 0ull;
      ta += va[m];
      tb += vb[m];
    }
    const unsigned long long ia = wave_incl_scan_u64(ta);
    const unsigned long long ib = wave_incl_scan_u64(tb);
    if (lane_id() == kWave - 1) { s_w[0][w] = ia; s_w[1][w] = ib; }
    __syncthreads();
    unsigned long long pa = ca + ia - ta, pb = cb + ib - tb;
    for (int i = 0; i < w; ++i) { pa += s_w[0][i]; pb += s_w[1][i]; }
#pragma unroll
    for (int m = 0; m < kPer; ++m) {
      if (i0 + m < count) {
        oa[i0 + m] = pa;
        if (ob) ob[i0 + m] = pb;
      }
      pa += va[m];
      pb += vb[m];
    }
    ca += s_w[0][0] + s_w[0][1] + s_w[0][2] + s_w[0][3];
    cb += s_w[1][0] + s_w[1][1] + s_w[1][2] + s_w[1][3];
    __syncthreads();
  }
}


// ---- the candidates of KB consecutive tiles (a unit or a batch) ------------------------
// pre[i] is the exclusive prefix of the tile counts inside the group; past the last tile
// (i >= nt, up to KB) it holds the total.  start[i] is the tile's pool position.  Entry j
// of the group (0 <= j < total) lies in the tile lo with pre[lo] <= j < pre[lo + 1], at
// pool position start[lo] + j - pre[lo]; taken in j order the entries are in index order.
template <int KB>
struct BatchTable {
  uint32_t pre[KB + 1];
  uint32_t start[KB];
  uint32_t wsum[2];
  uint32_t total;
};

// Fills the table for tiles [t0, t0 + nt); every thread calls it (it ends with a
// barrier) and gets the total.  KB <= 64 uses one wave, KB = 128 two.
template <int KB>
__device__ __forceinline__ uint32_t load_batch(BatchTable<KB>& bt, int64_t t0, int nt,
                                               const uint32_t* __restrict__ tile_start,
                                               const uint32_t* __restrict__ tile_count) {
  constexpr int kScanWidth = KB < kWave ? KB : kWave;
  if (threadIdx.x < (KB < kWave ? kWave : KB)) {
    const int li = threadIdx.x;
    uint32_t cn = 0;
    if (li < nt) {
      cn = tile_count[t0 + li];
      bt.start[li] = tile_start[t0 + li];
    }
    uint32_t inc = cn;
#pragma unroll
    for (int d = 1; d < kScanWidth; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
      if (lane_id() >= d) inc += o;
    }
    if (li < KB) bt.pre[li] = inc - cn;   // exclusive within the wave
    if (KB <= kWave) {
      if (li == KB - 1) { bt.pre[KB] = inc; bt.total = inc; }
    } else if (lane_id() == kWave - 1) {
      bt.wsum[li / kWave] = inc;
    }
  }
  __syncthreads();
  if (KB > kWave) {
    // the second wave adds the first wave's sum; padding entries (count 0) then hold the
    // total, and so does pre[KB]
    if (threadIdx.x >= kWave && threadIdx.x < KB) bt.pre[threadIdx.x] += bt.wsum[0];
    if (threadIdx.x == 0) { bt.total = bt.wsum[0] + bt.wsum[1]; bt.pre[KB] = bt.total; }
    __syncthreads();
  }
  return bt.total;
}

// Tile of entry j < total: the largest lo with pre[lo] <= j (that tile is non-empty).
// A fixed-step search (the padding entries equal the total, so they are never taken),
// which the compiler interleaves across a thread's independent entries.
template <int KB>
__device__ __forceinline__ int batch_tile(const BatchTable<KB>& bt, uint32_t j) {
  int lo = 0;
#pragma unroll
  for (int step = KB / 2; step > 0; step >>= 1)
    if (bt.pre[lo + step] <= j) lo += step;
  return lo;
}

// Next batch from the emit's work queue (every thread calls it; uniform result, or -1
// when the queue is empty, which every block reaches).  Dense batches hold ten times the
// average, so a queue keeps blocks from waiting on a fixed share of them.
__device__ __forceinline__ int64_t next_batch(TopkCtrl* ctrl, int64_t nbatch, int64_t* s_b) {
  __syncthreads();   // the previous batch is done with s_b and the batch table
  if (threadIdx.x == 0) *s_b = (int64_t)atomicAdd(&ctrl->emit_next, 1u);
  __syncthreads();
  const int64_t b = *s_b;
  return b < nbatch ? b : -1;
}

// Next batch of the batch emit (unordered claims): block blockIdx.x takes its batches from
// sub-queue q = blockIdx.x % nq (nq = min(kQueues, gridDim.x), so every sub-queue has a
// block), the batches b with b % nq == q in increasing order.  One counter claimed by
// every block serializes at the memory's atomic unit, about 11 ns per claim on one
// address: the 13,700 batches of a 7e9-element call spent 0.15 ms there.
__device__ __forceinline__ int64_t next_batch_split(TopkCtrl* ctrl, int64_t nbatch, int64_t* s_b) {
  __syncthreads();   // the previous batch is done with s_b and the batch table
  const int nq = gridDim.x < (unsigned)kQueues ? (int)gridDim.x : kQueues;
  const int q = (int)(blockIdx.x % (unsigned)nq);
  if (threadIdx.x == 0) *s_b = (int64_t)atomicAdd(&ctrl->emit_sub[q * 16], 1u) * nq + q;
  __syncthreads();
  const int64_t b = *s_b;
  return b < nbatch ? b : -1;
}

// ---- decoupled look-back over the emit's work queue -----------------------------------
// Items (batches of the pool, or tiles of the full c) are claimed in increasing order.
// Each item publishes a status word as soon as it knows its own counts (kLbAgg: key > T,
// key == T), then walks back over its predecessors for their sum and publishes the
// inclusive prefix (kLbIncl).  A predecessor that has not published yet is counted by
// the walking block itself, so no block ever waits for another.  Counts are 31-bit
// fields (gt <= k < 2^31; eq is clamped at need <= k, which leaves
// min(eq_before, need), all the emit uses, unchanged).  The words are relaxed agent-scope
// atomics: the word alone carries the data, so no fence is needed.  The stream pass
// zeroes one word per tile before the emit runs.
constexpr unsigned long long kLbAgg = 1ull << 62, kLbIncl = 2ull << 62;
constexpr int kLbPolls = 512;   // reads of an unpublished word before the walker counts it

__device__ __forceinline__ unsigned long long lb_pack(unsigned long long flag, unsigned long long gt,
                                                      unsigned long long eq) {
  return flag | (gt << 31) | eq;
}
__device__ __forceinline__ void lb_publish(unsigned long long* st, unsigned long long v) {
  __hip_atomic_store(st, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long lb_read(const unsigned long long* st) {
  return __hip_atomic_load(st, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

struct LbShared {
  unsigned long long gt, eq;   // running sums of the walk
  long long next;              // -1: done; otherwise the next item to look at
  long long count_item;        // >= 0: an unpublished item the block counts itself
  unsigned long long wg[kWaves], we[kWaves];   // per wave: sums of its lanes before its stop
  int wstop[kWaves];           // per wave: its first stopping lane (kWave: none)
  uint32_t wincl[kWaves];      // per wave: 1 if that lane holds an inclusive prefix
};

// Exclusive prefix of item i over items 0..i-1: every thread calls it and gets
// (*gx, *ex) with ex clamped at need.  Each step reads the kBlock nearest predecessors
// not yet summed (one per thread) and stops at the nearest inclusive word, or at the
// nearest unpublished item: that one is polled up to kLbPolls times and, if still
// unpublished, counted by count(p, &gt, &eq) block-wide (it may use barriers).  Every
// step sums at least one item, ends the walk, or leaves the next step an item that is
// published or counted, so the walk ends within 2i steps.
template <typename CountFn>
__device__ __forceinline__ void lookback(const unsigned long long* __restrict__ st, int64_t i,
                                         unsigned long long need, LbShared* sh, CountFn count,
                                         unsigned long long* gx, unsigned long long* ex) {
  if (threadIdx.x == 0) { sh->gt = 0ull; sh->eq = 0ull; sh->next = i - 1; sh->count_item = -1; }
  __syncthreads();
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  for (;;) {
    const long long p = sh->next;
    __syncthreads();    // every thread has p before sh is rewritten
    if (p < 0) break;   // uniform: the walk reached item 0's inclusive prefix (or item -1)
    // thread t reads item p - t: wave w covers p - 64w - lane
    const long long q = p - (long long)threadIdx.x;
    const unsigned long long v = q >= 0 ? lb_read(st + q) : kLbIncl;   // before item 0: 0, 0
    const uint32_t flag = (uint32_t)(v >> 62);
    const uint64_t incl = ballot(flag == 2u), none = ballot(flag == 0u);
    const uint64_t stop = incl | none;
    const int f = stop ? __ffsll((unsigned long long)stop) - 1 : kWave;
    // lanes below the wave's stop hold aggregates; an inclusive stop adds its own word
    const bool add = lane < f || (lane == f && ((incl >> lane) & 1ull));
    unsigned long long ag = add ? ((v >> 31) & kLbField) : 0ull;
    unsigned long long ae = add ? (v & kLbField) : 0ull;
    ag = wave_sum_u64(ag);
    ae = wave_sum_u64(ae);
    if (lane == 0) {
      sh->wg[w] = ag;
      sh->we[w] = ae;
      sh->wstop[w] = f;
      sh->wincl[w] = (f < kWave && ((incl >> f) & 1ull)) ? 1u : 0u;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      // waves in order: whole waves of aggregates, then the first wave with a stop
      long long nxt = p - kBlock;                 // no stop in kBlock items: keep walking
      for (int x = 0; x < kWaves; ++x) {
        sh->gt += sh->wg[x];
        sh->eq += sh->we[x];
        if (sh->wstop[x] < kWave) {
          if (sh->wincl[x]) {
            nxt = -1;                             // an inclusive prefix ends the walk
          } else {
            // unpublished: its block has claimed it and publishes its counts without
            // waiting on anything, so poll its word a bounded number of times; if it is
            // still unpublished after that, count it here
            const long long q = p - (kWave * x + sh->wstop[x]);
            bool seen = false;
            for (int it = 0; it < kLbPolls && !seen; ++it) seen = (lb_read(st + q) >> 62) != 0ull;
            if (seen) {
              nxt = q;                            // read it again as the next step's first item
            } else {
              sh->count_item = q;
              nxt = q - 1;
            }
          }
          break;
        }
      }
      sh->next = nxt;
    }
    __syncthreads();
    const long long c = sh->count_item;
    if (c >= 0) {
      unsigned long long cg = 0ull, ce = 0ull;
      count((int64_t)c, &cg, &ce);
      __syncthreads();
      if (threadIdx.x == 0) {
        // The item's owner may have published meanwhile, and may since have changed what
        // it counts (the full-c emit zeroes the residual at kept positions).  An owner
        // publishes its counts, and that store completes, before it writes anything else,
        // so: published now -> take the published word; still unpublished -> nothing was
        // written before this count read it, and the count stands.
        const unsigned long long v = lb_read(st + c);
        const uint32_t flag = (uint32_t)(v >> 62);
        if (flag == 0u) {
          sh->gt += cg;
          sh->eq += ce;
        } else {
          sh->gt += (v >> 31) & kLbField;
          sh->eq += v & kLbField;
          if (flag == 2u) sh->next = -1;   // an inclusive prefix covers everything below
        }
        sh->count_item = -1;
      }
      __syncthreads();
    }
  }
  *gx = sh->gt;
  *ex = sh->eq < need ? sh->eq : need;
  __syncthreads();   // sh is free again once every thread has read it
}

constexpr int kEmitU = 8;   // entries per thread per chunk of the batch emit
constexpr int kCountU = 4;  // entries per thread per chunk of the unit count

// Candidates only: per-unit counts of key > T and key == T, one unit of kUnit tiles per
// wave.  The wave loads its tiles' starts and counts in one step, then the first 64
// candidates of every tile at once (a Top-1% tile holds about 41), and goes on tile by tile
// only for tiles with more.  No LDS and no barrier: each unit costs two dependent loads
// (a block walking units one after another with a block-wide table and sum measured
// 186 us at 7e9 elements).  Every thread returns normally (k_bcount's last-block scan
// needs all of them).
__device__ __forceinline__ void bcount_body(const TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                            const uint32_t* __restrict__ tile_start,
                                            const uint32_t* __restrict__ tile_count,
                                            const float* __restrict__ pool_val,
                                            uint32_t* __restrict__ unit_gt,
                                            uint32_t* __restrict__ unit_eq) {
  if (ctrl->mode != MODE_CAND) return;
  const uint32_t T = ctrl->T;
  const int64_t nunit = cdiv(ntiles, kUnit);
  const int64_t b = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  if (b >= nunit) return;
  const int lane = lane_id();
  const int64_t t0 = b * kUnit;
  const int nt = (int)(ntiles - t0 < kUnit ? ntiles - t0 : kUnit);
  const uint32_t my_start = lane < nt ? tile_start[t0 + lane] : 0u;
  const uint32_t my_cnt = lane < nt ? tile_count[t0 + lane] : 0u;
  float v[kUnit];
#pragma unroll
  for (int i = 0; i < kUnit; ++i) {
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)my_cnt, i);
    const uint32_t s0 = (uint32_t)__builtin_amdgcn_readlane((int)my_start, i);
    v[i] = (uint32_t)lane < c ? pool_val[s0 + lane] : 0.f;
  }
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int i = 0; i < kUnit; ++i) {
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)my_cnt, i);
    if ((uint32_t)lane < c) {
      const uint32_t key = mag_key(v[i]);
      gt += key > T;
      eq += key == T;
    }
  }
  // tiles with more than 64 candidates
  for (int i = 0; i < nt; ++i) {
    const uint32_t c = (uint32_t)__builtin_amdgcn_readlane((int)my_cnt, i);
    if (c <= (uint32_t)kWave) continue;   // uniform
    const uint32_t s0 = (uint32_t)__builtin_amdgcn_readlane((int)my_start, i);
    for (uint32_t j = kWave + lane; j < c; j += kWave) {
      const uint32_t key = mag_key(pool_val[s0 + j]);
      gt += key > T;
      eq += key == T;
    }
  }
  gt = (uint32_t)wave_sum_u64(gt);
  eq = (uint32_t)wave_sum_u64(eq);
  if (lane == 0) { unit_gt[b] = gt; unit_eq[b] = eq; }
}

// Exclusive scan of kN <= 64 packed counts by the first wave (call between barriers).
template <int kN>
__device__ __forceinline__ void small_scan(const uint32_t* s_cnt, uint32_t* s_off, uint32_t* s_total) {
  static_assert(kN <= kWave, "one wave scans the counts");
  if (threadIdx.x < kWave) {
    const int t = threadIdx.x;
    const uint32_t v = t < kN ? s_cnt[t] : 0u;
    uint32_t inc = v;
#pragma unroll
    for (int d = 1; d < kN; d <<= 1) {
      const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
      if (t >= d) inc += o;
    }
    if (t < kN) s_off[t] = inc - v;
    if (t == kN - 1) *s_total = inc;
  }
}

// Candidates only: ordered compaction straight from the pool.  A chunk of a batch is
// kBlock * kEmitU entries; entry j = j0 + u * kBlock + threadIdx.x, so (u, wave) order
// is j order.  One packed scan counts both predicates: the low 16 bits count key > T and
// the high 16 bits key == T (a chunk holds 2048 entries, so neither field carries).
// RAND: the pool holds key bits, and the kept value is read from pool_c.
// DEFER: instead of writing the kept residual, record each kept entry's tile offset at
// its kept position, and write every tile's kept count and the kept position of its
// first entry (the batch's first position plus the prefix of its tiles' counts).
// KB: tiles per batch (kBatch, or kBatchSmall when there are fewer batches than CUs).
template <bool RAND, bool DEFER, int KB>
__device__ __forceinline__ void bemit_body(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                                  const uint32_t* __restrict__ tile_start,
                                                  const uint32_t* __restrict__ tile_count,
                                                  const float* __restrict__ pool_val,
                                                  const uint16_t* __restrict__ pool_off,
                                                  const unsigned long long* __restrict__ gt_excl,
                                                  const unsigned long long* __restrict__ eq_excl,
                                                  float* __restrict__ r, int64_t index_base,
                                                  int64_t* __restrict__ out_idx, float* __restrict__ out_val,
                                                  int zero_residual, int64_t k,
                                                  const float* __restrict__ pool_c, Pending pd) {
  __shared__ BatchTable<KB> bt;
  __shared__ uint32_t s_cnt[kEmitU * kWaves];
  __shared__ uint32_t s_off[kEmitU * kWaves];
  __shared__ uint32_t s_total;
  __shared__ int64_t s_b;
  __shared__ uint32_t s_kc[DEFER ? KB : 1];
  __shared__ uint32_t s_kw[2];
  if (ctrl->mode != MODE_CAND) return;
  const uint32_t T = ctrl->T;
  const unsigned long long need = ctrl->need;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t nbatch = cdiv(ntiles, KB);
  for (int64_t b; (b = next_batch_split(ctrl, nbatch, &s_b)) >= 0;) {
    const int64_t t0 = b * KB;
    const int nt = (int)(ntiles - t0 < KB ? ntiles - t0 : KB);
    if (DEFER && threadIdx.x < KB) s_kc[threadIdx.x] = 0u;   // visible after load_batch's barrier
    const uint32_t total = load_batch(bt, t0, nt, tile_start, tile_count);
    // the exclusive prefixes of the batch's first unit
    unsigned long long gt_run = gt_excl[b * (KB / kUnit)], eq_run = eq_excl[b * (KB / kUnit)];
    // kept entries before the batch: its first kept position
    const unsigned long long pos0 = gt_run + (eq_run < need ? eq_run : need);
    for (uint32_t j0 = 0; j0 < total; j0 += kBlock * kEmitU) {
      uint32_t src[kEmitU];
      int64_t tbase[kEmitU];
      int tlo[kEmitU];
      bool live[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        const uint32_t j = j0 + u * kBlock + threadIdx.x;
        live[u] = j < total;
        const int lo = live[u] ? batch_tile<KB>(bt, j) : 0;
        src[u] = bt.start[lo] + (j - bt.pre[lo]);
        tbase[u] = (t0 + lo) * kTile;
        tlo[u] = lo;
      }
      float v[kEmitU];
      uint32_t off[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        v[u] = live[u] ? pool_val[src[u]] : 0.f;
        off[u] = live[u] ? (uint32_t)pool_off[src[u]] : 0u;
      }
      uint32_t flag[kEmitU], gpre[kEmitU], epre[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        const uint32_t key = mag_key(v[u]);
        const bool gtf = live[u] && key > T;
        const bool eqf = live[u] && key == T;
        const uint64_t bg = ballot(gtf), be = ballot(eqf);
        gpre[u] = mbcnt(bg);
        epre[u] = mbcnt(be);
        flag[u] = (gtf ? 1u : 0u) | (eqf ? 2u : 0u);
        if (lane == 0) s_cnt[u * kWaves + w] = ((uint32_t)__popcll(be) << 16) | (uint32_t)__popcll(bg);
      }
      __syncthreads();
      small_scan<kEmitU * kWaves>(s_cnt, s_off, &s_total);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        bool kept = false;
        if (flag[u]) {
          const uint32_t o = s_off[u * kWaves + w];
          const unsigned long long gb = gt_run + (o & 0xFFFFu) + gpre[u];
          const unsigned long long eb = eq_run + (o >> 16) + epre[u];
          if ((flag[u] & 1u) || eb < need) {
            const unsigned long long pos = gb + (eb < need ? eb : need);
            const int64_t e = tbase[u] + off[u];
            if (pos < (unsigned long long)k) {   // exactly k are kept; the guard only bounds stores
              kept = true;
              out_idx[pos] = e + index_base;
              out_val[pos] = RAND ? pool_c[src[u]] : v[u];
              if (DEFER) *pend_off(pd.chunks, pos) = off[u];
            }
            if (!DEFER && zero_residual) r[e] = 0.f;
          }
        }
        if (DEFER) {
          // per-tile kept counts: the wave's entries are in index order, so each tile's
          // lanes form one run; the run's first lane adds the run's kept count (one LDS
          // atomic per tile and wave, not one per entry on a shared address)
          const uint64_t km = ballot(kept);
          const int prev = __shfl_up(tlo[u], 1, kWave);
          const uint64_t heads = ballot(lane == 0 || prev != tlo[u]);
          if (km != 0ull && ((heads >> lane) & 1ull)) {
            const uint64_t above = heads & ~((2ull << lane) - 1ull);   // heads of later runs (lane 63: none)
            const uint64_t upto = above ? (above & (0ull - above)) - 1ull : ~0ull;   // lanes below the next head
            const uint32_t c = (uint32_t)__popcll(km & upto & ~((1ull << lane) - 1ull));
            if (c) atomicAdd(&s_kc[tlo[u]], c);
          }
        }
      }
      const uint32_t tot = s_total;
      gt_run += tot & 0xFFFFu;
      eq_run += tot >> 16;
      __syncthreads();   // s_cnt / s_off / s_total are rewritten by the next chunk
    }
    if (DEFER) {
      // the batch's tiles: kept counts, and the kept position of each tile's first entry
      // (pos0 plus the exclusive prefix of the counts); the last chunk's barrier ordered
      // the count atomics before these reads
      const uint32_t c = threadIdx.x < KB ? s_kc[threadIdx.x] : 0u;
      uint32_t inc = c;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
        if (lane >= d) inc += o;
      }
      if (KB > kWave) {
        if (threadIdx.x == kWave - 1) s_kw[0] = inc;
        __syncthreads();
        if (threadIdx.x >= kWave) inc += s_kw[0];
      }
      if (threadIdx.x < nt) {
        pd.tile_cnt[t0 + threadIdx.x] = c;
        pd.tile_first[t0 + threadIdx.x] = pos0 + (inc - c);
      }
    }
  }
}

// Keys of the four entries at e..e+3 of the full source (e % 4 == 0; entries at or past n
// are not read and must be masked by the caller).  v receives the values of c.
template <bool RAND>
__device__ __forceinline__ void full_keys4(const float* __restrict__ full, int64_t n, int64_t e,
                                           uint64_t seed, int64_t index_base, bool need_val,
                                           float v[4], uint32_t key[4]) {
  if (RAND) {
    words4(seed, (uint64_t)(index_base + e), key);
#pragma unroll
    for (int m = 0; m < 4; ++m) key[m] = rand_key(key[m]);
  }
  if (!RAND || need_val) {
    if (e + 4 <= n) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(full + e);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) v[m] = e + m < n ? full[e + m] : 0.f;
    }
  }
  if (!RAND) {
#pragma unroll
    for (int m = 0; m < 4; ++m) key[m] = mag_key(v[m]);
  }
}

// Fallback only: per-tile counts of key > T and key == T over the full c (RAND: over the
// keys of all n indices, which need no load).
template <bool RAND>
__device__ __forceinline__ void count_body(const TopkCtrl* __restrict__ ctrl,
                                                  const float* __restrict__ full, int64_t n,
                                                  uint32_t* __restrict__ chunk_gt,
                                                  uint32_t* __restrict__ chunk_eq, uint64_t seed,
                                                  int64_t index_base) {
  __shared__ uint32_t s[2][kWaves];
  if (ctrl->mode != MODE_FULL) return;
  const int64_t nch = cdiv(n, kTile);
  const uint32_t T = ctrl->T;
  for (int64_t ch = blockIdx.x; ch < nch; ch += gridDim.x) {
    const int64_t base = ch * kTile;
    uint32_t gt = 0, eq = 0;
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
      if (e >= n) continue;
      float v[4];
      uint32_t key[4];
      full_keys4<RAND>(full, n, e, seed, index_base, false, v, key);
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (e + m < n) {
          gt += key[m] > T;
          eq += key[m] == T;
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

// Fallback only: ordered compaction of the full c, tile by tile: keep key > T, and the
// first `need` entries with key == T.  DEFER: record offsets, per-tile counts and first
// positions as the batch emit does.
template <bool RAND, bool DEFER>
__device__ __forceinline__ void emit_body(const TopkCtrl* __restrict__ ctrl,
                                                 float* __restrict__ r, int64_t n,
                                                 const unsigned long long* __restrict__ gt_excl,
                                                 const unsigned long long* __restrict__ eq_excl,
                                                 int64_t index_base, int64_t* __restrict__ out_idx,
                                                 float* __restrict__ out_val, int zero_residual,
                                                 int64_t k, uint64_t seed, Pending pd) {
  __shared__ uint32_t s_cnt[kRounds * kWaves];
  __shared__ uint32_t s_off[kRounds * kWaves];
  __shared__ uint32_t s_total;
  if (ctrl->mode != MODE_FULL) return;
  const int64_t nch = cdiv(n, kTile);
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
      uint32_t key[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < 4; ++m) v[j][m] = 0.f;
      if (e < n) full_keys4<RAND>(r, n, e, seed, index_base, true, v[j], key);
      uint32_t gb = 0, qb = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bool in = e + m < n;
        gb |= (in && key[m] > T) ? (1u << m) : 0u;
        qb |= (in && key[m] == T) ? (1u << m) : 0u;
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
    if (DEFER && threadIdx.x == 0) {
      pd.tile_cnt[ch] = s_total;
      pd.tile_first[ch] = kept0;
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (keep[j]) {
        unsigned long long pos = kept0 + s_off[j * kWaves + w] + pre[j];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (keep[j] & (1u << m)) {
            const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
            if (pos < (unsigned long long)k) {   // exactly k are kept; the guard only bounds stores
              out_idx[pos] = e + index_base;
              out_val[pos] = v[j][m];
              if (DEFER) *pend_off(pd.chunks, pos) = (uint32_t)(j * (kBlock * 4) + threadIdx.x * 4 + m);
            }
            if (!DEFER && zero_residual) r[e] = 0.f;
            ++pos;
          }
      }
    }
    __syncthreads();
  }
}

// ---- the emit with look-back: no separate count and scan -----------------------------
// Counts of key > T and key == T over tile ch of the full source (block-wide; every
// thread gets them).
template <bool RAND>
__device__ __forceinline__ void count_tile(const float* __restrict__ full, int64_t n, int64_t ch, uint32_t T,
                                           uint64_t seed, int64_t index_base, uint32_t (*s_red)[kWaves],
                                           unsigned long long* gt_out, unsigned long long* eq_out) {
  const int64_t base = ch * kTile;
  uint32_t gt = 0, eq = 0;
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
    if (e >= n) continue;
    float v[4];
    uint32_t key[4];
    full_keys4<RAND>(full, n, e, seed, index_base, false, v, key);
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (e + m < n) {
        gt += key[m] > T;
        eq += key[m] == T;
      }
  }
  gt = (uint32_t)wave_sum_u64(gt);
  eq = (uint32_t)wave_sum_u64(eq);
  if (lane_id() == 0) { s_red[0][threadIdx.x / kWave] = gt; s_red[1][threadIdx.x / kWave] = eq; }
  __syncthreads();
  *gt_out = (unsigned long long)s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
  *eq_out = (unsigned long long)s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
  __syncthreads();
}

// Counts of key > T and key == T over the pool entries of the batch whose table is bt
// (block-wide; every thread gets them).
template <int KB>
__device__ __forceinline__ void count_pool_batch(const BatchTable<KB>& bt, uint32_t total,
                                                 const float* __restrict__ pool_val, uint32_t T,
                                                 uint32_t (*s_red)[kWaves], unsigned long long* gt_out,
                                                 unsigned long long* eq_out) {
  uint32_t gt = 0, eq = 0;
  for (uint32_t j0 = 0; j0 < total; j0 += kBlock * kCountU) {
    uint32_t src[kCountU];
    bool live[kCountU];
#pragma unroll
    for (int u = 0; u < kCountU; ++u) {
      const uint32_t j = j0 + u * kBlock + threadIdx.x;
      live[u] = j < total;
      const int lo = live[u] ? batch_tile<KB>(bt, j) : 0;
      src[u] = bt.start[lo] + (j - bt.pre[lo]);
    }
#pragma unroll
    for (int u = 0; u < kCountU; ++u)
      if (live[u]) {
        const uint32_t key = mag_key(pool_val[src[u]]);
        gt += key > T;
        eq += key == T;
      }
  }
  gt = (uint32_t)wave_sum_u64(gt);
  eq = (uint32_t)wave_sum_u64(eq);
  if (lane_id() == 0) { s_red[0][threadIdx.x / kWave] = gt; s_red[1][threadIdx.x / kWave] = eq; }
  __syncthreads();
  *gt_out = (unsigned long long)s_red[0][0] + s_red[0][1] + s_red[0][2] + s_red[0][3];
  *eq_out = (unsigned long long)s_red[1][0] + s_red[1][1] + s_red[1][2] + s_red[1][3];
  __syncthreads();
}

// Ordered compaction of the full c, tile by tile from the work queue, each tile's
// exclusive counts found by look-back (status word per tile): keep key > T, and the
// entries with key == T whose rank among them is below need.  DEFER: record offsets,
// per-tile counts and first positions.
template <bool RAND, bool DEFER>
__device__ __forceinline__ void emit_full_lb(TopkCtrl* __restrict__ ctrl, float* __restrict__ r, int64_t n,
                                             unsigned long long* __restrict__ st, int64_t index_base,
                                             int64_t* __restrict__ out_idx, float* __restrict__ out_val,
                                             int zero_residual, int64_t k, uint64_t seed, Pending pd) {
  __shared__ uint32_t s_cnt[kRounds * kWaves];
  __shared__ uint32_t s_off[kRounds * kWaves];
  __shared__ uint32_t s_total;
  __shared__ uint32_t s_red[2][kWaves];
  __shared__ LbShared s_lb;
  __shared__ int64_t s_b;
  const int64_t nch = cdiv(n, kTile);
  const uint32_t T = ctrl->T;
  const unsigned long long need = ctrl->need;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  for (int64_t ch; (ch = next_batch(ctrl, nch, &s_b)) >= 0;) {
    const int64_t base = ch * kTile;
    float v[kRounds][4];
    uint32_t gtn[kRounds], eqn[kRounds], pre[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4;
      uint32_t key[4] = {0u, 0u, 0u, 0u};
#pragma unroll
      for (int m = 0; m < 4; ++m) v[j][m] = 0.f;
      if (e < n) full_keys4<RAND>(r, n, e, seed, index_base, true, v[j], key);
      uint32_t gb = 0, qb = 0;
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const bool in = e + m < n;
        gb |= (in && key[m] > T) ? (1u << m) : 0u;
        qb |= (in && key[m] == T) ? (1u << m) : 0u;
      }
      gtn[j] = gb;
      eqn[j] = qb;
      uint32_t wq, wg;
      pre[j] = rank_round(qb, &wq);
      (void)rank_round(gb, &wg);
      // packed (key > T) << 16 | (key == T): a tile holds 4096 entries, so neither carries
      if (lane == 0) s_cnt[j * kWaves + w] = (wg << 16) | wq;
    }
    __syncthreads();
    block_scan32(s_cnt, s_off, &s_total);
    __syncthreads();
    const unsigned long long gt_t = s_total >> 16, eq_t = s_total & 0xFFFFu;
    if (threadIdx.x == 0) lb_publish(st + ch, lb_pack(kLbAgg, gt_t, eq_t < need ? eq_t : need));
    unsigned long long gx, ex;
    lookback(st, ch, need, &s_lb,
             [&](int64_t p, unsigned long long* cg, unsigned long long* ce) {
               count_tile<RAND>(r, n, p, T, seed, index_base, s_red, cg, ce);
             },
             &gx, &ex);
    if (threadIdx.x == 0) {
      const unsigned long long ei = ex + eq_t;
      lb_publish(st + ch, lb_pack(kLbIncl, gx + gt_t, ei < need ? ei : need));
      // both status stores complete before the block writes anything (the barrier below
      // holds every other thread): a block that counts this tile itself then finds the
      // status published whenever it could have read a zeroed residual
      asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    }
    // ties: an entry with key == T is kept iff its rank among them is below need
    uint32_t keep[kRounds];
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t kb = gtn[j];
      unsigned long long r0 = ex + (s_off[j * kWaves + w] & 0xFFFFu) + pre[j];
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (eqn[j] & (1u << m)) {
          if (r0 < need) kb |= 1u << m;
          ++r0;
        }
      keep[j] = kb;
    }
    __syncthreads();   // s_cnt / s_off are rewritten below
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      uint32_t wc;
      pre[j] = rank_round(keep[j], &wc);
      if (lane == 0) s_cnt[j * kWaves + w] = wc;
    }
    __syncthreads();
    block_scan32(s_cnt, s_off, &s_total);
    __syncthreads();
    const unsigned long long kept0 = gx + ex;
    if (DEFER && threadIdx.x == 0) {
      pd.tile_cnt[ch] = s_total;
      pd.tile_first[ch] = kept0;
    }
#pragma unroll
    for (int j = 0; j < kRounds; ++j) {
      if (keep[j]) {
        unsigned long long pos = kept0 + s_off[j * kWaves + w] + pre[j];
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (keep[j] & (1u << m)) {
            const int64_t e = base + j * (kBlock * 4) + threadIdx.x * 4 + m;
            if (pos < (unsigned long long)k) {   // exactly k are kept; the guard only bounds stores
              out_idx[pos] = e + index_base;
              out_val[pos] = v[j][m];
              if (DEFER) *pend_off(pd.chunks, pos) = (uint32_t)(j * (kBlock * 4) + threadIdx.x * 4 + m);
            }
            if (!DEFER && zero_residual) r[e] = 0.f;
            ++pos;
          }
      }
    }
  }
}

// Ordered compaction straight from the pool, batch by batch from the work queue, each
// batch's exclusive counts found by look-back (status word per batch): a first pass
// over the batch's candidates counts them, the emit proper then reads them again (now
// in the cache).  Otherwise as bemit_body.
template <bool RAND, bool DEFER, int KB>
__device__ __forceinline__ void bemit_lb(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                         const uint32_t* __restrict__ tile_start,
                                         const uint32_t* __restrict__ tile_count,
                                         const float* __restrict__ pool_val, const uint16_t* __restrict__ pool_off,
                                         unsigned long long* __restrict__ st, float* __restrict__ r,
                                         int64_t index_base, int64_t* __restrict__ out_idx,
                                         float* __restrict__ out_val, int zero_residual, int64_t k,
                                         const float* __restrict__ pool_c, Pending pd) {
  __shared__ BatchTable<KB> bt;
  __shared__ BatchTable<KB> bt2;   // a predecessor counted during the look-back
  __shared__ uint32_t s_cnt[kEmitU * kWaves];
  __shared__ uint32_t s_off[kEmitU * kWaves];
  __shared__ uint32_t s_total;
  __shared__ uint32_t s_red[2][kWaves];
  __shared__ LbShared s_lb;
  __shared__ int64_t s_b;
  __shared__ uint32_t s_kc[DEFER ? KB : 1];
  __shared__ uint32_t s_kw[2];
  const uint32_t T = ctrl->T;
  const unsigned long long need = ctrl->need;
  const int w = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t nbatch = cdiv(ntiles, KB);
  for (int64_t b; (b = next_batch(ctrl, nbatch, &s_b)) >= 0;) {
    const int64_t t0 = b * KB;
    const int nt = (int)(ntiles - t0 < KB ? ntiles - t0 : KB);
    if (DEFER && threadIdx.x < KB) s_kc[threadIdx.x] = 0u;   // visible after load_batch's barrier
    const uint32_t total = load_batch(bt, t0, nt, tile_start, tile_count);
    unsigned long long gt_b, eq_b;
    count_pool_batch<KB>(bt, total, pool_val, T, s_red, &gt_b, &eq_b);
    if (threadIdx.x == 0) lb_publish(st + b, lb_pack(kLbAgg, gt_b, eq_b < need ? eq_b : need));
    unsigned long long gt_run, eq_run;
    lookback(st, b, need, &s_lb,
             [&](int64_t p, unsigned long long* cg, unsigned long long* ce) {
               const int64_t p0 = p * KB;
               const int pn = (int)(ntiles - p0 < KB ? ntiles - p0 : KB);
               const uint32_t ptot = load_batch(bt2, p0, pn, tile_start, tile_count);
               count_pool_batch<KB>(bt2, ptot, pool_val, T, s_red, cg, ce);
             },
             &gt_run, &eq_run);
    if (threadIdx.x == 0) {
      const unsigned long long ei = eq_run + eq_b;
      lb_publish(st + b, lb_pack(kLbIncl, gt_run + gt_b, ei < need ? ei : need));
    }
    // kept entries before the batch: its first kept position (eq_run is clamped at need)
    const unsigned long long pos0 = gt_run + eq_run;
    for (uint32_t j0 = 0; j0 < total; j0 += kBlock * kEmitU) {
      uint32_t src[kEmitU];
      int64_t tbase[kEmitU];
      int tlo[kEmitU];
      bool live[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        const uint32_t j = j0 + u * kBlock + threadIdx.x;
        live[u] = j < total;
        const int lo = live[u] ? batch_tile<KB>(bt, j) : 0;
        src[u] = bt.start[lo] + (j - bt.pre[lo]);
        tbase[u] = (t0 + lo) * kTile;
        tlo[u] = lo;
      }
      float v[kEmitU];
      uint32_t off[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        v[u] = live[u] ? pool_val[src[u]] : 0.f;
        off[u] = live[u] ? (uint32_t)pool_off[src[u]] : 0u;
      }
      uint32_t flag[kEmitU], gpre[kEmitU], epre[kEmitU];
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        const uint32_t key = mag_key(v[u]);
        const bool gtf = live[u] && key > T;
        const bool eqf = live[u] && key == T;
        const uint64_t bg = ballot(gtf), be = ballot(eqf);
        gpre[u] = mbcnt(bg);
        epre[u] = mbcnt(be);
        flag[u] = (gtf ? 1u : 0u) | (eqf ? 2u : 0u);
        if (lane == 0) s_cnt[u * kWaves + w] = ((uint32_t)__popcll(be) << 16) | (uint32_t)__popcll(bg);
      }
      __syncthreads();
      small_scan<kEmitU * kWaves>(s_cnt, s_off, &s_total);
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kEmitU; ++u) {
        bool kept = false;
        if (flag[u]) {
          const uint32_t o = s_off[u * kWaves + w];
          const unsigned long long gb = gt_run + (o & 0xFFFFu) + gpre[u];
          const unsigned long long eb = eq_run + (o >> 16) + epre[u];
          if ((flag[u] & 1u) || eb < need) {
            const unsigned long long pos = gb + (eb < need ? eb : need);
            const int64_t e = tbase[u] + off[u];
            if (pos < (unsigned long long)k) {   // exactly k are kept; the guard only bounds stores
              kept = true;
              out_idx[pos] = e + index_base;
              out_val[pos] = RAND ? pool_c[src[u]] : v[u];
              if (DEFER) *pend_off(pd.chunks, pos) = off[u];
            }
            if (!DEFER && zero_residual) r[e] = 0.f;
          }
        }
        if (DEFER) {
          const uint64_t km = ballot(kept);
          const int prev = __shfl_up(tlo[u], 1, kWave);
          const uint64_t heads = ballot(lane == 0 || prev != tlo[u]);
          if (km != 0ull && ((heads >> lane) & 1ull)) {
            const uint64_t above = heads & ~((2ull << lane) - 1ull);
            const uint64_t upto = above ? (above & (0ull - above)) - 1ull : ~0ull;
            const uint32_t c = (uint32_t)__popcll(km & upto & ~((1ull << lane) - 1ull));
            if (c) atomicAdd(&s_kc[tlo[u]], c);
          }
        }
      }
      const uint32_t tot = s_total;
      gt_run += tot & 0xFFFFu;
      eq_run += tot >> 16;
      __syncthreads();
    }
    if (DEFER) {
      const uint32_t c = threadIdx.x < KB ? s_kc[threadIdx.x] : 0u;
      uint32_t inc = c;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        const uint32_t o = (uint32_t)__shfl_up((int)inc, d, kWave);
        if (lane >= d) inc += o;
      }
      if (KB > kWave) {
        if (threadIdx.x == kWave - 1) s_kw[0] = inc;
        __syncthreads();
        if (threadIdx.x >= kWave) inc += s_kw[0];
      }
      if (threadIdx.x < nt) {
        pd.tile_cnt[t0 + threadIdx.x] = c;
        pd.tile_first[t0 + threadIdx.x] = pos0 + (inc - c);
      }
    }
  }
}

// The emit with look-back, either source (the mode the selection left in the control
// block).  zero_residual (pure Top-K, residual written directly): the kept positions'
// residual becomes +0.0.  DEFER: block 0 also writes the pending record's header.
template <bool RAND, bool DEFER, int KB>
__global__ __launch_bounds__(kBlock) void k_emit_lb(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                                    const uint32_t* __restrict__ tile_start,
                                                    const uint32_t* __restrict__ tile_count,
                                                    const float* __restrict__ pool_val,
                                                    const uint16_t* __restrict__ pool_off,
                                                    unsigned long long* __restrict__ st, float* __restrict__ r,
                                                    int64_t n, int64_t index_base, int64_t* __restrict__ out_idx,
                                                    float* __restrict__ out_val, int zero_residual, int64_t k,
                                                    const float* __restrict__ pool_c, uint64_t seed, Pending pd,
                                                    uint32_t has_vals) {
  if (DEFER && blockIdx.x == 0 && threadIdx.x == 0) {
    pd.hdr->n = (unsigned long long)n;
    pd.hdr->count = (unsigned long long)k;
    pd.hdr->has_vals = has_vals;
  }
  if (ctrl->mode == MODE_CAND)
    bemit_lb<RAND, DEFER, KB>(ctrl, ntiles, tile_start, tile_count, pool_val, pool_off, st, r, index_base, out_idx,
                              out_val, zero_residual, k, pool_c, pd);
  else
    emit_full_lb<RAND, DEFER>(ctrl, r, n, st, index_base, out_idx, out_val, zero_residual, k, seed, pd);
}

// Counts of the candidates per unit, and of the full source per tile in the fallback:
// two kernels (each returns at once unless the device-side mode is its own).  One
// kernel holding both bodies measured 302 us against 186 us for the candidate count at
// 7e9 elements, with the same code for that body, so they stay apart.
// SCAN (small counts only): the scan of the counts is folded in.  In k_bcount (the
// whole-input select, candidate mode) the last block to finish runs it; in k_count the
// last counting block runs it in the fallback, and block 0 at once in candidate mode,
// whose counts the previous kernel wrote.  Only as template variants: the extra code in
// the candidate count's kernel alone measured 300 us against 186 us at 7e9 elements.
template <bool SCAN>
__global__ __launch_bounds__(kBlock) void k_bcount(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                                   const uint32_t* __restrict__ tile_start,
                                                   const uint32_t* __restrict__ tile_count,
                                                   const float* __restrict__ pool_val,
                                                   uint32_t* __restrict__ chunk_gt, uint32_t* __restrict__ chunk_eq,
                                                   SmallScan sc) {
  bcount_body(ctrl, ntiles, tile_start, tile_count, pool_val, chunk_gt, chunk_eq);
  if (SCAN && last_block(&ctrl->ticket)) scan_small_body(sc);
}

template <bool RAND, bool SCAN>
__global__ __launch_bounds__(kBlock) void k_count(TopkCtrl* __restrict__ ctrl, const float* __restrict__ full,
                                                  int64_t n, uint32_t* __restrict__ chunk_gt,
                                                  uint32_t* __restrict__ chunk_eq, uint64_t seed, int64_t index_base,
                                                  SmallScan sc) {
  if (SCAN && ctrl->mode != MODE_FULL) {
    if (blockIdx.x == 0) scan_small_body(sc);
    return;
  }
  count_body<RAND>(ctrl, full, n, chunk_gt, chunk_eq, seed, index_base);
  if (SCAN && last_block(&ctrl->ticket)) scan_small_body(sc);
}

// Ordered compaction from the selected source in one launch (batch emit of the pool, or
// the fallback's tile emit).  DEFER: block 0 also writes the pending record's header for
// this call (the streaming pass, its only reader in this call, is done).
template <bool RAND, bool DEFER, int KB>
__global__ __launch_bounds__(kBlock) void k_emit_all(TopkCtrl* __restrict__ ctrl, int64_t ntiles,
                                                     const uint32_t* __restrict__ tile_start,
                                                     const uint32_t* __restrict__ tile_count,
                                                     const float* __restrict__ pool_val,
                                                     const uint16_t* __restrict__ pool_off,
                                                     const unsigned long long* __restrict__ gt_excl,
                                                     const unsigned long long* __restrict__ eq_excl,
                                                     float* __restrict__ r, int64_t n, int64_t index_base,
                                                     int64_t* __restrict__ out_idx, float* __restrict__ out_val,
                                                     int zero_residual, int64_t k, const float* __restrict__ pool_c,
                                                     uint64_t seed, Pending pd, uint32_t has_vals) {
  if (DEFER && blockIdx.x == 0 && threadIdx.x == 0) {
    pd.hdr->n = (unsigned long long)n;
    pd.hdr->count = (unsigned long long)k;
    pd.hdr->has_vals = has_vals;
  }
  bemit_body<RAND, DEFER, KB>(ctrl, ntiles, tile_start, tile_count, pool_val, pool_off, gt_excl, eq_excl, r,
                              index_base, out_idx, out_val, zero_residual, k, pool_c, pd);
  emit_body<RAND, DEFER>(ctrl, r, n, gt_excl, eq_excl, index_base, out_idx, out_val, zero_residual, k, seed, pd);
}

// QSGD over the kept values (groups in kept order, RNG index = kept position) and the
// residual update r[idx] = v - g_hat.  A block takes 1024 kept entries as 256 quads; the
// residuals go through LDS so that the scattered stores are issued in kept order, 64
// consecutive entries per wave store (neighbouring kept entries often share a sector).
// DEFER: the residuals go to the record's values, in kept order, instead of r.
// MON: the sum of g_hat^2 of each 1024 kept entries (float64, fixed order) goes to mon_g.
template <bool DEFER, bool MON, int LPG_LOG2>
__global__ __launch_bounds__(kBlock) void k_qsgd_kept(const float* __restrict__ vals, int64_t k,
                                                      float s, float ys, uint64_t seed,
                                                      int8_t* __restrict__ codes, float* __restrict__ norms,
                                                      const int64_t* __restrict__ idx, int64_t index_base,
                                                      float* __restrict__ r, int64_t n, Pending pd,
                                                      double* __restrict__ mon_g) {
  __shared__ float s_res[kBlock * 4];
  __shared__ double s_mon[MON ? kWaves : 1];
  const int64_t nquads = (k + 3) >> 2;
  constexpr int lpg_log2 = LPG_LOG2;
  constexpr int lpg = 1 << LPG_LOG2;
  const int lane = lane_id();
  const int64_t stride = (int64_t)gridDim.x * kBlock;
  for (int64_t base = (int64_t)blockIdx.x * kBlock; base < nquads; base += stride) {
    const int64_t q = base + threadIdx.x;
    const int64_t e0 = q << 2;
    const bool live = q < nquads;
    const bool full = e0 + 4 <= k;
    float v[4];
    if (live && full) {
      const f32x4 a = *reinterpret_cast<const f32x4*>(vals + e0);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) v[m] = (live && e0 + m < k) ? vals[e0 + m] : 0.f;
    }
    float ss = quad_sumsq(v);
    ss = seg_tree_sum_c<LPG_LOG2>(ss);
    __syncthreads();   // s_res is still being read by the previous iteration's scatter
    double gg = 0.0;
    if (live) {
      const float nu = sqrtf(ss);
      float u[4];
      uniforms4_t<true>(seed, (uint64_t)e0, u);   // e0 is a multiple of 4
      int lev[4];
      float gh[4];
      qsgd_quad(v, nu, s, ys, u, lev, gh);
      if (full) {
        *reinterpret_cast<uint32_t*>(codes + e0) = pack_codes4(lev);
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m)
          if (e0 + m < k) codes[e0 + m] = (int8_t)lev[m];
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) s_res[threadIdx.x * 4 + m] = v[m] - gh[m];
      if ((lane & (lpg - 1)) == 0) norms[e0 >> (lpg_log2 + 2)] = nu;
      if (MON) {
#pragma unroll
        for (int m = 0; m < 4; ++m) gg += (double)gh[m] * (double)gh[m];
      }
    }
    if (MON) {
      gg = wave_sum_f64(gg);
      if (lane == 0) s_mon[threadIdx.x / kWave] = gg;
    }
    __syncthreads();
    if (MON && threadIdx.x == 0) mon_g[base / kBlock] = ((s_mon[0] + s_mon[1]) + s_mon[2]) + s_mon[3];
    // entry base*4 + j sits at s_res[j]; entries at or beyond k were never kept
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int64_t j = base * 4 + m * kBlock + threadIdx.x;
      if (j < k) {
        if (DEFER) {
          *pend_val(pd.chunks, (unsigned long long)j) = s_res[m * kBlock + threadIdx.x];
        } else {
          const int64_t p = idx[j] - index_base;
          if (p >= 0 && p < n) r[p] = s_res[m * kBlock + threadIdx.x];
        }
      }
    }
  }
}

// The same for the deferred record without the norm monitor, as a streaming pass: each
// quad's residuals v - g_hat go to the record as one 16-byte store (four consecutive kept
// entries never straddle a 64-entry chunk of the record), so no LDS pass-through and no
// barrier is needed.  One 2048-entry tile per block (two quads per lane, the draws issued
// under the loads, every round computed before the first store, non-temporal loads and
// stores), as the bucket QSGD: 99.9 us at 7e9 against 122 us with plain loads and stores
// (one or four quads per lane: 104-105 us).
template <int LPG_LOG2>
__global__ __launch_bounds__(kBlock) void k_qsgd_kept_rec(const float* __restrict__ vals, int64_t k, float s,
                                                          float ys, uint64_t seed, int8_t* __restrict__ codes,
                                                          float* __restrict__ norms, Pending pd) {
  constexpr int R = 2;
  constexpr int lpg = 1 << LPG_LOG2;
  const int lane = lane_id();
  const int64_t base = (int64_t)blockIdx.x * (kBlock * 4 * R);
  float v[R][4];
  float u[R][4];
  const bool whole = base + kBlock * 4 * R <= k;   // block-uniform
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    if (whole) {
      const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(vals + e0));
      v[j][0] = a.x; v[j][1] = a.y; v[j][2] = a.z; v[j][3] = a.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) v[j][m] = e0 + m < k ? vals[e0 + m] : 0.f;
    }
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    uniforms4_t<true>(seed, (uint64_t)(base + j * (kBlock * 4) + threadIdx.x * 4), u[j]);
#pragma unroll
    for (int m = 0; m < 4; ++m) asm volatile("" : "+v"(u[j][m]));
  }
  uint32_t cw[R];
  float nus[R];
  float rv[R][4];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    nus[j] = sqrtf(seg_tree_sum_c<LPG_LOG2>(quad_sumsq(v[j])));
    int lev[4];
    float gh[4];
    qsgd_quad(v[j], nus[j], s, ys, u[j], lev, gh);
    cw[j] = pack_codes4(lev);
#pragma unroll
    for (int m = 0; m < 4; ++m) rv[j][m] = v[j][m] - gh[m];
  }
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    if (whole || e0 + 4 <= k) {
      __builtin_nontemporal_store(cw[j], reinterpret_cast<uint32_t*>(codes + e0));
      __builtin_nontemporal_store(f32x4{rv[j][0], rv[j][1], rv[j][2], rv[j][3]},
                                  reinterpret_cast<f32x4*>(pend_val(pd.chunks, (unsigned long long)e0)));
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m)
        if (e0 + m < k) {
          codes[e0 + m] = (int8_t)(uint8_t)(cw[j] >> (8 * m));
          *pend_val(pd.chunks, (unsigned long long)(e0 + m)) = rv[j][m];
        }
    }
    if ((lane & (lpg - 1)) == 0 && e0 < k) norms[e0 >> (LPG_LOG2 + 2)] = nus[j];
  }
}

// ---- norm monitor: float64 sums of squares in a fixed order --------------------------
// Sum of v^2 over each kKeptChunk entries of v (the kept values of pure selection).
__global__ __launch_bounds__(kBlock) void k_sq_chunks(const float* __restrict__ v, int64_t len,
                                                      double* __restrict__ part) {
  __shared__ double s[kWaves];
  const int64_t e0 = (int64_t)blockIdx.x * kKeptChunk + threadIdx.x * 4;
  double a = 0.0;
#pragma unroll
  for (int m = 0; m < 4; ++m)
    if (e0 + m < len) a += (double)v[e0 + m] * (double)v[e0 + m];
  a = wave_sum_f64(a);
  if (lane_id() == 0) s[threadIdx.x / kWave] = a;
  __syncthreads();
  if (threadIdx.x == 0) part[blockIdx.x] = ((s[0] + s[1]) + s[2]) + s[3];
}

// Block-level sum of up to kBlock * per consecutive doubles, each thread taking every
// kBlock-th one in order; every thread gets the result.
__device__ __forceinline__ double block_sum_f64(const double* __restrict__ in, int64_t count, double* s) {
  double a = 0.0;
  for (int64_t i = threadIdx.x; i < count; i += kBlock) a += in[i];
  a = wave_sum_f64(a);
  __syncthreads();
  if (lane_id() == 0) s[threadIdx.x / kWave] = a;
  __syncthreads();
  return ((s[0] + s[1]) + s[2]) + s[3];
}

// Second level: out[b] = sum of in[b * kSumChunk, (b + 1) * kSumChunk).
__global__ __launch_bounds__(kBlock) void k_sum_f64(const double* __restrict__ in, int64_t count,
                                                    double* __restrict__ out) {
  __shared__ double s[kWaves];
  const int64_t b0 = (int64_t)blockIdx.x * kSumChunk;
  const int64_t len = count - b0 < kSumChunk ? count - b0 : kSumChunk;
  const double t = block_sum_f64(in + b0, len, s);
  if (threadIdx.x == 0) out[blockIdx.x] = t;
}

// stats = {sum c^2, sum g_hat^2, sqrt(sum g_hat^2 / sum c^2)} (ratio 1 when c is zero).
__global__ __launch_bounds__(kBlock) void k_mon_final(const double* __restrict__ c2, int64_t nc,
                                                      const double* __restrict__ g2, int64_t ng,
                                                      double* __restrict__ stats) {
  __shared__ double s[kWaves];
  const double sc = block_sum_f64(c2, nc, s);
  const double sg = block_sum_f64(g2, ng, s);
  if (threadIdx.x == 0) {
    stats[0] = sc;
    stats[1] = sg;
    stats[2] = sc > 0.0 ? sqrt(sg / sc) : 1.0;
  }
}

// Writes every recorded correction into r, one wave per tile, so that r becomes the
// exact residual; k_pend_set then marks the record empty.
__global__ __launch_bounds__(kBlock) void k_pend_flush(float* __restrict__ r, int64_t n, Pending pd,
                                                       unsigned long long cap) {
  if (pd.hdr->n != (unsigned long long)n) return;
  const int64_t t = (int64_t)blockIdx.x * kWaves + threadIdx.x / kWave;
  if (t >= pd.ntiles) return;
  const uint32_t has_vals = pd.hdr->has_vals;
  unsigned long long f;
  uint32_t cnt;
  pend_range(pd, cap, t, &f, &cnt);
  for (uint32_t i = (uint32_t)lane_id(); i < cnt; i += kWave) {
    const int64_t e = t * kTile + (*pend_off(pd.chunks, f + i) & (uint32_t)(kTile - 1));
    if (e < n) r[e] = has_vals ? *pend_val(pd.chunks, f + i) : 0.f;
  }
}

__global__ void k_pend_set(PendHdr* __restrict__ hdr, unsigned long long n, unsigned long long count,
                           uint32_t has_vals) {
  if (threadIdx.x == 0) {
    hdr->n = n;
    hdr->count = count;
    hdr->has_vals = has_vals;
  }
}

// Entries a record of `bytes` bytes holds for n elements (0 if it is too small for the
// fixed part).
unsigned long long pending_capacity(int64_t n, size_t bytes) {
  const size_t fixed = pending_layout(nullptr, n, 0).bytes - 512;
  return bytes < fixed ? 0ull : (unsigned long long)((bytes - fixed) / 512) * 64ull;
}

int clamp_grid(int64_t want, int64_t cap) {
  if (want < 1) want = 1;
  return (int)(want > cap ? cap : want);
}

void launch_flush(float* res, int64_t n, const Pending& pd, unsigned long long cap, hipStream_t s) {
  hipLaunchKernelGGL(k_pend_flush, (unsigned)cdiv(pd.ntiles, kWaves), kBlock, 0, s, res, n, pd, cap);
  hipLaunchKernelGGL(k_pend_set, 1, 64, 0, s, pd.hdr, 0ull, 0ull, 0u);
}

// The whole pipeline for one key source (Top-K magnitudes, or Random-K index keys), with
// the kept set's residual written directly or recorded for the next call (DEFER).
template <bool RAND, bool DEFER>
hipError_t launch_select(const float* grad, float* res, int64_t n, int64_t k, int64_t index_base,
                         uint64_t select_seed, int64_t* out_idx, float* out_val, int qsgd_levels,
                         int64_t qsgd_group, uint64_t qsgd_seed, int8_t* out_codes, float* out_norms,
                         void* ws, void* pend, size_t pend_bytes, double* stats, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const bool mon = stats != nullptr;
  const int cus = device_cu_count();
  const unsigned long long cap = DEFER ? pending_capacity(n, pend_bytes) : 0ull;
  const Pending pd = DEFER ? pending_layout(pend, n, (int64_t)cap) : Pending{};
  if (k == 0) {
    // nothing is kept: apply what the previous call recorded, then the plain add
    if (DEFER) launch_flush(res, n, pd, cap, s);
    hipLaunchKernelGGL(k_ef_add, (unsigned)cdiv(n, kTile), kBlock, 0, s, grad, res, n);
    return hipGetLastError();
  }
  prof_mark(s, 0);
  const bool quant = qsgd_levels > 0;
  // the workspace is laid out for the largest use (QSGD with staging); out_val given or
  // not, the carve-outs stay where the size query put them
  const Layout l = make_layout(ws, n, k, quant, RAND);
  TopkCtrl* ctrl = l.ctrl;
  unsigned long long* lb_status = l.gt_excl;   // the emit's look-back words, one per tile
  float* vals = quant ? (out_val ? out_val : l.staging) : out_val;
  const int zero_res = (quant || DEFER) ? 0 : 1;
  const uint32_t has_vals = quant ? 1u : 0u;
  double* mon_c = mon ? l.mon_c : nullptr;

  // 1-2: sample and conservative bound L on the k-th largest key
  const int64_t m = sample_size(n);
  const int64_t j = sample_rank(n, k);
  const bool exact = m == n;   // the sample select is the exact select
  const int64_t nunit = cdiv(l.ntiles, kUnit);
  const int64_t nbatch = cdiv(l.ntiles, kBatch);
  hipLaunchKernelGGL((k_sample<RAND, DEFER>), clamp_grid(cdiv(m, 256), cus * 16), 256, 0, s, grad, res, n, m,
                     l.sample, select_seed, index_base, pd, cap, ctrl, (unsigned long long)j,
                     (unsigned long long)nunit);
  const int shifts[3] = {20, 9, 0}, widths[3] = {11, 11, 9};
  // pool histogram grid: each block clears and flushes a 2048-bin LDS histogram, so a
  // block takes at least 16384 of the candidates the pool is expected to hold
  const int sgrid = clamp_grid(cdiv(m, 2048), cus * 2);
  const int64_t expect_cand = (int64_t)((double)j * (double)n / (double)m);
  int hgrid = clamp_grid(cdiv(expect_cand, 16384), cus * 4);
  if (hgrid < 32) hgrid = 32;
  // a bound needs only the sample key's top 22 bits (L = that prefix, its low 9 bits 0:
  // 2^9 ulps below the sample's key); the exact select resolves all 31
  const int spasses = exact ? 3 : 2;
  for (int p = 0; p < spasses; ++p) {
    const int op = p == spasses - 1 ? (exact ? 3 : 1) : 0;
    const bool fuse = sgrid <= kFusePickGrid;
    hipLaunchKernelGGL((k_hist<0>), sgrid, kBlock, 0, s, ctrl, l.sample, m, (const float*)nullptr,
                       (int64_t)0, (const float*)nullptr, n, shifts[p], widths[p], (uint64_t)0, (int64_t)0,
                       (int64_t)0, 0ull, op, (unsigned long long)k, fuse ? 1 : 0, 0, 0);
    if (!fuse) hipLaunchKernelGGL(k_pick, 1, kBlock, 0, s, ctrl, shifts[p], op, (unsigned long long)k, 0);
  }

  // 3: the streaming pass.  On small calls the bound's slack, relative to the sample size,
  // often puts the k-th key one first digit above L's: up to 2^22 elements the pass then
  // also counts the keys two digits above, so that the pool select can still start at the
  // second digit (1e6 elements: 63.9 -> 58.7 us a call).  At 6.5M and 16.8M the second
  // count cost the streaming pass about what the skipped pool pass saved, and at 7e9 the
  // first count settles the digit
  const int count2 = n <= (int64_t(1) << 22) ? 1 : 0;
  prof_mark(s, 1);
  // Random-K keys: a lane's quad draws one Philox block when index_base % 4 == 0
#define GC_CAND_PASS3(M, A, C)                                                                            \
  hipLaunchKernelGGL((k_ef_cand<RAND, DEFER, M, A, C>), (unsigned)l.ntiles, kBlock, 0, s, grad, res, n, ctrl,  \
                     l.tile_start, l.tile_count, l.pool_val, l.pool_off, (uint32_t)l.region_cap, l.pool_c,       \
                     select_seed, index_base, pd, cap, mon_c, lb_status)
#define GC_CAND_PASS(M, A)                                  \
  do {                                                      \
    if (count2) GC_CAND_PASS3(M, A, true);                  \
    else GC_CAND_PASS3(M, A, false);                        \
  } while (0)
  if (!RAND || (index_base & 3) == 0) {
    if (mon) GC_CAND_PASS(true, true); else GC_CAND_PASS(false, true);
  } else {
    if constexpr (RAND) {
      if (mon) GC_CAND_PASS(true, false); else GC_CAND_PASS(false, false);
    }
  }
#undef GC_CAND_PASS
#undef GC_CAND_PASS3
  prof_mark(s, 2);

  // 4-5: unless the sample was the whole input (T and need already exact, and every
  // candidate is kept or a tie), the first pool pass decides the source; then the exact
  // k-th key over it.  The digits come from the control block: when the streaming pass's
  // counts already fix the first digit, the first launch takes the second and the third
  // launch (and its pick) returns at once
  if (!exact) {
    for (int p = 0; p < 3; ++p) {
      const bool fuse = hgrid <= kFusePickGrid;
      hipLaunchKernelGGL((k_hist<RAND ? 2 : 1>), hgrid, kBlock, 0, s, ctrl, (const uint32_t*)nullptr, (int64_t)0,
                         (const float*)l.pool_val, l.region_cap, (const float*)res, n, shifts[p], widths[p],
                         select_seed, index_base, l.ntiles, p == 0 ? (unsigned long long)k : 0ull,
                         p == 2 ? 2 : 0, (unsigned long long)k, fuse ? 1 : 0, 1, count2);
      if (!fuse)
        hipLaunchKernelGGL(k_pick, 1, kBlock, 0, s, ctrl, shifts[p], p == 2 ? 2 : 0, (unsigned long long)k, 1);
    }
  }

  // 6-7: ordered compaction.  Few work items (batches of the pool; tiles in the
  // fallback): each finds its exclusive counts by look-back inside the emit.  Many: a
  // count kernel and a scan first (the look-back's extra pass per item and its walks
  // measured slower than those at 7e9 elements, 13,672 batches).
  const bool small_batches = nbatch < cus;
  const int64_t items = small_batches ? nunit : nbatch;
  const int bgrid = clamp_grid(items, cus * 8);
  if (k <= (int64_t)kLbField && items <= 2 * (int64_t)cus) {
    if (small_batches)
      hipLaunchKernelGGL((k_emit_lb<RAND, DEFER, kBatchSmall>), bgrid, kBlock, 0, s, ctrl, l.ntiles, l.tile_start,
                         l.tile_count, (const float*)l.pool_val, (const uint16_t*)l.pool_off, lb_status, res, n,
                         index_base, out_idx, vals, zero_res, k, (const float*)l.pool_c, select_seed, pd, has_vals);
    else
      hipLaunchKernelGGL((k_emit_lb<RAND, DEFER, kBatch>), bgrid, kBlock, 0, s, ctrl, l.ntiles, l.tile_start,
                         l.tile_count, (const float*)l.pool_val, (const uint16_t*)l.pool_off, lb_status, res, n,
                         index_base, out_idx, vals, zero_res, k, (const float*)l.pool_c, select_seed, pd, has_vals);
  } else {
    const int cgrid = clamp_grid(l.ntiles, cus * 8);
    // counts per unit (candidates) or per tile (fallback), and their scan (folded into the
    // count kernel when the counts are few)
    const unsigned long long* nch_dev = &ctrl->nchunks;
    const bool small_scan = l.max_chunks <= 8 * kScanChunk;
    const SmallScan sc{l.chunk_gt, l.chunk_eq, nch_dev, 0, l.gt_excl, l.eq_excl};
    hipLaunchKernelGGL(k_bcount<false>, (unsigned)cdiv(nunit, kWaves), kBlock, 0, s, ctrl, l.ntiles, l.tile_start,
                       l.tile_count, (const float*)l.pool_val, l.chunk_gt, l.chunk_eq, sc);
    if (small_scan)
      hipLaunchKernelGGL((k_count<RAND, true>), cgrid, kBlock, 0, s, ctrl, (const float*)res, n, l.chunk_gt,
                         l.chunk_eq, select_seed, index_base, sc);
    else
      hipLaunchKernelGGL((k_count<RAND, false>), cgrid, kBlock, 0, s, ctrl, (const float*)res, n, l.chunk_gt,
                         l.chunk_eq, select_seed, index_base, sc);
    if (!small_scan) {
      const int cscan = clamp_grid(cdiv(l.max_chunks, kScanChunk), cus * 4);
      hipLaunchKernelGGL(k_scan_up, cscan, kBlock, 0, s, l.chunk_gt, l.chunk_eq, nch_dev, (int64_t)0, l.scan_up);
      hipLaunchKernelGGL(k_scan_mid, 1, kBlock, 0, s, nch_dev, (int64_t)0, l.scan_up);
      hipLaunchKernelGGL(k_scan_down, cscan, kBlock, 0, s, l.chunk_gt, l.chunk_eq, nch_dev, (int64_t)0,
                         (const unsigned long long*)l.scan_up, l.gt_excl, l.eq_excl);
    }
    if (small_batches)
      hipLaunchKernelGGL((k_emit_all<RAND, DEFER, kBatchSmall>), bgrid, kBlock, 0, s, ctrl, l.ntiles, l.tile_start,
                         l.tile_count, (const float*)l.pool_val, (const uint16_t*)l.pool_off,
                         (const unsigned long long*)l.gt_excl, (const unsigned long long*)l.eq_excl, res, n,
                         index_base, out_idx, vals, zero_res, k, (const float*)l.pool_c, select_seed, pd, has_vals);
    else
      hipLaunchKernelGGL((k_emit_all<RAND, DEFER, kBatch>), bgrid, kBlock, 0, s, ctrl, l.ntiles, l.tile_start,
                         l.tile_count, (const float*)l.pool_val, (const uint16_t*)l.pool_off,
                         (const unsigned long long*)l.gt_excl, (const unsigned long long*)l.eq_excl, res, n,
                         index_base, out_idx, vals, zero_res, k, (const float*)l.pool_c, select_seed, pd, has_vals);
  }

  // 8: QSGD on the kept values and the residual of the kept set (deferred: into the
  // record, whose per-tile counts and first positions the emit wrote)
  if (quant) {
    int lpg_log2 = 0;
    while ((int64_t(4) << lpg_log2) < qsgd_group) ++lpg_log2;
    const int qgrid = clamp_grid(cdiv(cdiv(k, 4), kBlock), cus * 16);
    double* mg = mon ? l.mon_g : nullptr;
#define GC_QSGD_KEPT(M, W)                                                                              \
  hipLaunchKernelGGL((k_qsgd_kept<DEFER, M, W>), qgrid, kBlock, 0, s, (const float*)vals, k,               \
                     (float)qsgd_levels, 1.0f / (float)qsgd_levels, qsgd_seed, out_codes, out_norms,     \
                     (const int64_t*)out_idx, index_base, res, n, pd, mg)
#define GC_QSGD_KEPT_W(M)                     \
  switch (lpg_log2) {                         \
    case 0: GC_QSGD_KEPT(M, 0); break;        \
    case 1: GC_QSGD_KEPT(M, 1); break;        \
    case 2: GC_QSGD_KEPT(M, 2); break;        \
    case 3: GC_QSGD_KEPT(M, 3); break;        \
    case 4: GC_QSGD_KEPT(M, 4); break;        \
    case 5: GC_QSGD_KEPT(M, 5); break;        \
    default: GC_QSGD_KEPT(M, 6); break;       \
  }
    if (DEFER && !mon) {
      // the record takes the residuals in kept order: the streaming form
      const unsigned rgrid = (unsigned)cdiv(k, (int64_t)kBlock * 8);
#define GC_QSGD_REC(W)                                                                                  \
  hipLaunchKernelGGL((k_qsgd_kept_rec<W>), rgrid, kBlock, 0, s, (const float*)vals, k, (float)qsgd_levels, \
                     1.0f / (float)qsgd_levels, qsgd_seed, out_codes, out_norms, pd)
      switch (lpg_log2) {
        case 0: GC_QSGD_REC(0); break;
        case 1: GC_QSGD_REC(1); break;
        case 2: GC_QSGD_REC(2); break;
        case 3: GC_QSGD_REC(3); break;
        case 4: GC_QSGD_REC(4); break;
        case 5: GC_QSGD_REC(5); break;
        default: GC_QSGD_REC(6); break;
      }
#undef GC_QSGD_REC
    } else if (mon) {
      GC_QSGD_KEPT_W(true)
    } else {
      GC_QSGD_KEPT_W(false)
    }
#undef GC_QSGD_KEPT_W
#undef GC_QSGD_KEPT
  } else if (mon) {
    // pure selection sends the kept values themselves
    hipLaunchKernelGGL(k_sq_chunks, (unsigned)l.kchunks, kBlock, 0, s, (const float*)vals, k, l.mon_g);
  }
  if (mon) {
    const int64_t nc2 = cdiv(l.ntiles, kSumChunk), ng2 = cdiv(l.kchunks, kSumChunk);
    hipLaunchKernelGGL(k_sum_f64, (unsigned)nc2, kBlock, 0, s, (const double*)l.mon_c, l.ntiles, l.mon_c2);
    hipLaunchKernelGGL(k_sum_f64, (unsigned)ng2, kBlock, 0, s, (const double*)l.mon_g, l.kchunks, l.mon_g2);
    hipLaunchKernelGGL(k_mon_final, 1, kBlock, 0, s, (const double*)l.mon_c2, nc2, (const double*)l.mon_g2, ng2,
                       stats);
  }
  prof_mark(s, 3);
  return hipGetLastError();
}

}  // namespace

size_t ef_topk_workspace(int64_t n, int64_t k, int qsgd_levels) {
  return make_layout(nullptr, n, k, qsgd_levels > 0, false).bytes;
}

size_t ef_randk_workspace(int64_t n, int64_t k, int qsgd_levels) {
  return make_layout(nullptr, n, k, qsgd_levels > 0, true).bytes;
}

size_t ef_pending_bytes(int64_t n, int64_t kmax) { return pending_layout(nullptr, n, kmax).bytes; }

unsigned long long ef_pending_capacity(int64_t n, size_t bytes) { return pending_capacity(n, bytes); }

hipError_t launch_ef(const EfArgs& a, hipStream_t s) {
  const bool defer = a.pending != nullptr;
#define GC_EF_LAUNCH(R, D)                                                                         \
  launch_select<R, D>(a.grad, a.res, a.n, a.k, a.index_base, a.select_seed, a.out_idx, a.out_val,  \
                      a.qsgd_levels, a.qsgd_group, a.qsgd_seed, a.out_codes, a.out_norms, a.ws,     \
                      a.pending, a.pending_bytes, a.stats, s)
  if (a.randk) return defer ? GC_EF_LAUNCH(true, true) : GC_EF_LAUNCH(true, false);
  return defer ? GC_EF_LAUNCH(false, true) : GC_EF_LAUNCH(false, false);
#undef GC_EF_LAUNCH
}

hipError_t launch_ef_flush(float* res, int64_t n, void* pend, size_t pend_bytes, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const unsigned long long cap = pending_capacity(n, pend_bytes);
  launch_flush(res, n, pending_layout(pend, n, (int64_t)cap), cap, s);
  return hipGetLastError();
}

}  // namespace gc
