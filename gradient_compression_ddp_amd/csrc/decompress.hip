// Decompression at the receiver: dense decode or scatter of one payload, gfx950.
//
// Operation: zyxy.net/archives/25733 "分布式训练中的梯度压缩算法", section 四 (each worker
// decompresses what it receives before the update) and section 二.2 (a sparsified
// gradient is dense with zeros off the kept set).  Each entry's value is the
// dequantization formula of its compressor, in binary32, then multiplied by alpha and
// stored to or added into out[pos].  The receive side of a data-parallel step (aiqz.cc
// "梯度聚合通信优化实战方案", section "通信瓶颈分析": the workers' gradients are summed and
// averaged) adds W payloads into one vector in payload order; k_decode_sum does it for W
// dense payloads of one shape in a single pass, k_merge_sparse for W sparse payloads tile
// by tile.  Streaming: one pass over the payload, scattered 4-byte stores.  A dense decode (no idx) with aligned buffers takes the tile kernel: one
// 4096-entry tile per block, a lane owns an aligned quad (codes loaded as one word,
// 16-byte non-temporal stores), all loads of the tile issued before any arithmetic.
#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

enum { KIND_F32 = 0, KIND_MINMAX8 = 1, KIND_MINMAX4 = 2, KIND_QSGD = 3, KIND_TERN = 4 };

constexpr int kBlock = 256;
constexpr int kRounds = 4;
constexpr int64_t kTile = (int64_t)kBlock * 4 * kRounds;   // 4096 entries

// The dequantized value of entry j from its code bits `q` (kind-specific meaning).
template <int KIND>
__device__ __forceinline__ float decode_one(uint32_t q, float m0, float m1, float s) {
  if (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) return (float)q * m1 + m0;
  if (KIND == KIND_QSGD) {
    const int c = (int)(int8_t)(uint8_t)q;
    const float level = (float)(c < 0 ? -c : c);
    const float mag = (m0 * level) / s;
    return c < 0 ? -mag : mag;
  }
  // KIND_TERN: 01 -> +s, 11 -> -s, 00 -> 0
  return q == 1u ? m0 : (q == 3u ? -m0 : 0.f);
}

// The four QSGD values of a quad from its code bytes (word, element m in byte m) and the
// norms of their groups: sign * fl(fl(nu * level) / s).  When every nu is >= 2^-100 each
// t = fl(nu * level) is 0 or >= 2^-100 and the quotient comes from div_level_count (the
// same value); otherwise from the division.
__device__ __forceinline__ void qsgd_decode4(uint32_t word, const float nu[4], float s, float ys,
                                             float v[4]) {
  float t[4], mag[4];
  bool small = false;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int c = (int)(int8_t)(uint8_t)(word >> (8 * m));
    t[m] = nu[m] * (float)(c < 0 ? -c : c);
    small |= !(nu[m] >= 0x1p-100f);
    mag[m] = div_level_count(t[m], s, ys);
  }
  if (small) {
#pragma unroll
    for (int m = 0; m < 4; ++m) mag[m] = t[m] / s;
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) v[m] = (int8_t)(uint8_t)(word >> (8 * m)) < 0 ? -mag[m] : mag[m];
}

// Dense decode, entries [0, count) to out[0, count).  Requires out 16-byte aligned and
// codes aligned to one quad's code bytes (16 for F32, 4 for 8-bit codes, 2 for int4).
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_decompress_dense(int64_t count, const void* __restrict__ codes,
                                                             const float* __restrict__ meta0,
                                                             const float* __restrict__ meta1, int64_t G,
                                                             int lg, float s, float ys, float alpha, int accumulate,
                                                             float* __restrict__ out) {
  const int64_t base = (int64_t)blockIdx.x * kTile;
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(codes);
  uint32_t word[kRounds];
  f32x4 fv[kRounds];
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    word[j] = 0u;
    fv[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (e0 + 4 <= count) {
      if (KIND == KIND_F32) fv[j] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(codes) + (e0 >> 2));
      else if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD)
        word[j] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c8 + e0));
      else if (KIND == KIND_MINMAX4)
        word[j] = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(c8 + (e0 >> 1)));
      else
        word[j] = c8[e0 >> 2];
    } else if (e0 < count) {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t e = e0 + m;
        if (e >= count) break;
        if (KIND == KIND_F32) fv[j][m] = reinterpret_cast<const float*>(codes)[e];
        else if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) word[j] |= (uint32_t)c8[e] << (8 * m);
        else if (KIND == KIND_MINMAX4) word[j] |= (uint32_t)((c8[e >> 1] >> (4 * (e & 1))) & 15u) << (4 * m);
        else word[j] |= (uint32_t)((c8[e >> 2] >> (2 * (e & 3))) & 3u) << (2 * m);
      }
    }
  }
#pragma unroll
  for (int j = 0; j < kRounds; ++j) {
    const int64_t e0 = base + j * (kBlock * 4) + threadIdx.x * 4;
    if (e0 >= count) continue;
    float v[4];
    if (KIND == KIND_QSGD) {
      float nu[4];
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t e = e0 + m;
        nu[m] = e < count ? meta0[lg >= 0 ? (e >> lg) : e / G] : 0.f;
      }
      qsgd_decode4(word[j], nu, s, ys, v);
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      if (KIND == KIND_QSGD) {
      } else if (KIND == KIND_F32) {
        v[m] = fv[j][m];
      } else {
        const int64_t e = e0 + m;
        const int64_t g = lg >= 0 ? (e >> lg) : e / G;
        const float m0 = (e < count) ? meta0[g] : 0.f;
        const float m1 = (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) && e < count ? meta1[g] : 0.f;
        uint32_t q;
        if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) q = (word[j] >> (8 * m)) & 0xFFu;
        else if (KIND == KIND_MINMAX4) q = (word[j] >> (4 * m)) & 15u;
        else q = (word[j] >> (2 * m)) & 3u;
        v[m] = decode_one<KIND>(q, m0, m1, s);
      }
    }
    if (e0 + 4 <= count) {
      f32x4 o;
      if (accumulate) {
        const f32x4 prev = *reinterpret_cast<const f32x4*>(out + e0);
        o.x = prev.x + alpha * v[0]; o.y = prev.y + alpha * v[1];
        o.z = prev.z + alpha * v[2]; o.w = prev.w + alpha * v[3];
      } else {
        o.x = alpha * v[0]; o.y = alpha * v[1]; o.z = alpha * v[2]; o.w = alpha * v[3];
      }
      __builtin_nontemporal_store(o, reinterpret_cast<f32x4*>(out + e0));
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        const int64_t e = e0 + m;
        if (e < count) {
          const float a = alpha * v[m];
          out[e] = accumulate ? out[e] + a : a;
        }
      }
    }
  }
}

template <int KIND>
__global__ void k_decompress(const int64_t* __restrict__ idx, int64_t count, int64_t index_base,
                             const void* __restrict__ codes, const float* __restrict__ meta0,
                             const float* __restrict__ meta1, int64_t G, int lg, float s,
                             float alpha, int accumulate, float* __restrict__ out, int64_t n_out) {
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(codes);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < count; j += stride) {
    const int64_t g = lg >= 0 ? (j >> lg) : j / G;
    float v;
    if (KIND == KIND_F32) {
      v = reinterpret_cast<const float*>(codes)[j];
    } else if (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) {
      uint32_t q;
      if (KIND == KIND_MINMAX8) {
        q = c8[j];
      } else {
        const uint32_t byte = c8[j >> 1];
        q = (j & 1) ? (byte >> 4) : (byte & 15u);
      }
      v = (float)q * meta1[g] + meta0[g];
    } else if (KIND == KIND_QSGD) {
      const int c = (int)reinterpret_cast<const int8_t*>(codes)[j];
      const float level = (float)(c < 0 ? -c : c);
      const float mag = (meta0[g] * level) / s;
      v = c < 0 ? -mag : mag;
    } else {
      const uint32_t b = (c8[j >> 2] >> (2 * (j & 3))) & 3u;
      const float sc = meta0[g];
      v = b == 1u ? sc : (b == 3u ? -sc : 0.f);
    }
    const float a = alpha * v;
    const int64_t pos = idx ? idx[j] - index_base : j;
    if (pos >= 0 && pos < n_out) out[pos] = accumulate ? out[pos] + a : a;
  }
}

// ---- the receive side: W dense payloads summed in one pass ---------------------------

constexpr int kMaxFused = 16;

struct FusedSrc {
  const void* codes[kMaxFused];
  const float* meta0[kMaxFused];
  const float* meta1[kMaxFused];
};

// out[e] = (accumulate ? out[e] : 0) + alpha * g_hat_0[e] + ... + alpha * g_hat_{W-1}[e],
// added one payload at a time in payload order, for e < count.  A lane owns an aligned
// quad; each payload's codes for the quad are one word (one float4 for F32).  Requires
// out 16-byte aligned and every codes pointer aligned to one quad's code bytes.  (One
// quad per lane measured fastest: 38 us for eight 25 MiB QSGD payloads against 51 us
// with four quads per lane and 48 us with all W payloads' loads hoisted, both of which
// cut the resident waves.)
template <int KIND>
__global__ __launch_bounds__(kBlock) void k_decode_sum(int W, FusedSrc src, int64_t count, int64_t G, int lg,
                                                       float s, float ys, float alpha, int accumulate,
                                                       float* __restrict__ out) {
  const int64_t e0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * 4;
  if (e0 >= count) return;
  const bool full = e0 + 4 <= count;
  float o[4];
  if (accumulate) {
    if (full) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(out + e0);
      o[0] = p.x; o[1] = p.y; o[2] = p.z; o[3] = p.w;
    } else {
#pragma unroll
      for (int m = 0; m < 4; ++m) o[m] = e0 + m < count ? out[e0 + m] : 0.f;
    }
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = 0.f;
  }
  int64_t g[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) g[m] = lg >= 0 ? ((e0 + m) >> lg) : (e0 + m) / G;
  for (int w = 0; w < W; ++w) {
    const uint8_t* c8 = reinterpret_cast<const uint8_t*>(src.codes[w]);
    float v[4];
    if (KIND == KIND_F32) {
      if (full) {
        const f32x4 a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src.codes[w]) + (e0 >> 2));
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) v[m] = e0 + m < count ? reinterpret_cast<const float*>(src.codes[w])[e0 + m] : 0.f;
      }
    } else {
      uint32_t word = 0u;
      if (full) {
        if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) word = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c8 + e0));
        else if (KIND == KIND_MINMAX4) word = __builtin_nontemporal_load(reinterpret_cast<const uint16_t*>(c8 + (e0 >> 1)));
        else word = c8[e0 >> 2];
      } else {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int64_t e = e0 + m;
          if (e >= count) break;
          if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) word |= (uint32_t)c8[e] << (8 * m);
          else if (KIND == KIND_MINMAX4) word |= (uint32_t)((c8[e >> 1] >> (4 * (e & 1))) & 15u) << (4 * m);
          else word |= (uint32_t)((c8[e >> 2] >> (2 * (e & 3))) & 3u) << (2 * m);
        }
      }
      if (KIND == KIND_QSGD) {
        float nu[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) nu[m] = e0 + m < count ? src.meta0[w][g[m]] : 0.f;
        qsgd_decode4(word, nu, s, ys, v);
      }
#pragma unroll
      for (int m = 0; m < 4; ++m) {
        if (KIND == KIND_QSGD) continue;
        const bool in = e0 + m < count;
        const float m0 = in ? src.meta0[w][g[m]] : 0.f;
        const float m1 = (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) && in ? src.meta1[w][g[m]] : 0.f;
        uint32_t q;
        if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) q = (word >> (8 * m)) & 0xFFu;
        else if (KIND == KIND_MINMAX4) q = (word >> (4 * m)) & 15u;
        else q = (word >> (2 * m)) & 3u;
        v[m] = decode_one<KIND>(q, m0, m1, s);
      }
    }
#pragma unroll
    for (int m = 0; m < 4; ++m) o[m] = o[m] + alpha * v[m];
  }
  if (full) {
    __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(out + e0));
  } else {
#pragma unroll
    for (int m = 0; m < 4; ++m)
      if (e0 + m < count) out[e0 + m] = o[m];
  }
}

// The same sum for packed codes (8-, 4- or 2-bit) whose groups are a power of two of at
// least 16 entries: a lane owns 16 entries of one group, so each payload costs it one
// load of its codes (16, 8 or 4 bytes) and one of each metadata array, and the loads of
// kSumChunk payloads are issued together before they are decoded and added in payload
// order (the same values and the same order of additions as k_decode_sum).  Requires
// out 16-byte aligned and every codes pointer aligned to 16 entries' code bytes; the
// lane holding the ragged end goes entry by entry.
constexpr int kEpl = 16;
constexpr int kSumChunk = 8;

template <int KIND>
__device__ __forceinline__ void decode16(const uint32_t cw[4], float m0, float m1, float s, float ys, float v[kEpl]) {
  if (KIND == KIND_QSGD) {
    // sign * fl(fl(nu * level) / s) = fl(fl(nu * code) / s): multiplication and division
    // round symmetrically, so the signed code gives the same bits; one norm per lane, so
    // the choice of quotient (div_level_count's domain, |t| >= 2^-100 or 0) is per lane
    float t[kEpl];
#pragma unroll
    for (int i = 0; i < kEpl; ++i) t[i] = m0 * (float)(int)(int8_t)(uint8_t)(cw[i >> 2] >> (8 * (i & 3)));
    if (m0 >= 0x1p-100f && m0 <= 0x1p120f) {
      // every t = fl(nu * code), |code| <= 127, is finite: no infinite-t select
#pragma unroll
      for (int i = 0; i < kEpl; ++i) {
        const float q0 = t[i] * ys;
        v[i] = __builtin_fmaf(__builtin_fmaf(-q0, s, t[i]), ys, q0);
      }
    } else if (m0 >= 0x1p-100f) {
#pragma unroll
      for (int i = 0; i < kEpl; ++i) {
        const float q0 = t[i] * ys;
        const float q = __builtin_fmaf(__builtin_fmaf(-q0, s, t[i]), ys, q0);
        v[i] = fabsf(t[i]) <= 3.40282346638528859812e+38f ? q : q0;
      }
    } else {
#pragma unroll
      for (int i = 0; i < kEpl; ++i) v[i] = t[i] / s;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kEpl; ++i) {
      uint32_t q;
      if (KIND == KIND_MINMAX8) q = (cw[i >> 2] >> (8 * (i & 3))) & 0xFFu;
      else if (KIND == KIND_MINMAX4) q = (cw[i >> 3] >> (4 * (i & 7))) & 15u;
      else q = (cw[0] >> (2 * i)) & 3u;
      v[i] = decode_one<KIND>(q, m0, m1, s);
    }
  }
}

template <int KIND>
__global__ __launch_bounds__(kBlock) void k_decode_sum16(int W, FusedSrc src, int64_t count, int lg, float s,
                                                         float ys, float alpha, int accumulate,
                                                         float* __restrict__ out) {
  __shared__ __align__(16) float s_tr[kBlock / kWave][kWave * kEpl];
  const int64_t e0 = ((int64_t)blockIdx.x * kBlock + threadIdx.x) * kEpl;
  if (e0 >= count) return;
  if (e0 + kEpl > count) {
    // the ragged end: entry by entry, payloads in order
    for (int64_t e = e0; e < count; ++e) {
      float o = accumulate ? out[e] : 0.f;
      const int64_t g = e >> lg;
      for (int w = 0; w < W; ++w) {
        const uint8_t* c8 = reinterpret_cast<const uint8_t*>(src.codes[w]);
        uint32_t q;
        if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) q = c8[e];
        else if (KIND == KIND_MINMAX4) q = (c8[e >> 1] >> (4 * (e & 1))) & 15u;
        else q = (c8[e >> 2] >> (2 * (e & 3))) & 3u;
        const float m1 = (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) ? src.meta1[w][g] : 0.f;
        o = o + alpha * decode_one<KIND>(q, src.meta0[w][g], m1, s);
      }
      out[e] = o;
    }
    return;
  }
  const int64_t g = e0 >> lg;
  float o[kEpl];
  if (accumulate) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const f32x4 p = *reinterpret_cast<const f32x4*>(out + e0 + 4 * q);
      o[4 * q] = p.x; o[4 * q + 1] = p.y; o[4 * q + 2] = p.z; o[4 * q + 3] = p.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kEpl; ++i) o[i] = 0.f;
  }
  for (int w0 = 0; w0 < W; w0 += kSumChunk) {
    uint32_t cw[kSumChunk][4];
    float m0[kSumChunk], m1[kSumChunk];
#pragma unroll
    for (int c = 0; c < kSumChunk; ++c) {
      const int w = w0 + c;
#pragma unroll
      for (int q = 0; q < 4; ++q) cw[c][q] = 0u;
      m0[c] = 0.f;
      m1[c] = 0.f;
      if (w < W) {
        const uint8_t* c8 = reinterpret_cast<const uint8_t*>(src.codes[w]);
        if (KIND == KIND_MINMAX8 || KIND == KIND_QSGD) {
          const u32x4 a = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(c8 + e0));
          cw[c][0] = a.x; cw[c][1] = a.y; cw[c][2] = a.z; cw[c][3] = a.w;
        } else if (KIND == KIND_MINMAX4) {
          const u32x2 a = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(c8 + (e0 >> 1)));
          cw[c][0] = a.x; cw[c][1] = a.y;
        } else {
          cw[c][0] = __builtin_nontemporal_load(reinterpret_cast<const uint32_t*>(c8 + (e0 >> 2)));
        }
        m0[c] = src.meta0[w][g];
        if (KIND == KIND_MINMAX8 || KIND == KIND_MINMAX4) m1[c] = src.meta1[w][g];
      }
    }
#pragma unroll
    for (int c = 0; c < kSumChunk; ++c) {
      if (w0 + c >= W) break;   // uniform
      float v[kEpl];
      decode16<KIND>(cw[c], m0[c], m1[c], s, ys, v);
#pragma unroll
      for (int i = 0; i < kEpl; ++i) o[i] = o[i] + alpha * v[i];
    }
  }
  // a wave inside the range stores through LDS, so each store instruction writes 1 KB of
  // consecutive floats (a lane's own 16 floats would make every instruction touch 64 lines)
  const int64_t ew = e0 - (int64_t)lane_id() * kEpl;   // the wave's first entry
  if (ew + kWave * kEpl <= count) {
    float* t = s_tr[threadIdx.x / kWave];
#pragma unroll
    for (int q = 0; q < 4; ++q)
      *reinterpret_cast<f32x4*>(t + lane_id() * kEpl + 4 * q) = f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]};
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(t + q * (kWave * 4) + lane_id() * 4),
                                  reinterpret_cast<f32x4*>(out + ew + q * (kWave * 4)) + lane_id());
  } else {
#pragma unroll
    for (int q = 0; q < 4; ++q)
      __builtin_nontemporal_store(f32x4{o[4 * q], o[4 * q + 1], o[4 * q + 2], o[4 * q + 3]},
                                  reinterpret_cast<f32x4*>(out + e0 + 4 * q));
  }
}

// ---- the receive side: W sparse payloads merged tile by tile --------------------------
// Each payload's idx is strictly ascending, so the entries of one output tile are a run of
// consecutive entries of every payload.  A block walks kMergeTilesPerBlock tiles of 4096
// outputs with one cursor per payload (a lower-bound search at its first tile).  Per tile,
// wave v stages the tile's run of payload g0 + v (position in the tile and alpha * g_hat)
// in LDS, then all threads add the staged runs into an LDS copy of the tile in payload
// order, one barrier per payload, and the tile is written once.  A run longer than the
// staging space is finished block-wide, in order, before the next payload.  The output
// is written once and each payload read once, where the per-payload scatter read and wrote
// a 64-byte sector of out for every entry (after a pass that cleared it).

constexpr int kMergeTile = 4096;
constexpr int kMergeTilesPerBlock = 8;
constexpr int kMergeCap = 512;     // staged entries per payload per tile
constexpr int kMergeBlock = 512;   // 8 waves: 8 payloads staged at once
constexpr int kMergeWaves = kMergeBlock / kWave;

struct SparseSrc {
  const int64_t* idx[kMaxFused];
  const void* codes[kMaxFused];
  const float* meta0[kMaxFused];
  const float* meta1[kMaxFused];
  int64_t count[kMaxFused];
  int64_t index_base[kMaxFused];
  int64_t G[kMaxFused];
  int lg[kMaxFused];      // log2(G), or -1
  int kind[kMaxFused];
  float s[kMaxFused];     // QSGD level count (1 for other kinds)
};

// g_hat of entry j of payload w, as k_decompress decodes it.
__device__ __forceinline__ float decode_entry(const SparseSrc& S, int w, int64_t j) {
  const int64_t g = S.lg[w] >= 0 ? (j >> S.lg[w]) : j / S.G[w];
  const uint8_t* c8 = reinterpret_cast<const uint8_t*>(S.codes[w]);
  switch (S.kind[w]) {
    case KIND_F32:
      return reinterpret_cast<const float*>(S.codes[w])[j];
    case KIND_MINMAX8:
      return (float)c8[j] * S.meta1[w][g] + S.meta0[w][g];
    case KIND_MINMAX4: {
      const uint32_t byte = c8[j >> 1];
      const uint32_t q = (j & 1) ? (byte >> 4) : (byte & 15u);
      return (float)q * S.meta1[w][g] + S.meta0[w][g];
    }
    case KIND_QSGD: {
      const int c = (int)reinterpret_cast<const int8_t*>(S.codes[w])[j];
      const float level = (float)(c < 0 ? -c : c);
      const float mag = (S.meta0[w][g] * level) / S.s[w];
      return c < 0 ? -mag : mag;
    }
    default: {
      const uint32_t b = (c8[j >> 2] >> (2 * (j & 3))) & 3u;
      const float sc = S.meta0[w][g];
      return b == 1u ? sc : (b == 3u ? -sc : 0.f);
    }
  }
}

// First entry of idx[0, count) that is >= key, by one wave: each step probes 64 evenly
// spaced entries of the open range and keeps the gap between the last probe below key and
// the first at or above it (the probes ascend, so the ones below key are a prefix of the
// lanes), a 64-fold cut per dependent load (4 loads for a million entries) instead of
// 2-fold.  Every lane of the wave calls it and gets the answer.
__device__ __forceinline__ int64_t lower_bound_wave(const int64_t* __restrict__ idx, int64_t count, int64_t key) {
  const int lane = lane_id();
  int64_t lo = 0, hi = count;   // the answer lies in [lo, hi]
  while (lo < hi) {
    const int64_t span = hi - lo;
    const int64_t step = span <= kWave ? 1 : (span + kWave - 1) / kWave;
    const int64_t p = lo + (int64_t)lane * step;
    const bool valid = p < hi;
    const uint64_t below = ballot(valid && idx[p] < key);
    const int m = __popcll(below);
    if (m == 0) return lo;
    const int nvalid = __popcll(ballot(valid));
    const int64_t last = lo + (int64_t)(m - 1) * step;   // the last probe below key
    hi = m < nvalid ? lo + (int64_t)m * step : hi;
    lo = last + 1;
  }
  return lo;
}

__global__ __launch_bounds__(kMergeBlock) void k_merge_sparse(int W, SparseSrc S, float alpha, int accumulate,
                                                         int vec, float* __restrict__ out, int64_t n_out) {
  __shared__ __align__(16) float tile[kMergeTile];
  __shared__ uint16_t st_pos[kMergeWaves][kMergeCap];
  __shared__ float st_val[kMergeWaves][kMergeCap];
  __shared__ int64_t cur[kMaxFused];
  __shared__ int st_n[kMergeWaves];
  __shared__ int st_done[kMergeWaves];
  __shared__ int s_cnt[kMergeWaves];
  const int wave = threadIdx.x / kWave;
  const int lane = lane_id();
  const int64_t ntiles = (n_out + kMergeTile - 1) / kMergeTile;
  const int64_t t0 = (int64_t)blockIdx.x * kMergeTilesPerBlock;
  const int64_t t1 = t0 + kMergeTilesPerBlock < ntiles ? t0 + kMergeTilesPerBlock : ntiles;
  for (int w = wave; w < W; w += kMergeWaves) {
    const int64_t c = lower_bound_wave(S.idx[w], S.count[w], t0 * kMergeTile + S.index_base[w]);
    if (lane == 0) cur[w] = c;
  }
  for (int64_t t = t0; t < t1; ++t) {
    const int64_t q0 = t * kMergeTile;
    const int len = n_out - q0 < kMergeTile ? (int)(n_out - q0) : kMergeTile;
    const bool full = vec && len == kMergeTile;
    if (full) {
      for (int i = threadIdx.x; i < kMergeTile / 4; i += kMergeBlock)
        reinterpret_cast<f32x4*>(tile)[i] =
            accumulate ? reinterpret_cast<const f32x4*>(out + q0)[i] : f32x4{0.f, 0.f, 0.f, 0.f};
    } else {
      for (int i = threadIdx.x; i < len; i += kMergeBlock) tile[i] = accumulate ? out[q0 + i] : 0.f;
    }
    __syncthreads();   // the tile is initialised; cur holds this tile's first entries
    for (int g0 = 0; g0 < W; g0 += kMergeWaves) {
      const int w = g0 + wave;
      if (w < W) {
        const int64_t lo = q0 + S.index_base[w], lim = lo + len;
        int64_t c = cur[w];
        int n = 0;
        bool done = false;
        while (!done && n + kWave <= kMergeCap) {
          const int64_t j = c + lane;
          // the entry's code and metadata loads do not wait for its index
          const bool in = j < S.count[w];
          const int64_t e = in ? S.idx[w][j] : 0;
          const float a = in ? alpha * decode_entry(S, w, j) : 0.f;
          const bool ok = in && e >= lo && e < lim;    // ascending: the ok lanes are a prefix
          const int cnt = __popcll(ballot(ok));
          if (ok) {
            st_pos[wave][n + lane] = (uint16_t)(e - lo);
            st_val[wave][n + lane] = a;
          }
          n += cnt;
          c += cnt;
          done = cnt < kWave;
        }
        if (lane == 0) { st_n[wave] = n; st_done[wave] = done ? 1 : 0; cur[w] = c; }
      }
      __syncthreads();
      for (int v = 0; v < kMergeWaves && g0 + v < W; ++v) {
        const int n = st_n[v];
        for (int i = threadIdx.x; i < n; i += kMergeBlock) {
          const int p = st_pos[v][i];
          tile[p] = tile[p] + st_val[v][i];
        }
        __syncthreads();
        if (!st_done[v]) {
          // the rest of payload g0 + v's run in this tile, block-wide and in order
          const int w2 = g0 + v;
          const int64_t lo = q0 + S.index_base[w2], lim = lo + len;
          for (;;) {
            const int64_t c = cur[w2];
            const int64_t j = c + threadIdx.x;
            int64_t e = 0;
            bool ok = j < S.count[w2];
            if (ok) e = S.idx[w2][j];
            ok = ok && e >= lo && e < lim;
            const int wc = __popcll(ballot(ok));   // every lane takes part in the ballot
            if (lane == 0) s_cnt[wave] = wc;
            if (ok) {
              const int p = (int)(e - lo);
              tile[p] = tile[p] + alpha * decode_entry(S, w2, j);
            }
            __syncthreads();
            int total = 0;
#pragma unroll
            for (int i = 0; i < kMergeWaves; ++i) total += s_cnt[i];
            __syncthreads();   // every thread has read cur[w2] and s_cnt
            if (threadIdx.x == 0) cur[w2] = c + total;
            __syncthreads();
            if (total < kMergeBlock) break;
          }
        }
      }
    }
    if (full) {
      for (int i = threadIdx.x; i < kMergeTile / 4; i += kMergeBlock)
        __builtin_nontemporal_store(reinterpret_cast<const f32x4*>(tile)[i], reinterpret_cast<f32x4*>(out + q0) + i);
    } else {
      for (int i = threadIdx.x; i < len; i += kMergeBlock) out[q0 + i] = tile[i];
    }
    __syncthreads();   // the tile is written before the next one is initialised
  }
}

__global__ void k_fill_zero(float* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0.f;
}

}  // namespace

hipError_t launch_decompress(int kind, const int64_t* idx, int64_t count, int64_t index_base,
                             const void* codes, const float* meta0, const float* meta1,
                             int64_t group, int levels, float alpha, int accumulate, float* out,
                             int64_t n_out, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const int64_t G = group == 0 ? count : group;
  int lg = -1;
  if ((G & (G - 1)) == 0) {
    lg = 0;
    while ((int64_t(1) << lg) < G) ++lg;
  }
  const auto al = [](const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; };
  const uintptr_t code_align = kind == KIND_F32 ? 16 : (kind == KIND_MINMAX4 ? 2 : (kind == KIND_TERN ? 1 : 4));
  if (!idx && al(out, 16) && al(codes, code_align)) {
    const int64_t tiles = (count + kTile - 1) / kTile;
    const float sd = (float)(levels > 0 ? levels : 1);
#define GC_LAUNCH_DENSE(K)                                                                          \
  hipLaunchKernelGGL((k_decompress_dense<K>), (unsigned)tiles, kBlock, 0, s, count, codes, meta0, meta1, \
                     G, lg, sd, 1.0f / sd, alpha, accumulate, out)
    switch (kind) {
      case KIND_F32: GC_LAUNCH_DENSE(KIND_F32); break;
      case KIND_MINMAX8: GC_LAUNCH_DENSE(KIND_MINMAX8); break;
      case KIND_MINMAX4: GC_LAUNCH_DENSE(KIND_MINMAX4); break;
      case KIND_QSGD: GC_LAUNCH_DENSE(KIND_QSGD); break;
      default: GC_LAUNCH_DENSE(KIND_TERN); break;
    }
#undef GC_LAUNCH_DENSE
    return hipGetLastError();
  }
  int64_t blocks = (count + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 16;
  if (blocks > cap) blocks = cap;
  const float sf = (float)(levels > 0 ? levels : 1);
#define GC_LAUNCH(K)                                                                           \
  hipLaunchKernelGGL((k_decompress<K>), (int)blocks, 256, 0, s, idx, count, index_base, codes, \
                     meta0, meta1, G, lg, sf, alpha, accumulate, out, n_out)
  switch (kind) {
    case KIND_F32: GC_LAUNCH(KIND_F32); break;
    case KIND_MINMAX8: GC_LAUNCH(KIND_MINMAX8); break;
    case KIND_MINMAX4: GC_LAUNCH(KIND_MINMAX4); break;
    case KIND_QSGD: GC_LAUNCH(KIND_QSGD); break;
    default: GC_LAUNCH(KIND_TERN); break;
  }
#undef GC_LAUNCH
  return hipGetLastError();
}

}  // namespace gc

namespace gc {

hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s) {
  if (n == 0) return hipSuccess;
  int64_t blocks = (n + 255) / 256;
  const int64_t cap = (int64_t)device_cu_count() * 8;
  if (blocks > cap) blocks = cap;
  hipLaunchKernelGGL(k_fill_zero, (unsigned)blocks, 256, 0, s, p, n);
  return hipGetLastError();
}

hipError_t launch_merge_sparse(int W, const int64_t* const* idx, const void* const* codes,
                               const float* const* meta0, const float* const* meta1, const int64_t* count,
                               const int64_t* index_base, const int64_t* group, const int* kind,
                               const int* levels, float alpha, int accumulate, float* out, int64_t n_out,
                               hipStream_t s) {
  if (n_out == 0 || W == 0) return hipSuccess;
  const int64_t ntiles = (n_out + kMergeTile - 1) / kMergeTile;
  const unsigned blocks = (unsigned)((ntiles + kMergeTilesPerBlock - 1) / kMergeTilesPerBlock);
  const int vec = (reinterpret_cast<uintptr_t>(out) % 16) == 0 ? 1 : 0;
  for (int w0 = 0; w0 < W; w0 += kMaxFused) {
    const int nw = W - w0 < kMaxFused ? W - w0 : kMaxFused;
    SparseSrc S{};
    for (int i = 0; i < nw; ++i) {
      const int w = w0 + i;
      const int64_t G = group[w] == 0 ? (count[w] > 0 ? count[w] : 1) : group[w];
      int lg = -1;
      if ((G & (G - 1)) == 0) {
        lg = 0;
        while ((int64_t(1) << lg) < G) ++lg;
      }
      S.idx[i] = idx[w];
      S.codes[i] = codes[w];
      S.meta0[i] = meta0[w];
      S.meta1[i] = meta1[w];
      S.count[i] = count[w];
      S.index_base[i] = index_base[w];
      S.G[i] = G;
      S.lg[i] = lg;
      S.kind[i] = kind[w];
      S.s[i] = (float)(levels[w] > 0 ? levels[w] : 1);
    }
    const int acc = w0 == 0 ? accumulate : 1;   // later launches add to what the first wrote
    hipLaunchKernelGGL(k_merge_sparse, blocks, kMergeBlock, 0, s, nw, S, alpha, acc, vec, out, n_out);
  }
  return hipGetLastError();
}

hipError_t launch_decode_sum(int kind, int W, const void* const* codes, const float* const* meta0,
                             const float* const* meta1, int64_t count, int64_t group, int levels, float alpha,
                             int accumulate, float* out, hipStream_t s) {
  if (count == 0 || W == 0) return hipSuccess;
  const int64_t G = group == 0 ? count : group;
  int lg = -1;
  if ((G & (G - 1)) == 0) {
    lg = 0;
    while ((int64_t(1) << lg) < G) ++lg;
  }
  const float sd = (float)(levels > 0 ? levels : 1);
  const unsigned blocks = (unsigned)((count + kBlock * 4 - 1) / (kBlock * 4));
  // the 16-entry path: packed codes, groups of a power of two >= 16, codes aligned to 16
  // entries' code bytes
  const int cbytes16 = kind == KIND_MINMAX8 || kind == KIND_QSGD ? 16 : (kind == KIND_MINMAX4 ? 8 : 4);
  bool wide = kind != KIND_F32 && lg >= 4;
  for (int i = 0; wide && i < W; ++i) wide = (reinterpret_cast<uintptr_t>(codes[i]) % cbytes16) == 0;
  const unsigned blocks16 = (unsigned)((count + kBlock * kEpl - 1) / (kBlock * kEpl));
  for (int w0 = 0; w0 < W; w0 += kMaxFused) {
    const int nw = W - w0 < kMaxFused ? W - w0 : kMaxFused;
    FusedSrc src{};
    for (int i = 0; i < nw; ++i) {
      src.codes[i] = codes[w0 + i];
      src.meta0[i] = meta0 ? meta0[w0 + i] : nullptr;
      src.meta1[i] = meta1 ? meta1[w0 + i] : nullptr;
    }
    const int acc = w0 == 0 ? accumulate : 1;   // later launches add to what the first wrote
#define GC_LAUNCH_SUM16(K) \
    hipLaunchKernelGGL((k_decode_sum16<K>), blocks16, kBlock, 0, s, nw, src, count, lg, sd, 1.0f / sd, alpha, acc, out)
    if (wide) {
      switch (kind) {
        case KIND_MINMAX8: GC_LAUNCH_SUM16(KIND_MINMAX8); break;
        case KIND_MINMAX4: GC_LAUNCH_SUM16(KIND_MINMAX4); break;
        case KIND_QSGD: GC_LAUNCH_SUM16(KIND_QSGD); break;
        default: GC_LAUNCH_SUM16(KIND_TERN); break;
      }
      continue;
    }
#undef GC_LAUNCH_SUM16
#define GC_LAUNCH_SUM(K) \
    hipLaunchKernelGGL((k_decode_sum<K>), blocks, kBlock, 0, s, nw, src, count, G, lg, sd, 1.0f / sd, alpha, acc, out)
    switch (kind) {
      case KIND_F32: GC_LAUNCH_SUM(KIND_F32); break;
      case KIND_MINMAX8: GC_LAUNCH_SUM(KIND_MINMAX8); break;
      case KIND_MINMAX4: GC_LAUNCH_SUM(KIND_MINMAX4); break;
      case KIND_QSGD: GC_LAUNCH_SUM(KIND_QSGD); break;
      default: GC_LAUNCH_SUM(KIND_TERN); break;
    }
#undef GC_LAUNCH_SUM
  }
  return hipGetLastError();
}

}  // namespace gc
