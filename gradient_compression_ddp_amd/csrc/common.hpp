// Device-side building blocks shared by the gfx950 kernels: the Philox4x32-10 counter
// RNG, wave64 reductions and scans, and the float <-> ordered-integer encodings used by
// the min/max and Top-K code.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gc {

constexpr int kWave = 64;

// Native 4 x fp32 vector (usable with the nontemporal load/store builtins).
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// ---------------------------------------------------------------------------------
// Philox4x32-10 (Salmon, Moraes, Dror, Shaw, SC'11).  One block: counter
// (c0, c1, 0, 0) under key (k0, k1).  Each round forms the two 32x32->64 products
// M0*x0 and M1*x2 and the new state (hi1^x1^k0, lo1, hi0^x3^k1, lo0); the key is
// bumped by the Weyl constants between rounds.  The key is wave-uniform (the seed), so
// its schedule stays in scalar registers.
// ---------------------------------------------------------------------------------
struct Words4 {
  uint32_t w[4];
};

// gfx950's three-input bitwise op with truth table 0x96 (a ^ b ^ c) forms each new state
// word in one instruction.
__device__ __forceinline__ uint32_t xor3(uint32_t a, uint32_t b, uint32_t c) {
  return __builtin_amdgcn_bitop3_b32(a, b, c, 0x96);
}

__device__ __forceinline__ Words4 philox10(uint32_t c0, uint32_t c1, uint32_t k0, uint32_t k1) {
  constexpr uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
  constexpr uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
  // the first Philox round: the counter's words 2 and 3 are 0, so M1 * x2 = 0
  const uint64_t q0 = (uint64_t)M0 * (uint64_t)c0;
  uint32_t x0 = c1 ^ k0, x1 = 0u, x2 = (uint32_t)(q0 >> 32) ^ k1, x3 = (uint32_t)q0;
  k0 += W0;
  k1 += W1;
#pragma unroll
  for (int r = 1; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)M0 * (uint64_t)x0;
    const uint64_t p1 = (uint64_t)M1 * (uint64_t)x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    x0 = xor3(hi1, x1, k0);
    x1 = lo1;
    x2 = xor3(hi0, x3, k1);
    x3 = lo0;
    k0 += W0;
    k1 += W1;
  }
  Words4 o;
  o.w[0] = x0; o.w[1] = x1; o.w[2] = x2; o.w[3] = x3;
  return o;
}

// Block holding element indices [4*ctr, 4*ctr+4) of the stream keyed by `seed`.
__device__ __forceinline__ Words4 philox_block(uint64_t seed, uint64_t ctr) {
  return philox10((uint32_t)ctr, (uint32_t)(ctr >> 32), (uint32_t)seed, (uint32_t)(seed >> 32));
}

// 24-bit uniform in [0,1): (word >> 8) * 2^-24, exact in fp32.
__device__ __forceinline__ float u24(uint32_t w) {
  return (float)(w >> 8) * 5.9604644775390625e-08f;
}

// Raw words of the four consecutive element indices e0..e0+3 (any alignment).  When
// e0 % 4 == 0 this is one Philox block; otherwise two blocks are stitched.
__device__ __forceinline__ void words4(uint64_t seed, uint64_t e0, uint32_t out[4]) {
  const uint64_t c = e0 >> 2;
  const uint32_t sh = (uint32_t)(e0 & 3u);
  const Words4 a = philox_block(seed, c);
  if (sh == 0) {
#pragma unroll
    for (int m = 0; m < 4; ++m) out[m] = a.w[m];
  } else {
    const Words4 b = philox_block(seed, c + 1);
    uint32_t w[8];
#pragma unroll
    for (int m = 0; m < 4; ++m) { w[m] = a.w[m]; w[4 + m] = b.w[m]; }
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      // select w[sh + m] without dynamic register indexing
      uint32_t v = w[m + 1];
      v = (sh == 2) ? w[m + 2] : v;
      v = (sh == 3) ? w[m + 3] : v;
      out[m] = v;
    }
  }
}

// Uniforms of the four consecutive element indices e0..e0+3 (any alignment).
__device__ __forceinline__ void uniforms4(uint64_t seed, uint64_t e0, float u[4]) {
  uint32_t w[4];
  words4(seed, e0, w);
#pragma unroll
  for (int m = 0; m < 4; ++m) u[m] = u24(w[m]);
}

// Raw words of e0..e0+3 when the caller knows at compile time whether e0 % 4 == 0.
template <bool ALIGNED>
__device__ __forceinline__ void words4_t(uint64_t seed, uint64_t e0, uint32_t out[4]) {
  if constexpr (ALIGNED) {
    const Words4 a = philox_block(seed, e0 >> 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) out[m] = a.w[m];
  } else {
    words4(seed, e0, out);
  }
}

// The same when the caller knows at compile time whether e0 % 4 == 0 (ALIGNED: one
// Philox block).  Kernels whose element indices are index_base + a multiple of 4 choose
// the variant at launch from index_base % 4: the alignment is uniform, yet with only the
// general form the compiler computed both blocks of words4 on every quad.
template <bool ALIGNED>
__device__ __forceinline__ void uniforms4_t(uint64_t seed, uint64_t e0, float u[4]) {
  if constexpr (ALIGNED) {
    const Words4 a = philox_block(seed, e0 >> 2);
#pragma unroll
    for (int m = 0; m < 4; ++m) u[m] = u24(a.w[m]);
  } else {
    uniforms4(seed, e0, u);
  }
}

// The word of one element index.
__device__ __forceinline__ uint32_t philox_word(uint64_t seed, uint64_t e) {
  const Words4 a = philox_block(seed, e >> 2);
  const uint32_t sh = (uint32_t)(e & 3u);
  uint32_t v = a.w[0];
  v = (sh == 1) ? a.w[1] : v;
  v = (sh == 2) ? a.w[2] : v;
  v = (sh == 3) ? a.w[3] : v;
  return v;
}

// ---------------------------------------------------------------------------------
// fl(t / s) for a QSGD level count s in [1, 127] and t = 0 or t >= 2^-100, with
// ys = fl(1/s): the product q0 = fl(t * ys), then one correction with the exact remainder
// fma(-q0, s, t).  On that domain it equals the IEEE quotient for every s (checked
// exhaustively on the CPU, every binary32 t of the domain) except t = +Inf, whose
// remainder is NaN; there, and for NaN t, q0 (+Inf or NaN) is the quotient.  Below 2^-100
// it can miss: for even s that are not powers of two a subnormal quotient can be an exact
// midpoint, which the correction rounds the wrong way, so callers divide there.  Three
// full-rate operations and a select in place of the division sequence.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ float div_level_count(float t, float s, float ys) {
  const float q0 = t * ys;
  const float r = __builtin_fmaf(-q0, s, t);
  const float q = __builtin_fmaf(r, ys, q0);
  return t <= 3.40282346638528859812e+38f ? q : q0;
}

// ---------------------------------------------------------------------------------
// Float encodings.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t fbits(float f) { return __float_as_uint(f); }
__device__ __forceinline__ float bitsf(uint32_t u) { return __uint_as_float(u); }

// Magnitude key: bit pattern with the sign cleared.
__device__ __forceinline__ uint32_t mag_key(float f) { return fbits(f) & 0x7FFFFFFFu; }

// Monotone map float -> uint32 for the total order -inf < ... < -0 < +0 < ... < +inf:
// a negative pattern has all its bits flipped, any other gets the sign bit set (one xor
// with the sign spread by an arithmetic shift).
__device__ __forceinline__ uint32_t ord_enc(float f) {
  const uint32_t b = fbits(f);
  return b ^ ((uint32_t)((int32_t)b >> 31) | 0x80000000u);
}
__device__ __forceinline__ float ord_dec(uint32_t e) {
  return bitsf((e & 0x80000000u) ? (e & 0x7FFFFFFFu) : ~e);
}

// ---------------------------------------------------------------------------------
// Wave64 helpers.
// ---------------------------------------------------------------------------------
__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Number of set bits of `mask` in lanes below this one.
__device__ __forceinline__ uint32_t mbcnt(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

template <typename T>
__device__ __forceinline__ T shfl_xor(T v, int m) { return __shfl_xor(v, m, kWave); }

// Butterfly min/max of ordered-encoded values over aligned segments of `width` lanes.
__device__ __forceinline__ uint32_t seg_min_u32(uint32_t v, int width) {
  for (int m = 1; m < width; m <<= 1) v = min(v, (uint32_t)shfl_xor((int)v, m));
  return v;
}
__device__ __forceinline__ uint32_t seg_max_u32(uint32_t v, int width) {
  for (int m = 1; m < width; m <<= 1) v = max(v, (uint32_t)shfl_xor((int)v, m));
  return v;
}

// Butterfly partner of compile-time step S (partner lane = lane ^ 2^S) for reductions in
// which every lane of a segment ends with the segment's result.  Steps 0 and 1 are DPP
// quad permutes ([1,0,3,2], [2,3,0,1]).  Once every quad holds one value, the half-row
// mirror (lane i <-> 7 - i within 8) pairs each lane with a lane of the other quad, and
// once every 8 lanes hold one value the row mirror (i <-> 15 - i within 16) pairs each
// with a lane of the other half: the same partial results the xor steps 2 and 3 pair, so
// the combined values are identical.  All four are DPP operand modifiers, with no LDS
// traffic; steps 4 and 5 (16 and 32 lanes) shuffle.  None of these permutes reads a lane
// outside its row, so bound_ctrl never applies, and leaving the old value undefined lets
// the compiler fold each move into the min, max or add that uses it (one instruction a step).
template <int S>
__device__ __forceinline__ uint32_t bfly_u32(uint32_t v) {
  static_assert(S >= 0 && S <= 5, "butterfly step");
  if constexpr (S == 0) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0xB1, 0xF, 0xF, true);
  else if constexpr (S == 1) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x4E, 0xF, 0xF, true);
  else if constexpr (S == 2) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x141, 0xF, 0xF, true);
  else if constexpr (S == 3) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x140, 0xF, 0xF, true);
  else return (uint32_t)__shfl_xor((int)v, 1 << S, kWave);
}

// Min / max / pairwise-tree sum over aligned segments of 2^W lanes, W known at compile time.
template <int W>
__device__ __forceinline__ uint32_t seg_min_c(uint32_t v) {
  if constexpr (W > 0) v = min(v, bfly_u32<0>(v));
  if constexpr (W > 1) v = min(v, bfly_u32<1>(v));
  if constexpr (W > 2) v = min(v, bfly_u32<2>(v));
  if constexpr (W > 3) v = min(v, bfly_u32<3>(v));
  if constexpr (W > 4) v = min(v, bfly_u32<4>(v));
  if constexpr (W > 5) v = min(v, bfly_u32<5>(v));
  return v;
}
template <int W>
__device__ __forceinline__ uint32_t seg_max_c(uint32_t v) {
  if constexpr (W > 0) v = max(v, bfly_u32<0>(v));
  if constexpr (W > 1) v = max(v, bfly_u32<1>(v));
  if constexpr (W > 2) v = max(v, bfly_u32<2>(v));
  if constexpr (W > 3) v = max(v, bfly_u32<3>(v));
  if constexpr (W > 4) v = max(v, bfly_u32<4>(v));
  if constexpr (W > 5) v = max(v, bfly_u32<5>(v));
  return v;
}
// the tree's level-S additions: a + b and b + a are the same IEEE result, so each lane's
// sum equals the tree's node
template <int W>
__device__ __forceinline__ float seg_tree_sum_c(float v) {
  if constexpr (W > 0) v = v + __uint_as_float(bfly_u32<0>(__float_as_uint(v)));
  if constexpr (W > 1) v = v + __uint_as_float(bfly_u32<1>(__float_as_uint(v)));
  if constexpr (W > 2) v = v + __uint_as_float(bfly_u32<2>(__float_as_uint(v)));
  if constexpr (W > 3) v = v + __uint_as_float(bfly_u32<3>(__float_as_uint(v)));
  if constexpr (W > 4) v = v + __uint_as_float(bfly_u32<4>(__float_as_uint(v)));
  if constexpr (W > 5) v = v + __uint_as_float(bfly_u32<5>(__float_as_uint(v)));
  return v;
}

// Float sum over aligned segments of `width` lanes as a balanced pairwise tree in lane
// order: the xor butterfly with offsets 1, 2, 4, ... adds exactly the pairs of the
// tree (a + b and b + a are the same IEEE result), and every lane ends with the sum.
__device__ __forceinline__ float seg_tree_sum(float v, int width) {
  for (int m = 1; m < width; m <<= 1) v = v + shfl_xor(v, m);
  return v;
}

// Inclusive scan (sum) of 64-bit counts across the wave.
__device__ __forceinline__ uint64_t wave_incl_scan_u64(uint64_t v) {
  const int l = lane_id();
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    const uint64_t o = __shfl_up(v, d, kWave);
    if (l >= d) v += o;
  }
  return v;
}

// float64 sum across the wave by the xor butterfly (a fixed order; every lane ends with
// the sum).
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

__device__ __forceinline__ uint64_t wave_sum_u64(uint64_t v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Last-block hand-off: every block of a grid calls this once, after its global writes and
// atomics; it returns true in exactly one block, the last to arrive, which then sees the
// writes of every block.  Nothing waits on anything, so every block runs to its end; the
// ticket is zero again once the last block has it.  One device-scope release per block
// (its first thread's ticket increment, after the barrier that orders the block's writes
// before it) and one acquire in the last block: a full fence in every wave costs an L2
// write-back and invalidate each, which measured slower than the launch this saves.
__device__ __forceinline__ bool last_block(uint32_t* ticket) {
  __shared__ uint32_t s_last;
  // each wave's own global stores and atomics have completed before the barrier (the
  // barrier alone does not wait for them), so the first thread's release covers them all
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t t = __hip_atomic_fetch_add(ticket, 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = t == gridDim.x - 1;
    if (last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      __hip_atomic_store(ticket, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    s_last = last ? 1u : 0u;
  }
  __syncthreads();
  return s_last != 0u;
}

}  // namespace gc
