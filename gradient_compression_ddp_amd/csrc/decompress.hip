// Decompression at the receiver: dense decode or scatter of one payload, gfx950.
//
// Operation: zyxy.net/archives/25733 "分布式训练中的梯度压缩算法", section 四 (each worker
// decompresses what it receives before the update) and section 二.2 (a sparsified
// gradient is dense with zeros off the kept set).  Each entry's value is the
// dequantization formula of its compressor, in binary32, then multiplied by alpha and
// stored to or added into out[pos].  Streaming: one pass over the payload, scattered
// 4-byte stores (contiguous for a dense decode).
#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

enum { KIND_F32 = 0, KIND_MINMAX8 = 1, KIND_MINMAX4 = 2, KIND_QSGD = 3, KIND_TERN = 4 };

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
