// gc_ef_compress_noalloc: gc_ef_compress whose workspace is a fixed device array of this
// library, for callers that cannot allocate device memory (code under stream capture,
// serving loops that must not call the allocator).
//
// The array lives in the library's code object, so every GPU the library runs on holds
// its own copy until the process ends.  Host code never passes the array's name to a
// kernel (on the host that name is only a stand-in, not a device address): the first
// call on each device looks up the device address of that device's copy with
// hipGetSymbolAddress and keeps it, and every later call on that device passes the
// kept address as the workspace.  The EF Top-K / Random-K pipeline resets the parts of
// its workspace that must start at zero on every call, so a call does not depend on
// what the previous call left behind.  Calls that overlap on one GPU (several streams or
// threads at once) share the one array and race.
#include <hip/hip_runtime.h>

#include <mutex>

#include "gc.h"
#include "internal.hpp"

namespace {

constexpr size_t kScratchBytes = size_t(32) << 20;     // 32 MiB per GPU
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices] = {};

// Device address of the current device's copy of `scratch`, looked up once per device.
int scratch_address(void** out) {
  int dev = -1;
  const hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return gc::report(GC_EHIP, "hipGetDevice: %s", hipGetErrorString(e));
  if (dev < 0 || dev >= kMaxDevices) return gc::report(GC_EINVAL, "device %d beyond the %d this call supports", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* p = nullptr;
    const hipError_t g = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (g != hipSuccess || !p)
      return gc::report(GC_EHIP, "hipGetSymbolAddress of the scratch array on device %d: %s", dev,
                        hipGetErrorString(g));
    g_scratch[dev] = p;
  }
  *out = g_scratch[dev];
  return GC_OK;
}

}  // namespace

extern "C" {

size_t gc_noalloc_scratch_bytes(void) { return kScratchBytes; }

int gc_ef_compress_noalloc(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                           int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group,
                           uint64_t qsgd_seed, int8_t* out_codes, float* out_norms, const gc_ef_options* opts,
                           void* stream) {
  size_t need = 0;
  const int st = gc::ef_compress_check(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group,
                                       out_codes, out_norms, opts, &need);
  if (st != GC_OK) return st;
  if (need > kScratchBytes)
    return gc::report(GC_EWORKSPACE,
                      "gc_ef_compress_noalloc: n = %lld, k = %lld needs %zu bytes of workspace, more than the "
                      "%zu-byte fixed scratch; call gc_ef_compress with a workspace instead",
                      (long long)n, (long long)k, need, kScratchBytes);
  if (need == 0)   // n == 0 or k == 0: no workspace is touched
    return gc_ef_compress(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group, qsgd_seed,
                          out_codes, out_norms, opts, nullptr, 0, stream);
  void* ws = nullptr;
  const int a = scratch_address(&ws);
  if (a != GC_OK) return a;
  return gc_ef_compress(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group, qsgd_seed,
                        out_codes, out_norms, opts, ws, kScratchBytes, stream);
}

}  // extern "C"
