// Host-side launchers of the gfx950 kernels.  capi.cpp validates every argument
// before calling these; the launchers only size grids and enqueue work on `stream`.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

struct gc_ef_options;   // include/gc.h

namespace gc {

// Round a byte count up to the 256-byte alignment used for every workspace carve-out.
inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

// ---- min-max -------------------------------------------------------------------
// Small groups (power of two in [4,256]): one pass, a group spans group/4 lanes.
hipError_t launch_minmax_small(const float* x, float* res, int64_t n, int64_t group, int bits,
                               uint8_t* codes, float* mins, float* scales, hipStream_t s);
// Large groups (> 256, or the whole tensor): reduce, finalize, quantize.
size_t minmax_large_workspace(int64_t n, int64_t group);
hipError_t launch_minmax_large(const float* x, float* res, int64_t n, int64_t group, int bits,
                               uint8_t* codes, float* mins, float* scales, void* ws,
                               hipStream_t s);

// out[i] = (x[i] > 0): the 4 B -> 1 B streaming floor benchmarks time beside the quantizers.
hipError_t launch_stream_floor(const float* x, uint8_t* out, int64_t n, hipStream_t s);

// ---- QSGD ----------------------------------------------------------------------
hipError_t launch_qsgd(const float* x, float* res, int64_t n, int64_t group, int levels,
                       uint64_t seed, int64_t index_base, int8_t* codes, float* norms,
                       hipStream_t s);

// ---- TernGrad ------------------------------------------------------------------
size_t terngrad_workspace(int64_t n, int nseg);
hipError_t launch_terngrad(const float* x, float* res, int nseg, const int64_t* seg_offsets_host,
                           uint64_t seed, int64_t index_base, uint8_t* packed, float* scales,
                           void* ws, hipStream_t s);

// ---- EF Top-K / Random-K, direct or deferred residual, optional norm monitor -------
struct EfArgs {
  const float* grad;
  float* res;
  int64_t n, k, index_base;
  bool randk;
  uint64_t select_seed;
  int64_t* out_idx;
  float* out_val;
  int qsgd_levels;
  int64_t qsgd_group;
  uint64_t qsgd_seed;
  int8_t* out_codes;
  float* out_norms;
  void* ws;
  void* pending;          // null: the kept set's residual is written by the call
  size_t pending_bytes;
  double* stats;          // null: no norm monitor
};
size_t ef_topk_workspace(int64_t n, int64_t k, int qsgd_levels);
size_t ef_randk_workspace(int64_t n, int64_t k, int qsgd_levels);
size_t ef_pending_bytes(int64_t n, int64_t kmax);
unsigned long long ef_pending_capacity(int64_t n, size_t bytes);
hipError_t launch_ef(const EfArgs& a, hipStream_t s);
hipError_t launch_ef_flush(float* res, int64_t n, void* pend, size_t pend_bytes, hipStream_t s);

// ---- PowerSGD ------------------------------------------------------------------
size_t powersgd_workspace(int64_t rows, int64_t cols, int rank);
hipError_t launch_powersgd(const float* grad, float* res, int64_t rows, int64_t cols, int rank,
                           float* Q, float* P, void* ws, hipStream_t s);

// ---- decompress ----------------------------------------------------------------
hipError_t launch_decompress(int kind, const int64_t* idx, int64_t count, int64_t index_base,
                             const void* codes, const float* meta0, const float* meta1,
                             int64_t group, int levels, float alpha, int accumulate, float* out,
                             int64_t n_out, hipStream_t s);
// out[0..count) = (accumulate ? out : 0) + sum_w alpha * decode(payload w), W dense payloads
// of one kind and shape, summed in payload order (16 payloads per launch).
hipError_t launch_decode_sum(int kind, int W, const void* const* codes, const float* const* meta0,
                             const float* const* meta1, int64_t count, int64_t group, int levels,
                             float alpha, int accumulate, float* out, hipStream_t s);
hipError_t launch_fill_zero(float* p, int64_t n, hipStream_t s);
// out[0..n_out) = (accumulate ? out : 0) + sum_w alpha * g_hat_w for W sparse payloads with
// strictly ascending idx, merged tile by tile in payload order (16 payloads per launch).
hipError_t launch_merge_sparse(int W, const int64_t* const* idx, const void* const* codes,
                               const float* const* meta0, const float* const* meta1, const int64_t* count,
                               const int64_t* index_base, const int64_t* group, const int* kind,
                               const int* levels, float alpha, int accumulate, float* out, int64_t n_out,
                               hipStream_t s);

// Every argument check of gc_ef_compress except the workspace's (a rejected call makes no
// HIP call); *need receives the workspace bytes the call needs.
int ef_compress_check(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                      int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group, int8_t* out_codes,
                      float* out_norms, const ::gc_ef_options* opts, size_t* need);

// Sets the calling thread's gc_last_error text and returns `status` (for entry points
// defined outside capi.cpp).
int report(int status, const char* fmt, ...);

// Number of compute units of the current device (cached per device).
int device_cu_count();

// Stage timing of gc_ef_topk (see gc_profile_enable): stage 0 = call start, 1 = before the
// streaming pass, 2 = after it, 3 = call end.  No-op unless profiling is enabled.
void prof_mark(hipStream_t s, int stage);

}  // namespace gc
