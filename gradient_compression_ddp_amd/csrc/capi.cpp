// C ABI of libgc.so: argument validation, workspace sizing and dispatch to the gfx950
// launchers.  Every check runs on the host before anything is enqueued, so a rejected
// call touches no memory and makes no HIP call.  See include/gc.h for the contract.
#include "gc.h"

#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <array>
#include <mutex>
#include <vector>

#include "internal.hpp"

namespace {

thread_local char g_err[512] = "";

int fail(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int ok() {
  g_err[0] = '\0';
  return GC_OK;
}

int hip_status(hipError_t e, const char* what) {
  if (e == hipSuccess) return ok();
  return fail(GC_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool aligned(const void* p, size_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }
bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

constexpr int64_t kMaxN = int64_t(1) << 40;   // far beyond one GPU's HBM; keeps index math in 64 bits

#define GC_REQUIRE(cond, ...) \
  do {                        \
    if (!(cond)) return fail(GC_EINVAL, __VA_ARGS__); \
  } while (0)

int check_workspace(void* ws, size_t have, size_t need) {
  if (need == 0) return GC_OK;
  if (!ws) return fail(GC_EWORKSPACE, "workspace is NULL but %zu bytes are needed", need);
  if (!aligned(ws, 256)) return fail(GC_EINVAL, "workspace must be 256-byte aligned");
  if (have < need) return fail(GC_EWORKSPACE, "workspace has %zu bytes, needs %zu", have, need);
  return GC_OK;
}

}  // namespace

namespace gc {

int report(int status, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return status;
}

int device_cu_count() {
  static std::mutex mu;
  static int cache[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) dev = 0;
  std::lock_guard<std::mutex> lock(mu);
  if (cache[dev] == 0) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
      cus = 256;
    cache[dev] = cus;
  }
  return cache[dev];
}

// ---- stage timing -----------------------------------------------------------------
namespace {
struct ProfState {
  std::mutex mu;
  bool on = false;
  std::vector<hipEvent_t> free_events;
  std::vector<std::array<hipEvent_t, 4>> calls;   // completed sets, waiting for collection
  std::array<hipEvent_t, 4> open{};                // set being filled by the current call
  int filled = 0;
};
ProfState& prof() {
  static ProfState p;
  return p;
}
hipEvent_t take_event(ProfState& p) {
  if (!p.free_events.empty()) {
    hipEvent_t e = p.free_events.back();
    p.free_events.pop_back();
    return e;
  }
  hipEvent_t e = nullptr;
  if (hipEventCreate(&e) != hipSuccess) return nullptr;
  return e;
}
}  // namespace

void prof_mark(hipStream_t s, int stage) {
  ProfState& p = prof();
  std::lock_guard<std::mutex> lock(p.mu);
  if (!p.on) return;
  hipEvent_t e = take_event(p);
  if (!e) return;
  (void)hipEventRecord(e, s);
  p.open[stage] = e;
  if (stage == 3) {
    p.calls.push_back(p.open);
    p.open = {};
  }
}

}  // namespace gc

static_assert(sizeof(gc_payload_header) == 128, "the wire header is 128 bytes");

namespace {

uint64_t round256(uint64_t b) { return (b + 255u) & ~uint64_t(255); }

int64_t code_bytes(int kind, int64_t count) {
  switch (kind) {
    case GC_KIND_F32: return 4 * count;
    case GC_KIND_MINMAX8: return count;
    case GC_KIND_MINMAX4: return (count + 1) / 2;
    case GC_KIND_QSGD: return count;
    default: return (count + 3) / 4;   // GC_KIND_TERN
  }
}

int layout(int kind, int64_t n, int64_t count, int64_t group, int levels, int sparse, int64_t index_base,
           gc_payload_header* h) {
  GC_REQUIRE(kind >= GC_KIND_F32 && kind <= GC_KIND_TERN, "unknown payload kind %d", kind);
  GC_REQUIRE(n >= 0 && n <= kMaxN && count >= 0 && count <= n, "need 0 <= count <= n <= 2^40");
  GC_REQUIRE(group >= 0, "group must be >= 0");
  GC_REQUIRE(kind != GC_KIND_QSGD || (levels >= 1 && levels <= 127), "QSGD levels must lie in [1, 127]");
  GC_REQUIRE(index_base >= 0, "index_base must be >= 0");
  std::memset(h, 0, sizeof(*h));
  h->magic = GC_PAYLOAD_MAGIC;
  h->version = GC_PAYLOAD_VERSION;
  h->kind = (uint16_t)kind;
  h->flags = sparse ? GC_PAYLOAD_SPARSE : 0u;
  h->levels = kind == GC_KIND_QSGD ? levels : 0;
  h->n = n;
  h->count = count;
  h->index_base = index_base;
  h->group = group;
  const int64_t G = group == 0 ? (count > 0 ? count : 1) : group;
  const int64_t ng = count == 0 ? 0 : (count + G - 1) / G;
  uint64_t off = 256;   // the header, padded
  if (sparse) { h->off_idx = off; off = round256(off + 8u * (uint64_t)count); }
  h->off_codes = off;
  off = round256(off + (uint64_t)code_bytes(kind, count));
  if (kind != GC_KIND_F32) { h->off_meta0 = off; off = round256(off + 4u * (uint64_t)ng); }
  if (kind == GC_KIND_MINMAX8 || kind == GC_KIND_MINMAX4) { h->off_meta1 = off; off = round256(off + 4u * (uint64_t)ng); }
  h->bytes = off;
  return GC_OK;
}

}  // namespace

extern "C" {

int gc_payload_layout(int kind, int64_t n, int64_t count, int64_t group, int levels, int sparse,
                      int64_t index_base, gc_payload_header* hdr) {
  GC_REQUIRE(hdr != nullptr, "hdr must be non-NULL");
  const int st = layout(kind, n, count, group, levels, sparse, index_base, hdr);
  return st == GC_OK ? ok() : st;
}

int gc_decompress_payloads(int W, const void* const* payloads, const gc_payload_header* headers,
                           float alpha, int accumulate, float* out, int64_t n_out, void* stream) {
  GC_REQUIRE(W >= 1 && W <= 1024, "W must lie in [1, 1024]");
  GC_REQUIRE(payloads && headers, "payloads and headers (host arrays) must be non-NULL");
  GC_REQUIRE(n_out >= 0 && n_out <= kMaxN, "n_out out of range");
  GC_REQUIRE(out != nullptr && aligned(out, 4), "out must be non-NULL and 4-byte aligned");
  // every header must be exactly what gc_payload_layout gives for its own fields
  for (int w = 0; w < W; ++w) {
    const gc_payload_header& h = headers[w];
    GC_REQUIRE(h.magic == GC_PAYLOAD_MAGIC && h.version == GC_PAYLOAD_VERSION, "payload %d: bad magic or version", w);
    GC_REQUIRE((h.flags & ~GC_PAYLOAD_SPARSE) == 0u, "payload %d: unknown flags", w);
    gc_payload_header want;
    const int st = layout(h.kind, h.n, h.count, h.group, h.levels, (h.flags & GC_PAYLOAD_SPARSE) != 0u,
                          h.index_base, &want);
    if (st != GC_OK) return st;
    GC_REQUIRE(want.off_idx == h.off_idx && want.off_codes == h.off_codes && want.off_meta0 == h.off_meta0 &&
                   want.off_meta1 == h.off_meta1 && want.bytes == h.bytes,
               "payload %d: section offsets do not match the layout", w);
    GC_REQUIRE(h.n <= n_out, "payload %d encodes %lld elements, out has %lld", w, (long long)h.n, (long long)n_out);
    GC_REQUIRE(payloads[w] != nullptr && aligned(payloads[w], 256), "payload %d must be non-NULL and 256-byte aligned", w);
  }
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  const auto at = [&](int w, uint64_t off) -> const char* {
    return off ? reinterpret_cast<const char*>(payloads[w]) + off : nullptr;
  };
  bool fused = aligned(out, 16);
  for (int w = 0; w < W && fused; ++w) {
    const gc_payload_header& h = headers[w];
    fused = !(h.flags & GC_PAYLOAD_SPARSE) && h.kind == headers[0].kind && h.count == headers[0].count &&
            h.group == headers[0].group && h.levels == headers[0].levels;
  }
  if (fused) {
    std::vector<const void*> codes(W);
    std::vector<const float*> m0(W), m1(W);
    for (int w = 0; w < W; ++w) {
      codes[w] = at(w, headers[w].off_codes);
      m0[w] = reinterpret_cast<const float*>(at(w, headers[w].off_meta0));
      m1[w] = reinterpret_cast<const float*>(at(w, headers[w].off_meta1));
    }
    return hip_status(gc::launch_decode_sum(headers[0].kind, W, codes.data(), m0.data(), m1.data(),
                                            headers[0].count, headers[0].group, headers[0].levels, alpha,
                                            accumulate, out, s),
                      "gc_decompress_payloads launch");
  }
  bool sparse = true;
  for (int w = 0; w < W && sparse; ++w) sparse = (headers[w].flags & GC_PAYLOAD_SPARSE) != 0u;
  if (sparse) {
    // every payload sparse: merged tile by tile, out written once
    std::vector<const int64_t*> ix(W);
    std::vector<const void*> codes(W);
    std::vector<const float*> m0(W), m1(W);
    std::vector<int64_t> count(W), base(W), group(W);
    std::vector<int> kind(W), levels(W);
    for (int w = 0; w < W; ++w) {
      const gc_payload_header& h = headers[w];
      ix[w] = reinterpret_cast<const int64_t*>(at(w, h.off_idx));
      codes[w] = at(w, h.off_codes);
      m0[w] = reinterpret_cast<const float*>(at(w, h.off_meta0));
      m1[w] = reinterpret_cast<const float*>(at(w, h.off_meta1));
      count[w] = h.count;
      base[w] = h.index_base;
      group[w] = h.group;
      kind[w] = h.kind;
      levels[w] = h.levels;
    }
    return hip_status(gc::launch_merge_sparse(W, ix.data(), codes.data(), m0.data(), m1.data(), count.data(),
                                              base.data(), group.data(), kind.data(), levels.data(), alpha,
                                              accumulate, out, n_out, s),
                      "gc_decompress_payloads launch");
  }
  if (!accumulate) {
    const hipError_t e = gc::launch_fill_zero(out, n_out, s);
    if (e != hipSuccess) return hip_status(e, "gc_decompress_payloads launch");
  }
  for (int w = 0; w < W; ++w) {
    const gc_payload_header& h = headers[w];
    const hipError_t e = gc::launch_decompress(
        h.kind, reinterpret_cast<const int64_t*>(at(w, h.off_idx)), h.count, h.index_base, at(w, h.off_codes),
        reinterpret_cast<const float*>(at(w, h.off_meta0)), reinterpret_cast<const float*>(at(w, h.off_meta1)),
        h.group, h.levels, alpha, 1, out, n_out, s);
    if (e != hipSuccess) return hip_status(e, "gc_decompress_payloads launch");
  }
  return ok();
}

int gc_profile_enable(int on) {
  gc::ProfState& p = gc::prof();
  std::lock_guard<std::mutex> lock(p.mu);
  p.on = on != 0;
  return ok();
}

int gc_profile_collect(int64_t* calls, double* ms_before, double* ms_pass, double* ms_after) {
  GC_REQUIRE(calls && ms_before && ms_pass && ms_after, "output pointers must be non-NULL");
  gc::ProfState& p = gc::prof();
  std::lock_guard<std::mutex> lock(p.mu);
  double acc[3] = {0.0, 0.0, 0.0};
  for (auto& set : p.calls) {
    for (int i = 0; i < 4; ++i)
      if (hipEventSynchronize(set[i]) != hipSuccess) return fail(GC_EHIP, "hipEventSynchronize failed");
    for (int i = 0; i < 3; ++i) {
      float ms = 0.f;
      if (hipEventElapsedTime(&ms, set[i], set[i + 1]) != hipSuccess)
        return fail(GC_EHIP, "hipEventElapsedTime failed");
      acc[i] += ms;
    }
    for (int i = 0; i < 4; ++i) p.free_events.push_back(set[i]);
  }
  *calls = (int64_t)p.calls.size();
  *ms_before = acc[0];
  *ms_pass = acc[1];
  *ms_after = acc[2];
  p.calls.clear();
  return ok();
}


const char* gc_status_string(int status) {
  switch (status) {
    case GC_OK: return "GC_OK";
    case GC_EINVAL: return "GC_EINVAL: invalid argument";
    case GC_EWORKSPACE: return "GC_EWORKSPACE: workspace missing or too small";
    case GC_EUNSUPPORTED: return "GC_EUNSUPPORTED: not implemented";
    case GC_EHIP: return "GC_EHIP: HIP runtime error";
    default: return "unknown gc status";
  }
}

const char* gc_last_error(void) { return g_err; }

int gc_version(void) { return 100; }

int gc_workspace_size(int op, int64_t n, int64_t k, int64_t aux, size_t* bytes) {
  GC_REQUIRE(bytes != nullptr, "bytes is NULL");
  *bytes = 0;
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n out of range");
  switch (op) {
    case GC_OP_EF_TOPK:
      GC_REQUIRE(k >= 0 && k <= n, "k must lie in [0, n]");
      GC_REQUIRE(aux >= 0 && aux <= 127, "qsgd levels must lie in [0, 127]");
      *bytes = (n == 0 || k == 0) ? 0 : gc::ef_topk_workspace(n, k, (int)aux);
      return ok();
    case GC_OP_EF_RANDK:
      GC_REQUIRE(k >= 0 && k <= n, "k must lie in [0, n]");
      GC_REQUIRE(aux >= 0 && aux <= 127, "qsgd levels must lie in [0, 127]");
      *bytes = (n == 0 || k == 0) ? 0 : gc::ef_randk_workspace(n, k, (int)aux);
      return ok();
    case GC_OP_EF_PENDING:
      GC_REQUIRE(k >= 0 && k <= n, "k must lie in [0, n]");
      *bytes = n == 0 ? 0 : gc::ef_pending_bytes(n, k);
      return ok();
    case GC_OP_QUANT_MINMAX:
      GC_REQUIRE(k == 0 || k >= 4, "group must be 0 or >= 4");
      *bytes = (k == 0 || k > 256) ? gc::minmax_large_workspace(n, k) : 0;
      return ok();
    case GC_OP_QSGD:
    case GC_OP_DECOMPRESS:
      return ok();
    case GC_OP_TERNGRAD:
      GC_REQUIRE(k >= 0 && k <= (int64_t(1) << 30), "nseg out of range");
      *bytes = gc::terngrad_workspace(n, (int)k);
      return ok();
    case GC_OP_POWERSGD:
      GC_REQUIRE(n >= 1 && k >= 1 && aux >= 1 && aux <= 4, "rows, cols >= 1 and rank in [1,4]");
      *bytes = gc::powersgd_workspace(n, k, (int)aux);
      return ok();
    default:
      return fail(GC_EINVAL, "unknown op %d", op);
  }
}

// Argument checks shared by the two sparsifiers (everything but the workspace).
static int check_sparsify(const float* grad, float* residual, int64_t n, int64_t k,
                          int64_t index_base, int64_t* out_idx, float* out_val, int qsgd_levels,
                          int64_t qsgd_group, int8_t* out_codes, float* out_norms) {
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n must lie in [0, 2^40]");
  GC_REQUIRE(k >= 0 && k <= n, "k must lie in [0, n]");
  GC_REQUIRE(index_base >= 0 && index_base <= (int64_t(1) << 62) - n, "index_base out of range");
  GC_REQUIRE(qsgd_levels >= 0 && qsgd_levels <= 127, "qsgd_levels must lie in [0, 127]");
  if (n == 0) return ok();
  GC_REQUIRE(grad && residual, "grad and residual must be non-NULL");
  GC_REQUIRE(aligned(grad, 16) && aligned(residual, 16), "grad and residual must be 16-byte aligned");
  if (k > 0) {
    GC_REQUIRE(out_idx && aligned(out_idx, 8), "out_idx must be non-NULL and 8-byte aligned");
    if (qsgd_levels == 0) {
      GC_REQUIRE(out_val && aligned(out_val, 4), "out_val must be non-NULL and 4-byte aligned");
    } else {
      GC_REQUIRE(pow2(qsgd_group) && qsgd_group >= 4 && qsgd_group <= 256,
                 "qsgd_group must be a power of two in [4, 256]");
      GC_REQUIRE(out_codes && aligned(out_codes, 4), "out_codes must be non-NULL and 4-byte aligned");
      GC_REQUIRE(out_norms && aligned(out_norms, 4), "out_norms must be non-NULL");
      GC_REQUIRE(!out_val || aligned(out_val, 16), "out_val must be 16-byte aligned when given");
    }
  }
  return ok();
}

static_assert(sizeof(gc_ef_options) == 40, "gc_ef_options layout");

}  // extern "C"

namespace gc {

// Every check of gc_ef_compress except the workspace's; *need receives the workspace
// bytes the call needs (0 when it touches none).
int ef_compress_check(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                      int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group, int8_t* out_codes,
                      float* out_norms, const gc_ef_options* opts, size_t* need) {
  *need = 0;
  gc_ef_options o{};
  if (opts) {
    GC_REQUIRE(opts->size >= sizeof(gc_ef_options), "opts->size must be sizeof(gc_ef_options)");
    o = *opts;
  }
  GC_REQUIRE(o.select == GC_SELECT_TOPK || o.select == GC_SELECT_RANDK, "opts->select must be TOPK or RANDK");
  const int c = check_sparsify(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels,
                               qsgd_group, out_codes, out_norms);
  if (c != GC_OK || n == 0) return c;
  GC_REQUIRE(!o.stats || k > 0, "the norm monitor needs k > 0");
  GC_REQUIRE(!o.stats || aligned(o.stats, 8), "opts->stats must be 8-byte aligned");
  if (o.pending) {
    GC_REQUIRE(aligned(o.pending, 256), "opts->pending must be 256-byte aligned");
    if (o.pending_bytes < gc::ef_pending_bytes(n, k))
      return fail(GC_EWORKSPACE, "pending record of %zu bytes is smaller than the %zu this n and k need",
                  o.pending_bytes, gc::ef_pending_bytes(n, k));
  }
  if (k > 0)
    *need = o.select == GC_SELECT_RANDK ? gc::ef_randk_workspace(n, k, qsgd_levels)
                                        : gc::ef_topk_workspace(n, k, qsgd_levels);
  return ok();
}

}  // namespace gc

extern "C" {

int gc_ef_compress(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                   int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
                   int8_t* out_codes, float* out_norms, const gc_ef_options* opts, void* workspace,
                   size_t workspace_bytes, void* stream) {
  size_t need = 0;
  const int c = gc::ef_compress_check(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group,
                                      out_codes, out_norms, opts, &need);
  if (c != GC_OK || n == 0) return c;
  gc_ef_options o{};
  if (opts) o = *opts;
  const bool randk = o.select == GC_SELECT_RANDK;
  if (k > 0) {
    const int w = check_workspace(workspace, workspace_bytes, need);
    if (w != GC_OK) return w;
  }
  gc::EfArgs a{};
  a.grad = grad; a.res = residual; a.n = n; a.k = k; a.index_base = index_base;
  a.randk = randk; a.select_seed = o.select_seed;
  a.out_idx = out_idx; a.out_val = out_val;
  a.qsgd_levels = qsgd_levels; a.qsgd_group = qsgd_group; a.qsgd_seed = qsgd_seed;
  a.out_codes = out_codes; a.out_norms = out_norms;
  a.ws = workspace; a.pending = o.pending; a.pending_bytes = o.pending_bytes; a.stats = o.stats;
  return hip_status(gc::launch_ef(a, reinterpret_cast<hipStream_t>(stream)), "gc_ef_compress launch");
}

int gc_ef_topk(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
               int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group,
               uint64_t qsgd_seed, int8_t* out_codes, float* out_norms, void* workspace,
               size_t workspace_bytes, void* stream) {
  return gc_ef_compress(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group, qsgd_seed,
                        out_codes, out_norms, nullptr, workspace, workspace_bytes, stream);
}

int gc_ef_topk_deferred(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                        int64_t* out_idx, float* out_val, int qsgd_levels, int64_t qsgd_group,
                        uint64_t qsgd_seed, int8_t* out_codes, float* out_norms, void* pending,
                        size_t pending_bytes, void* workspace, size_t workspace_bytes, void* stream) {
  GC_REQUIRE(n == 0 || pending, "pending must be non-NULL");
  gc_ef_options o{};
  o.size = sizeof(o);
  o.pending = pending;
  o.pending_bytes = pending_bytes;
  return gc_ef_compress(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group, qsgd_seed,
                        out_codes, out_norms, &o, workspace, workspace_bytes, stream);
}

int gc_ef_randk(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                uint64_t select_seed, int64_t* out_idx, float* out_val, int qsgd_levels,
                int64_t qsgd_group, uint64_t qsgd_seed, int8_t* out_codes, float* out_norms,
                void* workspace, size_t workspace_bytes, void* stream) {
  gc_ef_options o{};
  o.size = sizeof(o);
  o.select = GC_SELECT_RANDK;
  o.select_seed = select_seed;
  return gc_ef_compress(grad, residual, n, k, index_base, out_idx, out_val, qsgd_levels, qsgd_group, qsgd_seed,
                        out_codes, out_norms, &o, workspace, workspace_bytes, stream);
}

int gc_ef_flush(float* residual, int64_t n, void* pending, size_t pending_bytes, void* stream) {
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n must lie in [0, 2^40]");
  if (n == 0) return ok();
  GC_REQUIRE(residual && aligned(residual, 16), "residual must be non-NULL and 16-byte aligned");
  GC_REQUIRE(pending && aligned(pending, 256), "pending must be non-NULL and 256-byte aligned");
  if (pending_bytes < gc::ef_pending_bytes(n, 0))
    return fail(GC_EWORKSPACE, "pending record of %zu bytes is too small for n", pending_bytes);
  return hip_status(gc::launch_ef_flush(residual, n, pending, pending_bytes, reinterpret_cast<hipStream_t>(stream)),
                    "gc_ef_flush launch");
}

int gc_quant_minmax(const float* x, float* residual, int64_t n, int64_t group, int bits,
                    uint8_t* codes, float* mins, float* scales, void* workspace,
                    size_t workspace_bytes, void* stream) {
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n must lie in [0, 2^40]");
  GC_REQUIRE(bits == 8 || bits == 4, "bits must be 8 or 4");
  GC_REQUIRE(group == 0 || group >= 4, "group must be 0 or >= 4");
  GC_REQUIRE(group == 0 || group > 256 || pow2(group), "a group of at most 256 must be a power of two");
  if (n == 0) return ok();
  GC_REQUIRE(x && aligned(x, 16), "x must be non-NULL and 16-byte aligned");
  GC_REQUIRE(!residual || aligned(residual, 16), "residual must be 16-byte aligned");
  GC_REQUIRE(codes && aligned(codes, bits == 8 ? 4 : 2), "codes must be non-NULL and aligned");
  GC_REQUIRE(mins && scales && aligned(mins, 4) && aligned(scales, 4), "mins and scales must be non-NULL");
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (group != 0 && group <= 256)
    return hip_status(gc::launch_minmax_small(x, residual, n, group, bits, codes, mins, scales, s),
                      "gc_quant_minmax launch");
  const size_t need = gc::minmax_large_workspace(n, group);
  const int w = check_workspace(workspace, workspace_bytes, need);
  if (w != GC_OK) return w;
  return hip_status(gc::launch_minmax_large(x, residual, n, group, bits, codes, mins, scales, workspace, s),
                    "gc_quant_minmax launch");
}

int gc_qsgd(const float* x, float* residual, int64_t n, int64_t group, int levels, uint64_t seed,
            int64_t index_base, int8_t* codes, float* norms, void* stream) {
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n must lie in [0, 2^40]");
  GC_REQUIRE(pow2(group) && group >= 4 && group <= 256, "group must be a power of two in [4, 256]");
  GC_REQUIRE(levels >= 1 && levels <= 127, "levels must lie in [1, 127]");
  GC_REQUIRE(index_base >= 0 && index_base <= (int64_t(1) << 62) - n, "index_base out of range");
  if (n == 0) return ok();
  GC_REQUIRE(x && aligned(x, 16), "x must be non-NULL and 16-byte aligned");
  GC_REQUIRE(!residual || aligned(residual, 16), "residual must be 16-byte aligned");
  GC_REQUIRE(codes && aligned(codes, 4), "codes must be non-NULL and 4-byte aligned");
  GC_REQUIRE(norms && aligned(norms, 4), "norms must be non-NULL");
  return hip_status(gc::launch_qsgd(x, residual, n, group, levels, seed, index_base, codes, norms,
                                    reinterpret_cast<hipStream_t>(stream)),
                    "gc_qsgd launch");
}

int gc_stream_floor(const float* x, uint8_t* out, int64_t n, void* stream) {
  GC_REQUIRE(n >= 0 && n <= kMaxN, "n must lie in [0, 2^40]");
  if (n == 0) return ok();
  GC_REQUIRE(x && aligned(x, 16), "x must be non-NULL and 16-byte aligned");
  GC_REQUIRE(out && aligned(out, 4), "out must be non-NULL and 4-byte aligned");
  return hip_status(gc::launch_stream_floor(x, out, n, reinterpret_cast<hipStream_t>(stream)),
                    "gc_stream_floor launch");
}

int gc_terngrad(const float* x, float* residual, int nseg, const int64_t* seg_offsets, uint64_t seed,
                int64_t index_base, uint8_t* packed, float* scales, void* workspace,
                size_t workspace_bytes, void* stream) {
  GC_REQUIRE(nseg >= 0, "nseg must be >= 0");
  if (nseg == 0) return ok();
  GC_REQUIRE(seg_offsets != nullptr, "seg_offsets (host) must be non-NULL");
  GC_REQUIRE(seg_offsets[0] == 0, "seg_offsets[0] must be 0");
  for (int i = 0; i < nseg; ++i)
    GC_REQUIRE(seg_offsets[i + 1] >= seg_offsets[i], "seg_offsets must be nondecreasing");
  const int64_t n = seg_offsets[nseg];
  GC_REQUIRE(n <= kMaxN, "n must lie in [0, 2^40]");
  GC_REQUIRE(index_base >= 0 && index_base <= (int64_t(1) << 62) - n, "index_base out of range");
  GC_REQUIRE(scales && aligned(scales, 4), "scales must be non-NULL");
  if (n > 0) {
    GC_REQUIRE(x && aligned(x, 16), "x must be non-NULL and 16-byte aligned");
    GC_REQUIRE(!residual || aligned(residual, 16), "residual must be 16-byte aligned");
    GC_REQUIRE(packed != nullptr, "packed must be non-NULL");
  }
  const size_t need = gc::terngrad_workspace(n, nseg);
  const int w = check_workspace(workspace, workspace_bytes, need);
  if (w != GC_OK) return w;
  return hip_status(gc::launch_terngrad(x, residual, nseg, seg_offsets, seed, index_base, packed, scales,
                                        workspace, reinterpret_cast<hipStream_t>(stream)),
                    "gc_terngrad launch");
}

int gc_powersgd_step(const float* grad, float* residual, int64_t rows, int64_t cols, int rank,
                     float* Q, float* P, void* workspace, size_t workspace_bytes, void* stream) {
  GC_REQUIRE(rows >= 1 && cols >= 1 && rows <= kMaxN && cols <= kMaxN && rows * cols <= kMaxN && rank <= cols,
             "rows and cols must be >= 1 with rows*cols <= 2^40");
  GC_REQUIRE(cols % 4 == 0, "cols must be a multiple of 4");
  GC_REQUIRE(rank >= 1 && rank <= 4, "rank must lie in [1, 4]");
  GC_REQUIRE(grad && aligned(grad, 16), "grad must be non-NULL and 16-byte aligned");
  GC_REQUIRE(!residual || aligned(residual, 16), "residual must be 16-byte aligned");
  GC_REQUIRE(Q && P && aligned(Q, 4) && aligned(P, 4), "Q and P must be non-NULL");
  const size_t need = gc::powersgd_workspace(rows, cols, rank);
  const int w = check_workspace(workspace, workspace_bytes, need);
  if (w != GC_OK) return w;
  const hipError_t e = gc::launch_powersgd(grad, residual, rows, cols, rank, Q, P, workspace,
                                           reinterpret_cast<hipStream_t>(stream));
  if (e == hipErrorNotSupported) return fail(GC_EUNSUPPORTED, "gc_powersgd_step is not built yet");
  return hip_status(e, "gc_powersgd_step launch");
}

int gc_decompress_scatter(int kind, const int64_t* idx, int64_t count, int64_t index_base,
                          const void* codes, const float* meta0, const float* meta1, int64_t group,
                          int levels, float alpha, int accumulate, float* out, int64_t n_out,
                          void* stream) {
  GC_REQUIRE(kind >= GC_KIND_F32 && kind <= GC_KIND_TERN, "unknown payload kind %d", kind);
  GC_REQUIRE(count >= 0 && count <= kMaxN && n_out >= 0 && n_out <= kMaxN, "count/n_out out of range");
  GC_REQUIRE(group >= 0, "group must be >= 0");
  GC_REQUIRE(index_base >= 0, "index_base must be >= 0");
  if (count == 0) return ok();
  GC_REQUIRE(codes != nullptr && out != nullptr, "codes and out must be non-NULL");
  GC_REQUIRE(aligned(out, 4) && (kind != GC_KIND_F32 || aligned(codes, 4)), "misaligned pointer");
  GC_REQUIRE(!idx || aligned(idx, 8), "idx must be 8-byte aligned");
  if (!idx) GC_REQUIRE(count <= n_out, "a dense decode needs count <= n_out");
  if (kind == GC_KIND_MINMAX8 || kind == GC_KIND_MINMAX4)
    GC_REQUIRE(meta0 && meta1, "min-max payloads need meta0 (mins) and meta1 (scales)");
  if (kind == GC_KIND_QSGD) {
    GC_REQUIRE(meta0 != nullptr, "QSGD payloads need meta0 (norms)");
    GC_REQUIRE(levels >= 1 && levels <= 127, "levels must lie in [1, 127]");
  }
  if (kind == GC_KIND_TERN) GC_REQUIRE(meta0 != nullptr, "TernGrad payloads need meta0 (scales)");
  return hip_status(gc::launch_decompress(kind, idx, count, index_base, codes, meta0, meta1, group, levels,
                                          alpha, accumulate, out, n_out,
                                          reinterpret_cast<hipStream_t>(stream)),
                    "gc_decompress_scatter launch");
}

}  // extern "C"
