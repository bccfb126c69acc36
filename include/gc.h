/*
 * gc.h -- C ABI of the MI355X (gfx950) gradient-compression library (libgc.so).
 *
 * The library compresses one GPU's flat fp32 gradient bucket in HBM before it is sent
 * anywhere: error-feedback Top-K and Random-K, min-max int8/int4, QSGD, TernGrad, PowerSGD,
 * and the matching decompression.
 *
 * Conventions for every call
 *   - Data pointers are DEVICE pointers (HBM) unless a comment says "host".
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream.  Every call
 *     only enqueues work on `stream` and returns; nothing is synchronized, nothing is
 *     read back to the host, and no memory is allocated or freed by the library.
 *   - The caller owns every buffer.  Scratch memory is passed in as `workspace` of
 *     `workspace_bytes` bytes; gc_workspace_size() says how much a call needs.
 *     A workspace may be reused by consecutive calls on one stream, not by calls that
 *     can run concurrently.
 *   - Outputs must not alias inputs, except the residual, which is updated in place.
 *   - Sizes and indices are 64-bit.  fp32 arrays read with vector loads (grad, residual,
 *     x) must be 16-byte aligned; torch allocations are.
 *   - Arguments are checked on the host before anything is enqueued.  A failing check
 *     returns GC_EINVAL / GC_EWORKSPACE / GC_EUNSUPPORTED and touches no memory; the
 *     reason is available from gc_last_error() in the calling thread.  A failed launch
 *     returns GC_EHIP.
 *   - Floating point is IEEE binary32 with round-to-nearest-even, correctly rounded
 *     division and square root, no fused multiply-add and no flush of denormals, so the
 *     results are bit-reproducible and match a plain CPU implementation.  Non-finite
 *     inputs produce unspecified (but finite-time, in-bounds) results, except in Top-K,
 *     where NaN and Inf are ordered by their bit pattern.
 *
 * Random draws (QSGD, TernGrad, Random-K) use Philox4x32-10 (Salmon et al., "Parallel Random
 * Numbers: As Easy as 1, 2, 3", SC'11): element e takes word (e & 3) of the block at
 * counter (e >> 2, 0) under key (seed_lo, seed_hi), and U = (word >> 8) * 2^-24.
 * Rounding goes up when U < p.  The draw depends only on (seed, e), never on the
 * launch configuration.
 *
 * Sources of the operations (web pages on gradient compression):
 *   [P1] blog.hotdry.top, "gradient-compression-quantization-sparsification"
 *   [P2] zyxy.net/archives/25733, "分布式训练中的梯度压缩算法：性能瓶颈、收敛性影响与实现细节"
 *   [P3] 5688vip.com, "4、梯度累积与梯度压缩" (multi-GPU sync efficiency series, part 04)
 *   [P4] aiqz.cc, "梯度聚合通信优化实战方案"
 */
#ifndef GC_H
#define GC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum gc_status {
  GC_OK = 0,
  GC_EINVAL = 1,        /* bad argument: null pointer, size, k, bits, levels, group, alignment */
  GC_EWORKSPACE = 2,    /* workspace missing or smaller than gc_workspace_size() */
  GC_EUNSUPPORTED = 3,  /* valid request the library does not implement */
  GC_EHIP = 4           /* a HIP runtime call or kernel launch failed */
};

/* Operation selectors for gc_workspace_size(). */
enum gc_op {
  GC_OP_EF_TOPK = 1,       /* n = elements, k = kept, aux = QSGD levels (0: none)       */
  GC_OP_QUANT_MINMAX = 2,  /* n = elements, k = group (0: whole tensor), aux unused      */
  GC_OP_QSGD = 3,          /* needs no workspace                                         */
  GC_OP_TERNGRAD = 4,      /* n = total elements, k = number of segments                 */
  GC_OP_POWERSGD = 5,      /* n = rows, k = cols, aux = rank                             */
  GC_OP_DECOMPRESS = 6,    /* needs no workspace                                         */
  GC_OP_EF_RANDK = 7,      /* n = elements, k = kept, aux = QSGD levels (0: none)       */
  GC_OP_EF_PENDING = 8     /* size of a pending record: n = elements, k = largest k     */
};

/* Payload kinds for gc_decompress_scatter(). */
enum gc_kind {
  GC_KIND_F32 = 0,      /* codes: float[count] values                                   */
  GC_KIND_MINMAX8 = 1,  /* codes: uint8[count]; meta0 = mins, meta1 = scales per group   */
  GC_KIND_MINMAX4 = 2,  /* codes: uint8[ceil(count/2)], entry 2j in the low nibble       */
  GC_KIND_QSGD = 3,     /* codes: int8[count] = sign*level; meta0 = norms; `levels` = s   */
  GC_KIND_TERN = 4      /* codes: uint8[ceil(count/4)], 2 bits each; meta0 = scales      */
};

/* Static string for a status value. Host only, never fails. */
const char* gc_status_string(int status);

/* Reason for the last non-GC_OK return in the calling thread ("" if none). */
const char* gc_last_error(void);

/* Library version, major*10000 + minor*100 + patch. */
int gc_version(void);

/* Bytes of workspace the call selected by `op` needs for the given sizes (host only;
 * no device call).  Returns GC_EINVAL for impossible sizes. */
int gc_workspace_size(int op, int64_t n, int64_t k, int64_t aux, size_t* bytes);

/*
 * gc_ef_topk -- error-feedback Top-K sparsification, optionally followed by QSGD on
 * the kept values.
 *
 * Operation ([P1] section 2 and 2.1; [P3] section 4.2.1 topk_compress and its error
 * accumulation; [P4] "Python 演示" error_feedback_compress; hybrid with 8-bit
 * quantization of what is sent: [P3] section 4.3):
 *   c      = fl(grad + residual)                                  (every element)
 *   key(c) = bit pattern of c with the sign bit cleared (31-bit unsigned magnitude)
 *   S      = the k elements with the largest key; among equal keys the lower index wins
 *   out_idx[j] = index_base + (j-th smallest index in S)          (strictly ascending)
 *   pure Top-K (qsgd_levels == 0):
 *       out_val[j]      = c[idx_j]            (bit-exact copy)
 *       residual[idx_j] = +0.0,  residual[i] = c[i] elsewhere
 *   with QSGD (qsgd_levels in [1,127]), applied to v = (c[idx_0], ..., c[idx_{k-1}]):
 *       groups of qsgd_group consecutive kept values (power of two in [4,256]);
 *       out_norms[g] = fl(sqrt(pairwise-tree sum of v^2 over group g)), float[ceil(k/group)];
 *       out_codes[j] = sign(v_j) * level_j (int8), level from stochastic rounding of
 *           fl(fl(|v_j|/nu)*s) with the Philox draw of element index j under qsgd_seed;
 *       residual[idx_j] = fl(v_j - g_hat_j), g_hat_j = sign * fl(fl(nu*level)/s);
 *       out_val may be NULL; if given it receives v.
 *
 * grad: const float[n], 16-byte aligned.  residual: float[n], 16-byte aligned, in: the
 * previous residual (zeros on the first step), out: the new residual.  out_idx: int64[k].
 * k == 0 performs only residual = c.  n == 0 is a no-op.  Requires 0 <= k <= n.
 * Workspace: gc_workspace_size(GC_OP_EF_TOPK, n, k, qsgd_levels).
 * The selection is exact for every input: an internal fast path keeps a candidate set
 * above a sampled threshold, and falls back to a full exact selection on the device if
 * the candidate set cannot contain the answer.
 */
int gc_ef_topk(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
               int64_t* out_idx, float* out_val,
               int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
               int8_t* out_codes, float* out_norms,
               void* workspace, size_t workspace_bytes, void* stream);

/* Selectors of gc_ef_options.select. */
enum gc_select {
  GC_SELECT_TOPK = 0,   /* the k largest magnitudes (gc_ef_topk)        */
  GC_SELECT_RANDK = 1   /* the k largest Philox index keys (gc_ef_randk) */
};

/* Options of gc_ef_compress (a HOST struct; zero-fill it, then set `size`). */
typedef struct gc_ef_options {
  uint32_t size;          /* sizeof(gc_ef_options)                                       */
  uint32_t select;        /* GC_SELECT_TOPK or GC_SELECT_RANDK                           */
  uint64_t select_seed;   /* Random-K key seed (see gc_ef_randk)                         */
  void* pending;          /* NULL: the kept set's residual is written by the call; else a
                             pending record as in gc_ef_topk_deferred                      */
  size_t pending_bytes;
  double* stats;          /* NULL, or DEVICE double[3] receiving the norm monitor        */
} gc_ef_options;

/*
 * gc_ef_compress -- one error-feedback sparsification step with every option: Top-K or
 * Random-K selection, the kept set's residual written by the call or deferred to the
 * next one, and the gradient-norm-ratio monitor.  gc_ef_topk, gc_ef_topk_deferred and
 * gc_ef_randk are this call with the matching options.  opts == NULL selects Top-K,
 * direct residual, no monitor.
 *
 * Norm monitor ([P1] section 3.2 item 2: watch the ratio of the gradient norm after
 * compression to the norm before it; a ratio that stays below 0.9 means the compression
 * is too strong).  With opts->stats set (k > 0 required), the call writes
 *   stats[0] = sum over all n of c^2           (c = fl(grad + residual), what is compressed)
 *   stats[1] = sum over the kept set of g_hat^2 (the decoded payload: the kept values, or
 *              their QSGD reconstruction fl(nu*level)/s with QSGD)
 *   stats[2] = sqrt(stats[1] / stats[0])        (1 when stats[0] == 0)
 * The squares are exact float64 products of the float32 values; the sums are float64 in
 * a fixed order (per 4096-element tile inside the streaming pass, per 1024 kept entries,
 * then two fixed-shape reduction levels), so the result is deterministic and within the
 * float64 rounding of the exact sums.  The monitor adds no pass over the gradient.
 *
 * Workspace: gc_workspace_size(GC_OP_EF_TOPK or GC_OP_EF_RANDK, n, k, qsgd_levels).
 * Everything else as gc_ef_topk.
 */
int gc_ef_compress(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                   int64_t* out_idx, float* out_val,
                   int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
                   int8_t* out_codes, float* out_norms, const gc_ef_options* opts,
                   void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_ef_compress_noalloc -- gc_ef_compress with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP stream capture, serving loops and
 * harnesses that must not call the allocator.
 *
 * Same operation, arguments (less workspace and workspace_bytes), outputs and errors as
 * gc_ef_compress.  Its workspace is a fixed array of gc_noalloc_scratch_bytes() bytes
 * (32 MiB) inside the library's code object, one copy per GPU, held until the process
 * ends.  The call allocates and frees nothing.  The first call on a device looks up that
 * device's copy (hipGetSymbolAddress, with the device current) and keeps its address.
 * Every call resets whatever part of the array must start at zero, so it does not depend
 * on what an earlier call left there.
 *
 * Limit: a call whose gc_workspace_size(GC_OP_EF_TOPK or GC_OP_EF_RANDK, n, k,
 * qsgd_levels) exceeds the array returns GC_EWORKSPACE before any HIP call.  At k = 1%
 * of n with QSGD that allows n up to about 1.5e8 (Top-K) or 1.0e8 (Random-K), so a
 * 25 MiB bucket (6,553,600 elements) fits at any k up to a quarter of it.  Calls that overlap
 * in time on one GPU (two streams or threads at once) share the array and race: the
 * caller serializes them, e.g. by issuing them on one stream.
 */
int gc_ef_compress_noalloc(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                           int64_t* out_idx, float* out_val,
                           int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
                           int8_t* out_codes, float* out_norms, const gc_ef_options* opts,
                           void* stream);

/* Size in bytes of gc_ef_compress_noalloc's fixed per-GPU array. */
size_t gc_noalloc_scratch_bytes(void);

/*
 * gc_ef_topk_deferred -- gc_ef_topk with the residual update of the kept set deferred to
 * the next call on the same residual.
 *
 * Same operation and outputs as gc_ef_topk ([P1] section 2.1: what is not sent is kept
 * and added to the next step's gradient).  The difference is only where the new
 * residual of the kept entries lives between calls: this call leaves c in `residual` at
 * every position and records, in the caller-owned `pending` record, each kept entry's
 * residual value (+0.0, or fl(v - g_hat) with QSGD).  The next gc_ef_topk_deferred or
 * gc_ef_flush on the same residual applies them: the next call does so inside its one
 * coalesced pass over the residual, which saves the scattered writes of the kept set.
 * Indices, values, codes and norms are bit-identical to gc_ef_topk's, and so is the
 * residual once flushed.
 *
 * pending: device memory, 256-byte aligned, of pending_bytes >=
 *   gc_workspace_size(GC_OP_EF_PENDING, n, k_max, 0) for the largest k it will see.  It
 *   must be zero-filled before its first use (empty) and belongs to one residual of n
 *   elements until it is flushed: calls with another residual or another n must not use
 *   it.  Between calls, the exact residual is `residual` patched by the record; call
 *   gc_ef_flush before reading the residual or using it with any other call.
 * k == 0 applies the record, performs residual = c and leaves the record empty.
 * Other arguments, the workspace and errors as gc_ef_topk; a too small record returns
 * GC_EWORKSPACE.
 */
int gc_ef_topk_deferred(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                        int64_t* out_idx, float* out_val,
                        int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
                        int8_t* out_codes, float* out_norms,
                        void* pending, size_t pending_bytes,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_ef_flush -- apply a pending record to its residual and empty the record.
 *
 * residual: float[n] of the gc_ef_topk_deferred calls that filled `pending`; afterwards
 * it equals the residual gc_ef_topk would have left.  An empty record (or one filled for
 * another n) changes nothing.  n == 0 is a no-op.
 */
int gc_ef_flush(float* residual, int64_t n, void* pending, size_t pending_bytes, void* stream);

/*
 * gc_ef_randk -- error-feedback Random-K sparsification, optionally followed by QSGD on
 * the kept values.
 *
 * Operation ([P1] section 2.2 Random-K, with the error feedback of section 2.1; [P2]
 * section 二.2 random sparsification).  The pages fix only that a random subset of the
 * gradient is kept; this call keeps exactly k entries, drawn without replacement from a
 * counter-based generator, so that the payload has a fixed size and the choice is
 * reproducible on any rank and independent of the values:
 *   key_i  = (Philox word of global index index_base + i under select_seed) >> 1
 *            (the same word the quantizers draw, see the top of this file; 31 bits)
 *   S      = the k elements with the largest key; among equal keys the lower index wins
 * and then everything as gc_ef_topk with this S: c = fl(grad + residual), out_idx
 * ascending (plus index_base), out_val = c[idx] or QSGD of those values, and the residual
 * at kept positions +0.0 (pure) or fl(v - g_hat) (with QSGD).  The choice depends only on
 * (select_seed, index_base, n, k); callers pass a new seed each step.
 *
 * Arguments, layout, ownership and errors as gc_ef_topk.
 * Workspace: gc_workspace_size(GC_OP_EF_RANDK, n, k, qsgd_levels).
 */
int gc_ef_randk(const float* grad, float* residual, int64_t n, int64_t k, int64_t index_base,
                uint64_t select_seed, int64_t* out_idx, float* out_val,
                int qsgd_levels, int64_t qsgd_group, uint64_t qsgd_seed,
                int8_t* out_codes, float* out_norms,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_quant_minmax -- per-group min-max (linear) quantization with deterministic
 * rounding.
 *
 * Operation ([P2] section 二.1 linear quantization and section 三 error
 * compensation; [P4] "Python 演示" quantize; grouping: [P1] section 1.2):
 *   x'    = fl(x + residual) if residual != NULL, else x
 *   per group: mn = min, mx = max, scale = fl(fl(mx - mn) / (2^bits - 1))
 *   q     = scale == 0 ? 0 : clamp(rint(fl(fl(x' - mn) / scale)), 0, 2^bits - 1)
 *   g_hat = fl(fl(q * scale) + mn);  residual := fl(x' - g_hat) if residual != NULL
 * group: 0 (one group over all n), a power of two in [4,256], or any value > 256.  The
 * last group may be partial.  bits: 8 -> codes uint8[n]; 4 -> codes uint8[ceil(n/2)],
 * element 2j in the low nibble of byte j, an odd tail leaves the high nibble 0.
 * mins, scales: float[ngroups].  x, residual: 16-byte aligned.
 * Workspace: gc_workspace_size(GC_OP_QUANT_MINMAX, n, group, 0) (0 for small groups).
 */
int gc_quant_minmax(const float* x, float* residual, int64_t n, int64_t group, int bits,
                    uint8_t* codes, float* mins, float* scales,
                    void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_qsgd -- QSGD stochastic quantization onto `levels` levels of the group L2 norm.
 *
 * Operation ([P1] section 1.1: stochastic rounding between levels, unbiased, used with
 * error feedback; grouping [P1] section 1.2; levels of the norm as in the QSGD paper
 * [P1] cites):
 *   x' = fl(x + residual) if residual != NULL, else x
 *   nu = fl(sqrt(sum of x'^2 over the group, balanced pairwise tree in index order))
 *   u = fl(fl(|x'|/nu) * s), l = floor(u), p = u - l,
 *   level = min(l + (U(seed, index_base + i) < p), s), code = (x' < 0 ? -level : level)
 *   nu == 0 gives code 0.  residual := fl(x' - g_hat), g_hat = sign * fl(fl(nu*level)/s).
 * group: power of two in [4,256].  levels: [1,127].  codes: int8[n]; norms: float[ngroups].
 * index_base >= 0.  Needs no workspace.
 */
int gc_qsgd(const float* x, float* residual, int64_t n, int64_t group, int levels,
            uint64_t seed, int64_t index_base, int8_t* codes, float* norms, void* stream);

/*
 * gc_stream_floor -- calibration for benchmarks, not part of any compressor:
 * out[i] = (x[i] > 0) ? 1 : 0 for i < n, and nothing else.  It moves the bytes a one-pass
 * 8-bit quantizer of x moves (4 read and 1 written per element, 16-byte loads, 4-byte
 * stores), so its time at a given size is the floor such a pass is measured against.
 * x: float[n], 16-byte aligned.  out: uint8[n], 4-byte aligned.  n in [0, 2^40].
 * Errors: GC_EINVAL (checked on the host), GC_EHIP.
 */
int gc_stream_floor(const float* x, uint8_t* out, int64_t n, void* stream);

/*
 * gc_terngrad -- TernGrad ternary codes with one scale per segment (layer).
 *
 * Operation ([P1] section 1.1: codes in {-1,0,+1}, layer-wise normalization; the scheme
 * of the TernGrad paper [P1] cites):
 *   x' = fl(x + residual) if residual != NULL, else x
 *   per segment s: scale_s = max |x'|;  p = fl(|x'| / scale_s)
 *   code = (U(seed, index_base + i) < p) ? (x' < 0 ? -1 : +1) : 0, for global position i
 *   scale_s == 0 gives code 0.  residual := fl(x' - code*scale_s).
 * seg_offsets: HOST int64[nseg+1], seg_offsets[0] == 0, nondecreasing; n = seg_offsets[nseg].
 * packed: segment s occupies bytes [B_s, B_s + ceil(len_s/4)), B_s = sum_{j<s} ceil(len_j/4);
 *   element t of the segment sits in bits 2(t%4)..2(t%4)+1 of byte B_s + t/4, with
 *   0 -> 00, +1 -> 01, -1 -> 11; unused bits are 0.  scales: float[nseg].
 * x, residual: 16-byte aligned.  index_base >= 0.
 * Workspace: gc_workspace_size(GC_OP_TERNGRAD, n, nseg, 0) bytes, about 0.64 bytes per
 * element (two sets of 64 partial maxima per segment, and per tile of 4032 elements a
 * list of up to 128 bytes whose codes the streaming pass could not settle, with their
 * values); 0 when n == 0.  Calls that share a workspace must not overlap on the device.
 */
int gc_terngrad(const float* x, float* residual, int nseg, const int64_t* seg_offsets,
                uint64_t seed, int64_t index_base, uint8_t* packed, float* scales,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_powersgd_step -- one PowerSGD power-iteration step with error feedback.
 *
 * Operation ([P1] section 3.1: low-rank approximation, only the two thin factors are
 * sent, rebuilt at the receiver; [P4] "梯度压缩原理": run with error compensation; the
 * step of the PowerSGD paper [P1] cites):
 *   M = fl(grad + residual) (M = grad if residual == NULL)
 *   P = M Q;  P^ = modified Gram-Schmidt of P's columns (norm-0 column -> 0)
 *   Q' = M^T P^;  residual := M - P^ Q'^T  (skipped if residual == NULL)
 * grad, residual: rows x cols row-major float, 16-byte aligned, cols % 4 == 0.
 * Q: cols x rank row-major float, in: Q_{t-1}, out: Q'.  P: rows x rank row-major, out: P^.
 * rank: [1,4].  Products accumulate in fp32; agreement with a float64 evaluation is to
 * about 1e-6 relative (Frobenius).
 * Workspace: gc_workspace_size(GC_OP_POWERSGD, rows, cols, rank).
 */
int gc_powersgd_step(const float* grad, float* residual, int64_t rows, int64_t cols, int rank,
                     float* Q, float* P, void* workspace, size_t workspace_bytes, void* stream);

/*
 * gc_decompress_scatter -- decode a payload and store or add it into a dense fp32 vector.
 *
 * Operation ([P2] section 四: the receiver decompresses before the update; section 二.2:
 * the sparse gradient is dense with zeros off the kept set).  For entry j < count,
 * g_hat_j is the dequantization of the payload kind (see enum gc_kind and the matching
 * compressor above); group g = j / group (group 0: one group).  Then
 *   pos_j = idx ? idx[j] - index_base : j
 *   out[pos_j] = fl(alpha * g_hat_j)            (accumulate == 0)
 *   out[pos_j] = fl(out[pos_j] + fl(alpha * g_hat_j))   (accumulate != 0)
 * Entries whose pos_j falls outside [0, n_out) are skipped.  idx entries must be
 * distinct (Top-K output is).  levels is used by GC_KIND_QSGD only.
 */
int gc_decompress_scatter(int kind, const int64_t* idx, int64_t count, int64_t index_base,
                          const void* codes, const float* meta0, const float* meta1,
                          int64_t group, int levels, float alpha, int accumulate,
                          float* out, int64_t n_out, void* stream);

/*
 * Wire format of one payload, and the receive side of a data-parallel step.
 *
 * Operation ([P2] section 四: each worker sends its compressed gradient, the gradients
 * are aggregated and every worker decompresses before the update; [P4] "通信瓶颈分析":
 * aggregation sums the workers' gradients and averages them).  Codes of different
 * workers cannot be summed as they are (each has its own scales or index set), so a
 * receiver gathers W payloads and computes out = sum_w alpha * g_hat_w, with alpha = 1/W
 * for the average.
 *
 * A payload is one contiguous byte buffer: this 128-byte header, then the sections it
 * lists, each starting at a multiple of 256 bytes from the payload start:
 *   idx    int64[count], strictly ascending  (sparse payloads only; flags & GC_PAYLOAD_SPARSE)
 *   codes  as for gc_decompress_scatter: float[count] (F32), uint8[count] (MINMAX8),
 *          uint8[ceil(count/2)] (MINMAX4), int8[count] (QSGD), uint8[ceil(count/4)] (TERN)
 *   meta0  float[ng]: mins (MINMAX*), norms (QSGD), scales (TERN); absent for F32
 *   meta1  float[ng]: scales (MINMAX*); absent otherwise
 * with ng = ceil(count / group) (group 0: one group).  Multi-byte fields are
 * little-endian.  An absent section has offset 0.  The producer fills the sections by
 * pointing the compressors at them.
 */
#define GC_PAYLOAD_MAGIC 0x31504347u   /* "GCP1" */
#define GC_PAYLOAD_VERSION 1u
#define GC_PAYLOAD_SPARSE 1u

typedef struct gc_payload_header {
  uint32_t magic;        /* GC_PAYLOAD_MAGIC */
  uint16_t version;      /* GC_PAYLOAD_VERSION */
  uint16_t kind;         /* enum gc_kind */
  uint32_t flags;        /* GC_PAYLOAD_SPARSE */
  int32_t levels;        /* QSGD levels (0 for other kinds) */
  int64_t n;             /* length of the dense gradient the payload encodes */
  int64_t count;         /* entries */
  int64_t index_base;    /* subtracted from idx (sparse payloads) */
  int64_t group;         /* entries per metadata group, 0 = one group */
  uint64_t off_idx;      /* byte offsets of the sections from the payload start */
  uint64_t off_codes;
  uint64_t off_meta0;
  uint64_t off_meta1;
  uint64_t bytes;        /* total payload size */
  uint8_t reserved[40];  /* zero */
} gc_payload_header;

/*
 * gc_payload_layout -- fill *hdr (host) for a payload of the given shape: the offsets of
 * its sections and its total size.  Host only; no device call.  sparse != 0 adds the
 * idx section.  Errors: GC_EINVAL for an unknown kind, count < 0, count > n for a dense
 * payload, a group that is negative, or levels outside [1, 127] for QSGD.
 */
int gc_payload_layout(int kind, int64_t n, int64_t count, int64_t group, int levels, int sparse,
                      int64_t index_base, gc_payload_header* hdr);

/*
 * gc_decompress_payloads -- out = (accumulate ? out : 0) + sum over w = 0..W-1, in this
 * order, of alpha * g_hat_w, where g_hat_w is payload w decoded as gc_decompress_scatter
 * decodes it (scattered through its idx when sparse).  Every element receives its terms
 * one at a time in payload order: out_e = fl(out_e + fl(alpha * g_hat_{w,e})).
 * payloads: HOST array of W device pointers, each 256-byte aligned; headers: HOST array of
 * their W headers (the caller holds them: it built them, or read them after the gather).
 * Each payload must encode n <= n_out elements.  W in [1, 1024].
 * When every payload is dense with the same kind, count, group and levels, one pass
 * reads all W code streams and writes out once (up to 16 payloads per launch).  When
 * every payload is sparse, the payloads are merged tile by tile (their idx must be
 * strictly ascending, as the wire format requires and gc_ef_compress writes them; with
 * unsorted idx the result is undefined but every access stays inside its buffers), each
 * payload read once and out written once (up to 16 payloads per launch).  Otherwise out
 * is cleared (if accumulate == 0) and the payloads are added one launch each.  Needs no
 * workspace.
 */
int gc_decompress_payloads(int W, const void* const* payloads, const gc_payload_header* headers,
                           float alpha, int accumulate, float* out, int64_t n_out, void* stream);

/*
 * Stage timing (profiling aid, not part of any operation).  While enabled, every
 * gc_ef_topk call records four HIP events on its stream: call start, start and end of the
 * full streaming pass (the fused add + candidate kernel), and call end.
 * gc_profile_collect() waits for the recorded events, returns the number of calls and the
 * summed milliseconds of [start, pass start), [pass start, pass end) and [pass end, end),
 * and clears the record.  Host-side state, guarded by a mutex; events are created by the
 * HIP runtime (no device memory is allocated by the library).
 */
int gc_profile_enable(int on);
int gc_profile_collect(int64_t* calls, double* ms_before, double* ms_pass, double* ms_after);

#ifdef __cplusplus
}
#endif

#endif /* GC_H */
