// PowerSGD rank-r step (r <= 4) with error feedback, gfx950.
//
// Operation: hotdry.top "gradient-compression-quantization-sparsification", section 3.1
// (low-rank approximation; only the two thin factors are sent and the product is rebuilt
// at the receiver; extra compute) and aiqz.cc "梯度聚合通信优化实战方案", section
// "梯度压缩原理" (run with error compensation); one power-iteration step of the PowerSGD
// paper the first page cites:
//   M = G + E;  P = M Q;  P^ = Gram-Schmidt(P);  Q' = M^T P^;  E' = M - P^ Q'^T.
//
// At rank 4 both products are skinny (about 1 flop per byte of M), so the step is
// HBM-bound: three passes over M (12 + 4 + 8 bytes per element).  The two products run on
// the matrix cores with v_mfma_f32_4x4x1_16b_f32: its 16 blocks are 4x4 outer products,
// which at rank 4 leave no lane idle.
//   pass 1: lane (b, i) of a wave loads a float4 of row i at columns 4b..4b+3 of a 64-column
//           step; MFMA s (s = 0..3) uses component s, so block b accumulates
//           M[row i][k] * Q[k][j] for k = base + 4b + s; the 16 blocks are summed at the end.
//   pass 2: lane (b, j) loads a float4 of one row; block b gets columns 16b + 4i + s of that
//           row as A and P^[row][j] as B, accumulating Q' partials over the rows.
//   pass 3: E' = M - P^ Q'^T on the vector ALU (4 fused multiply-adds per element).
// Partial sums over column / row panels are reduced in a fixed order, so the result is
// deterministic.  Gram-Schmidt runs on the 4x4 Gram matrix P^T P accumulated in float64:
// P^ = P T with T upper triangular, computed by modified Gram-Schmidt in coefficient space.
#include "common.hpp"
#include "internal.hpp"

namespace gc {
namespace {

constexpr int kBlock = 256;
constexpr int kP1Cols = 256;      // column panel of pass 1 (4 steps of 64)
constexpr int kRowsPerWave = 16;  // pass 1 and 2: 16 rows per wave, 64 per block
constexpr int kRowsPerBlock = 64;
constexpr int kP3Rows = 16;       // pass 3 rows per block
constexpr int kGramBlocks = 64;    // the last one sums their Gram partials, one per lane

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct PLayout {
  float* ppart;   // [ncp * rows * 4]          pass-1 partials per column panel
  float* p;       // [rows * 4]                P = M Q
  double* gram;   // [kGramBlocks * 10]        Gram partials
  float* phat;    // [rows * 4]
  float* qpart;   // [nrp * cols * 4]          pass-2 partials per row panel
  float* qn;      // [cols * 4]                Q'
  double* T;      // [16]                      Gram-Schmidt coefficients, row-major
  uint32_t* ticket;   // last-block hand-off of the Gram reduction
  int64_t ncp, nrp;
  size_t bytes;
};

PLayout make_playout(void* base, int64_t rows, int64_t cols) {
  PLayout l{};
  l.ncp = cdiv(cols, kP1Cols);
  l.nrp = cdiv(rows, kRowsPerBlock);
  size_t off = 0;
  char* b = reinterpret_cast<char*>(base);
  auto take = [&](size_t bytes) -> void* {
    void* p = b ? b + off : nullptr;
    off += align256(bytes);
    return p;
  };
  l.ppart = (float*)take(sizeof(float) * l.ncp * rows * 4);
  l.p = (float*)take(sizeof(float) * rows * 4);
  l.gram = (double*)take(sizeof(double) * kGramBlocks * 10);
  l.phat = (float*)take(sizeof(float) * rows * 4);
  l.qpart = (float*)take(sizeof(float) * l.nrp * cols * 4);
  l.qn = (float*)take(sizeof(float) * cols * 4);
  l.T = (double*)take(sizeof(double) * 16);
  l.ticket = (uint32_t*)take(sizeof(uint32_t));
  l.bytes = off;
  return l;
}

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ f32x4 load4_or_zero(const float* p, bool ok) {
  if (ok) return *reinterpret_cast<const f32x4*>(p);
  f32x4 z = {0.f, 0.f, 0.f, 0.f};
  return z;
}

// Pass 1: M = G + E (written over E when E is given) and P partials per column panel.
// Lane (b, i) takes Q[col + s][i] for the 4 columns col = kg*64 + 4b of its step (zero
// outside cols x rank); Q is small enough to stay in cache.
template <bool EF>
__global__ __launch_bounds__(kBlock) void k_p1(const float* __restrict__ G, float* __restrict__ E,
                                               int64_t rows, int64_t cols, const float* __restrict__ Q,
                                               int rank, float* __restrict__ ppart, uint32_t* __restrict__ ticket) {
  // the Gram reduction's hand-off ticket starts at zero (the workspace is the caller's)
  if (blockIdx.x == 0 && blockIdx.y == 0 && threadIdx.x == 0) *ticket = 0u;
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int64_t cp = blockIdx.x;
  const int64_t r0 = (int64_t)blockIdx.y * kRowsPerBlock + w * kRowsPerWave;
  const int b = lane >> 2, i = lane & 3;
  f32x4 acc[4];
#pragma unroll
  for (int g = 0; g < 4; ++g) acc[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int ks = 0; ks < kP1Cols / 64; ++ks) {
    const int64_t kg = cp * (kP1Cols / 64) + ks;
    const int64_t col = kg * 64 + 4 * b;
    const bool col_ok = col < cols;
    f32x4 qv;
#pragma unroll
    for (int s = 0; s < 4; ++s) qv[s] = (col + s < cols && i < rank) ? Q[(col + s) * rank + i] : 0.f;
    f32x4 m[4];
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int64_t row = r0 + 4 * g + i;
      const bool ok = col_ok && row < rows;
      const int64_t off = row * cols + col;
      m[g] = load4_or_zero(G + off, ok);
      if (EF) {
        const f32x4 e = load4_or_zero(E + off, ok);
        m[g] = f32x4{m[g].x + e.x, m[g].y + e.y, m[g].z + e.z, m[g].w + e.w};
        if (ok) *reinterpret_cast<f32x4*>(E + off) = m[g];
      }
    }
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      acc[g] = mfma4(m[g].x, qv.x, acc[g]);
      acc[g] = mfma4(m[g].y, qv.y, acc[g]);
      acc[g] = mfma4(m[g].z, qv.z, acc[g]);
      acc[g] = mfma4(m[g].w, qv.w, acc[g]);
    }
  }
  // sum the 16 blocks (lanes with equal lane%4) in a fixed butterfly order
#pragma unroll
  for (int g = 0; g < 4; ++g) {
#pragma unroll
    for (int m = 4; m < kWave; m <<= 1) {
      acc[g].x += __shfl_xor(acc[g].x, m, kWave);
      acc[g].y += __shfl_xor(acc[g].y, m, kWave);
      acc[g].z += __shfl_xor(acc[g].z, m, kWave);
      acc[g].w += __shfl_xor(acc[g].w, m, kWave);
    }
  }
  if (lane < 4) {
    const int j = lane;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float v[4] = {acc[g].x, acc[g].y, acc[g].z, acc[g].w};
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int64_t row = r0 + 4 * g + ii;
        if (row < rows) ppart[(cp * rows + row) * 4 + j] = v[ii];
      }
    }
  }
}

// Modified Gram-Schmidt in coefficient space: columns of T give P^ = P T.  A column in the
// span of the previous ones becomes 0; numerically, one whose projected norm is at most
// 1e-5 of its own norm (squared: 1e-10), below which its direction is rounding noise.
// One wave: lane l sums the block partials l, l + 64, ... in order, then a fixed xor
// butterfly combines the lanes (deterministic); lane 0 runs the 4x4 Gram-Schmidt.
// Called by the first wave of a block; lane 0 writes T (4 x 4, row-major) to `T`.
__device__ __forceinline__ void gram_schmidt_t(const double* __restrict__ gram, int nblocks, int rank,
                                               double* T) {
  double g[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) g[t] = 0.0;
  for (int b = threadIdx.x; b < nblocks; b += kWave)
#pragma unroll
    for (int t = 0; t < 10; ++t) g[t] += gram[b * 10 + t];
#pragma unroll
  for (int t = 0; t < 10; ++t)
    for (int m = 1; m < kWave; m <<= 1) g[t] += __shfl_xor(g[t], m, kWave);
  if (threadIdx.x != 0) return;
  double G[4][4];
  int t = 0;
  for (int a = 0; a < 4; ++a)
    for (int bb = a; bb < 4; ++bb) { G[a][bb] = g[t]; G[bb][a] = g[t]; ++t; }
  double Tm[4][4] = {{0}};
  for (int j = 0; j < rank; ++j) {
    double v[4] = {0, 0, 0, 0};
    v[j] = 1.0;
    for (int i = 0; i < j; ++i) {
      // c = <p^_i, v> = T_i^T G v
      double c = 0.0;
      for (int a = 0; a < 4; ++a) {
        double gv = 0.0;
        for (int bb = 0; bb < 4; ++bb) gv += G[a][bb] * v[bb];
        c += Tm[a][i] * gv;
      }
      for (int a = 0; a < 4; ++a) v[a] -= c * Tm[a][i];
    }
    double nrm2 = 0.0;
    for (int a = 0; a < 4; ++a) {
      double gv = 0.0;
      for (int bb = 0; bb < 4; ++bb) gv += G[a][bb] * v[bb];
      nrm2 += v[a] * gv;
    }
    const bool zero = !(nrm2 > 1e-10 * G[j][j]) || !(G[j][j] > 0.0);
    const double inv = zero ? 0.0 : 1.0 / sqrt(nrm2);
    for (int a = 0; a < 4; ++a) Tm[a][j] = v[a] * inv;
  }
  for (int a = 0; a < 4; ++a)
    for (int bb = 0; bb < 4; ++bb) T[a * 4 + bb] = Tm[a][bb];
}

// P = sum of the panel partials (in panel order); float64 partials of the Gram matrix.
// The last block to finish sums the partials and derives T (gram_schmidt_t), so pass 2
// can form P^ = P T row by row.
__global__ __launch_bounds__(kBlock) void k_psum_gram(const float* __restrict__ ppart, int64_t ncp,
                                                      int64_t rows, float* __restrict__ p,
                                                      double* __restrict__ gram, int rank,
                                                      double* __restrict__ T, uint32_t* __restrict__ ticket) {
  __shared__ double s[kBlock / kWave][10];
  double acc[10];
#pragma unroll
  for (int t = 0; t < 10; ++t) acc[t] = 0.0;
  for (int64_t row = (int64_t)blockIdx.x * kBlock + threadIdx.x; row < rows;
       row += (int64_t)gridDim.x * kBlock) {
    // panel partials in panel order; 8 loads are issued ahead of their additions
    constexpr int kAhead = 8;
    float v[4] = {0.f, 0.f, 0.f, 0.f};
    int64_t c = 0;
    for (; c + kAhead <= ncp; c += kAhead) {
      f32x4 q[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) q[u] = *reinterpret_cast<const f32x4*>(ppart + ((c + u) * rows + row) * 4);
#pragma unroll
      for (int u = 0; u < kAhead; ++u) { v[0] += q[u].x; v[1] += q[u].y; v[2] += q[u].z; v[3] += q[u].w; }
    }
    for (; c < ncp; ++c) {
      const f32x4 q = *reinterpret_cast<const f32x4*>(ppart + (c * rows + row) * 4);
      v[0] += q.x; v[1] += q.y; v[2] += q.z; v[3] += q.w;
    }
    *reinterpret_cast<f32x4*>(p + row * 4) = f32x4{v[0], v[1], v[2], v[3]};
    int t = 0;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int bb = a; bb < 4; ++bb) acc[t++] += (double)v[a] * (double)v[bb];
  }
#pragma unroll
  for (int t = 0; t < 10; ++t)
    for (int m = 1; m < kWave; m <<= 1) acc[t] += __shfl_xor(acc[t], m, kWave);
  if (lane_id() == 0)
    for (int t = 0; t < 10; ++t) s[threadIdx.x / kWave][t] = acc[t];
  __syncthreads();
  if (threadIdx.x < 10)
    gram[blockIdx.x * 10 + threadIdx.x] = ((s[0][threadIdx.x] + s[1][threadIdx.x]) + s[2][threadIdx.x]) +
                                          s[3][threadIdx.x];
  if (last_block(ticket) && threadIdx.x < kWave) gram_schmidt_t(gram, (int)gridDim.x, rank, T);
}

// Row `row` of P^ = P T, component j (float64 accumulation in i order, one rounding;
// components j >= rank are 0).
__device__ __forceinline__ float phat_of(const float* __restrict__ p, const double* __restrict__ T, int64_t row,
                                         int j, int rank) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p + row * 4);
  const double pv[4] = {v.x, v.y, v.z, v.w};
  double a = 0.0;
#pragma unroll
  for (int i = 0; i < 4; ++i) a += pv[i] * T[i * 4 + j];
  return j < rank ? (float)a : 0.f;
}

// Pass 2: Q' partials per row panel, Q'[c][j] = sum_rows M[row][c] * P^[row][j], with
// P^ = P T formed here for the block's 64 rows (one value per thread, into LDS); the
// first column panel also writes P^ (padded, for pass 3) and the caller's rows x rank P.
__global__ __launch_bounds__(kBlock) void k_p2(const float* __restrict__ M, int64_t rows, int64_t cols,
                                               const float* __restrict__ p, const double* __restrict__ Tg,
                                               int rank, float* __restrict__ phat, float* __restrict__ P_out,
                                               float* __restrict__ qpart) {
  __shared__ float s_acc[kBlock / kWave][kWave][16];
  __shared__ double sT[16];
  __shared__ float s_ph[kRowsPerBlock * 4];
  constexpr int kPre = 4;   // rows of M loaded before P^ is formed
  static_assert(kRowsPerBlock * 4 == kBlock, "one P^ value per thread");
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int64_t c0 = (int64_t)blockIdx.x * 256;
  const int64_t rp = blockIdx.y;
  const int64_t r0 = rp * kRowsPerBlock + w * kRowsPerWave;
  const int64_t col = c0 + 4 * lane;
  const bool col_ok = col < cols;
  f32x4 pre[kPre];
#pragma unroll
  for (int rr = 0; rr < kPre; ++rr) pre[rr] = load4_or_zero(M + (r0 + rr) * cols + col, r0 + rr < rows && col_ok);
  if (threadIdx.x < 16) sT[threadIdx.x] = Tg[threadIdx.x];
  __syncthreads();
  {
    const int64_t row = rp * kRowsPerBlock + (threadIdx.x >> 2);
    const int j = threadIdx.x & 3;
    const float v = row < rows ? phat_of(p, sT, row, j, rank) : 0.f;
    s_ph[threadIdx.x] = v;
    if (blockIdx.x == 0 && row < rows) {
      phat[row * 4 + j] = v;
      if (j < rank) P_out[row * rank + j] = v;
    }
  }
  __syncthreads();
  f32x4 acc[4];
#pragma unroll
  for (int s = 0; s < 4; ++s) acc[s] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int rr = 0; rr < kPre; ++rr) {
    const float bv = s_ph[(w * kRowsPerWave + rr) * 4 + (lane & 3)];
    acc[0] = mfma4(pre[rr].x, bv, acc[0]);
    acc[1] = mfma4(pre[rr].y, bv, acc[1]);
    acc[2] = mfma4(pre[rr].z, bv, acc[2]);
    acc[3] = mfma4(pre[rr].w, bv, acc[3]);
  }
#pragma unroll 4
  for (int rr = kPre; rr < kRowsPerWave; ++rr) {
    const int64_t row = r0 + rr;
    const bool ok = row < rows;
    const f32x4 m = load4_or_zero(M + row * cols + col, ok && col_ok);
    const float bv = s_ph[(w * kRowsPerWave + rr) * 4 + (lane & 3)];
    acc[0] = mfma4(m.x, bv, acc[0]);
    acc[1] = mfma4(m.y, bv, acc[1]);
    acc[2] = mfma4(m.z, bv, acc[2]);
    acc[3] = mfma4(m.w, bv, acc[3]);
  }
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    s_acc[w][lane][s * 4 + 0] = acc[s].x;
    s_acc[w][lane][s * 4 + 1] = acc[s].y;
    s_acc[w][lane][s * 4 + 2] = acc[s].z;
    s_acc[w][lane][s * 4 + 3] = acc[s].w;
  }
  __syncthreads();
  // thread t owns column c0 + t: lane (b, j) register (s, i) holds column 16b + 4i + s
  const int co = threadIdx.x;
  const int bb = co >> 4, i = (co >> 2) & 3, s = co & 3;
  if (c0 + co < cols) {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int L = 4 * bb + j, reg = s * 4 + i;
      const float v = ((s_acc[0][L][reg] + s_acc[1][L][reg]) + s_acc[2][L][reg]) + s_acc[3][L][reg];
      qpart[(rp * cols + c0 + co) * 4 + j] = v;
    }
  }
}

// Q' = sum of the row-panel partials (in panel order); padded copy and the caller's Q.
// Thread t owns entry (column t/4, component t%4): neighbouring threads read neighbouring
// floats, and 8 partials are loaded ahead of their (in-order) additions.
__global__ __launch_bounds__(256) void k_qsum(const float* __restrict__ qpart, int64_t nrp, int64_t cols,
                                              int rank, float* __restrict__ qn, float* __restrict__ Q_out) {
  constexpr int kAhead = 8;
  const int64_t total = cols * 4;
  for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < total;
       t += (int64_t)gridDim.x * blockDim.x) {
    const int64_t c = t >> 2;
    const int j = (int)(t & 3);
    float v = 0.f;
    int64_t r = 0;
    for (; r + kAhead <= nrp; r += kAhead) {
      float a[kAhead];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) a[u] = qpart[(r + u) * total + t];
#pragma unroll
      for (int u = 0; u < kAhead; ++u) v += a[u];
    }
    for (; r < nrp; ++r) v += qpart[r * total + t];
    if (j >= rank) v = 0.f;
    qn[t] = v;
    if (j < rank) Q_out[c * rank + j] = v;
  }
}

// Pass 3: E' = M - P^ Q'^T.  A thread owns 4 columns for a band of rows.
__global__ __launch_bounds__(kBlock) void k_p3(const float* __restrict__ M, float* __restrict__ Eout,
                                               int64_t rows, int64_t cols, const float* __restrict__ phat,
                                               const float* __restrict__ qn) {
  const int64_t col = (int64_t)blockIdx.x * (kBlock * 4) + 4 * threadIdx.x;
  if (col >= cols) return;
  float q[4][4];
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(qn + (col + m) * 4);
    q[m][0] = v.x; q[m][1] = v.y; q[m][2] = v.z; q[m][3] = v.w;
  }
  const int64_t r0 = (int64_t)blockIdx.y * kP3Rows;
#pragma unroll 4
  for (int rr = 0; rr < kP3Rows; ++rr) {
    const int64_t row = r0 + rr;
    if (row >= rows) break;
    const f32x4 ph = *reinterpret_cast<const f32x4*>(phat + row * 4);
    // the last read of M and the one write of E: non-temporal (4096^2 90.8 -> 86.8 us,
    // 4096x11008 210.8 -> 200.6 us a step; the same hint on pass 1's reads of G and E
    // helped the square shape and slowed the others)
    const f32x4 m = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(M + row * cols + col));
    const float mv[4] = {m.x, m.y, m.z, m.w};
    float o[4];
#pragma unroll
    for (int mm = 0; mm < 4; ++mm) {
      float d = ph.x * q[mm][0];
      d = fmaf(ph.y, q[mm][1], d);
      d = fmaf(ph.z, q[mm][2], d);
      d = fmaf(ph.w, q[mm][3], d);
      o[mm] = mv[mm] - d;
    }
    __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<f32x4*>(Eout + row * cols + col));
  }
}

int clamp_grid(int64_t want, int64_t cap) {
  if (want < 1) want = 1;
  return (int)(want > cap ? cap : want);
}

}  // namespace

size_t powersgd_workspace(int64_t rows, int64_t cols, int) { return make_playout(nullptr, rows, cols).bytes; }

hipError_t launch_powersgd(const float* grad, float* res, int64_t rows, int64_t cols, int rank, float* Q,
                           float* P, void* ws, hipStream_t s) {
  const PLayout l = make_playout(ws, rows, cols);
  const int cus = device_cu_count();
  const dim3 g1((unsigned)l.ncp, (unsigned)l.nrp);
  if (res)
    hipLaunchKernelGGL((k_p1<true>), g1, kBlock, 0, s, grad, res, rows, cols, (const float*)Q, rank, l.ppart, l.ticket);
  else
    hipLaunchKernelGGL((k_p1<false>), g1, kBlock, 0, s, grad, res, rows, cols, (const float*)Q, rank, l.ppart, l.ticket);
  hipLaunchKernelGGL(k_psum_gram, kGramBlocks, kBlock, 0, s, l.ppart, l.ncp, rows, l.p, l.gram, rank, l.T, l.ticket);
  const float* M = res ? res : grad;
  const dim3 g2((unsigned)cdiv(cols, 256), (unsigned)l.nrp);
  hipLaunchKernelGGL(k_p2, g2, kBlock, 0, s, M, rows, cols, (const float*)l.p, (const double*)l.T, rank, l.phat, P,
                     l.qpart);
  hipLaunchKernelGGL(k_qsum, clamp_grid(cdiv(cols * 4, 256), cus * 8), 256, 0, s, l.qpart, l.nrp, cols, rank, l.qn, Q);
  if (res) {
    const dim3 g3((unsigned)cdiv(cols, kBlock * 4), (unsigned)cdiv(rows, kP3Rows));
    hipLaunchKernelGGL(k_p3, g3, kBlock, 0, s, M, res, rows, cols, l.phat, l.qn);
  }
  return hipGetLastError();
}

}  // namespace gc
