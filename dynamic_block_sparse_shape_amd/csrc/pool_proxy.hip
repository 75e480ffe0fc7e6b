// Stage 2: block mean-pooling and the block proxy score.
//
// README "Overview": block-level features stand for a block; the abstract
// page ("Prism: Dynamic Sparse Attention ...") routes on block proxy scores.
// qbar_i = mean of block i's 64 query rows (fp64; a sum of 64 bf16 values
// is exact in fp64), proxy_i = softmax_j(<qbar_i, kbar_j> / sqrt(d)) in fp64
// so that the selection downstream decides on fp64 values.
//
//   pool_blocks    one workgroup per (b, h, block): 16-byte loads of the 64
//                  gathered rows, fp64 accumulation, fixed-order reduction.
//   proxy_logits   fp64 MFMA (v_mfma_f64_16x16x4) GEMM, 64x64 tile per
//                  workgroup, k-slices of 32 staged in LDS; writes scaled
//                  logits into the proxy buffer.
//   row_softmax    one workgroup per row, row held in registers; max, exp,
//                  sum, normalise in fp64, written in place.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kThreads = 256;

template <typename E>
__device__ __forceinline__ double elem(const unsigned char* p);
template <>
__device__ __forceinline__ double elem<uint16_t>(const unsigned char* p) {
  return (double)bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}
template <>
__device__ __forceinline__ double elem<float>(const unsigned char* p) {
  return (double)*reinterpret_cast<const float*>(p);
}

template <typename E, int D>
__global__ __launch_bounds__(kThreads) void pool_blocks(
    const unsigned char* __restrict__ q, const unsigned char* __restrict__ k,
    const int32_t* __restrict__ perm, int Hh, int N,
    double* __restrict__ q_mean, double* __restrict__ k_mean) {
  constexpr int RB = D * (int)sizeof(E);     // bytes per row
  constexpr int TPR = RB / 16;               // threads per row
  constexpr int RPP = kThreads / TPR;        // rows per pass
  constexpr int EPV = 16 / (int)sizeof(E);   // elements per 16 B
  __shared__ double part[RPP][D];
  __shared__ int rows[64];

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  if (threadIdx.x < 64) rows[threadIdx.x] = perm[(long long)b * N + 64 * i + threadIdx.x];
  __syncthreads();
  const int piece = threadIdx.x % TPR;
  const int rg = threadIdx.x / TPR;
  const long long head_off = ((long long)b * Hh + h) * N;
  const long long out_off = (((long long)b * Hh + h) * Nb + i) * D;

  for (int t = 0; t < 2; ++t) {
    const unsigned char* src = t == 0 ? q : k;
    double acc[EPV];
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
#pragma unroll
    for (int r = rg; r < 64; r += RPP) {
      const uint4 v = *reinterpret_cast<const uint4*>(
          src + (head_off + rows[r]) * RB + piece * 16);
      const unsigned char* pv = reinterpret_cast<const unsigned char*>(&v);
#pragma unroll
      for (int e = 0; e < EPV; ++e) acc[e] += elem<E>(pv + e * sizeof(E));
    }
#pragma unroll
    for (int e = 0; e < EPV; ++e) part[rg][piece * EPV + e] = acc[e];
    __syncthreads();
    if (threadIdx.x < D) {
      double s = 0.0;
      for (int g = 0; g < RPP; ++g) s += part[g][threadIdx.x];
      (t == 0 ? q_mean : k_mean)[out_off + threadIdx.x] = s * (1.0 / 64.0);
    }
    __syncthreads();
  }
}

// Z = Qbar Kbar^T / sqrt(d) with fp64 MFMA.  v_mfma_f64_16x16x4 operands:
// A[i][k] in lane i + 16k, B[k][j] in lane j + 16k, D[i][j] in lane
// j + 16 (i % 4), element i / 4 (unlike the fp32 16x16 layout).
constexpr int kTile = 64;
constexpr int kKs = 32;                 // k-slice staged in LDS
constexpr int kLd = kKs + 1;            // padded LDS row (doubles)

typedef double f64x4 __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void proxy_logits(
    const double* __restrict__ qm, const double* __restrict__ km, int Nb,
    int d, double sqrt_d, double* __restrict__ z) {
  __shared__ double As[kTile * kLd];
  __shared__ double Bs[kTile * kLd];
  const int ti = blockIdx.x, tj = blockIdx.y, bh = blockIdx.z;
  const double* Q = qm + (long long)bh * Nb * d;
  const double* K = km + (long long)bh * Nb * d;
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  const int wi = (wave >> 1) * 32, wj = (wave & 1) * 32;   // wave's 32x32
  f64x4 acc[2][2];
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int c = 0; c < 2; ++c) acc[a][c] = f64x4{0.0, 0.0, 0.0, 0.0};

  // each thread holds 8 doubles of each operand's next k-slice in registers
  // (rows r = tid / 32 + 8 u, column tid % 32): the global loads of slice
  // k0 + 32 are in flight while slice k0 is multiplied from LDS
  constexpr int kPer = kTile * kKs / kThreads;   // 8
  double ra[kPer], rb[kPer];
  const int rc = threadIdx.x % kKs, rr = threadIdx.x / kKs;
  auto load = [&](int k0) __attribute__((always_inline)) {
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int r = rr + (kThreads / kKs) * u;
      const int gi = ti * kTile + r, gj = tj * kTile + r;
      ra[u] = gi < Nb ? Q[(long long)gi * d + k0 + rc] : 0.0;
      rb[u] = gj < Nb ? K[(long long)gj * d + k0 + rc] : 0.0;
    }
  };
  load(0);
  for (int k0 = 0; k0 < d; k0 += kKs) {
    __syncthreads();
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int r = rr + (kThreads / kKs) * u;
      As[r * kLd + rc] = ra[u];
      Bs[r * kLd + rc] = rb[u];
    }
    __syncthreads();
    if (k0 + kKs < d) load(k0 + kKs);
#pragma unroll
    for (int kk = 0; kk < kKs; kk += 4) {
      double a[2], bb[2];
#pragma unroll
      for (int m = 0; m < 2; ++m)
        a[m] = As[(wi + 16 * m + lane % 16) * kLd + kk + lane / 16];
#pragma unroll
      for (int n = 0; n < 2; ++n)
        bb[n] = Bs[(wj + 16 * n + lane % 16) * kLd + kk + lane / 16];
#pragma unroll
      for (int m = 0; m < 2; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n)
          acc[m][n] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[m], bb[n], acc[m][n], 0, 0, 0);
    }
  }
  double* Z = z + (long long)bh * Nb * Nb;
#pragma unroll
  for (int m = 0; m < 2; ++m)
#pragma unroll
    for (int n = 0; n < 2; ++n)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int gi = ti * kTile + wi + 16 * m + 4 * e + lane / 16;
        const int gj = tj * kTile + wj + 16 * n + lane % 16;
        if (gi < Nb && gj < Nb) Z[(long long)gi * Nb + gj] = acc[m][n][e] / sqrt_d;
      }
}

__device__ __forceinline__ double wave_max(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v = fmax(v, __shfl_xor(v, off, 64));
  return v;
}
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int NPT>
__global__ __launch_bounds__(kThreads) void row_softmax(double* __restrict__ p,
                                                        int Nb) {
  __shared__ double red[kThreads / 64];
  double* row = p + (long long)blockIdx.x * Nb;
  double x[NPT];
  double m = -INFINITY;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = threadIdx.x + e * kThreads;
    x[e] = j < Nb ? row[j] : -INFINITY;
    m = fmax(m, x[e]);
  }
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  m = wave_max(m);
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = fmax(fmax(red[0], red[1]), fmax(red[2], red[3]));
  __syncthreads();
  double s = 0.0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = threadIdx.x + e * kThreads;
    x[e] = j < Nb ? exp(x[e] - m) : 0.0;
    s += x[e];
  }
  s = wave_sum(s);
  if (lane == 0) red[wave] = s;
  __syncthreads();
  s = (red[0] + red[1]) + (red[2] + red[3]);
  const double inv_s = 1.0 / s;     // within 1 ulp of dividing each entry
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = threadIdx.x + e * kThreads;
    if (j < Nb) row[j] = x[e] * inv_s;
  }
}

template <typename E, int D>
prism_status launch_pool(const void* q, const void* k, const int32_t* perm,
                         int B, int Hh, int N, double* qm, double* km,
                         hipStream_t stream) {
  dim3 grid(N / 64, Hh, B);
  PRISM_LAUNCH("pool_blocks", (pool_blocks<E, D>), grid, dim3(kThreads), 0, stream,
                     static_cast<const unsigned char*>(q),
                     static_cast<const unsigned char*>(k), perm, Hh, N, qm, km);
  return check_launch("pool_blocks");
}

}  // namespace

prism_status launch_pool_means(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               hipStream_t stream) {
  if (dtype == PRISM_BF16)
    return d == 128 ? launch_pool<uint16_t, 128>(q, k, perm, B, Hh, N, q_mean, k_mean, stream)
                    : launch_pool<uint16_t, 64>(q, k, perm, B, Hh, N, q_mean, k_mean, stream);
  return d == 128 ? launch_pool<float, 128>(q, k, perm, B, Hh, N, q_mean, k_mean, stream)
                  : launch_pool<float, 64>(q, k, perm, B, Hh, N, q_mean, k_mean, stream);
}

prism_status launch_pool_proxy(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               double* proxy, hipStream_t stream) {
  prism_status st = launch_pool_means(q, k, dtype, perm, B, Hh, N, d, q_mean,
                                      k_mean, stream);
  if (st != PRISM_OK) return st;

  const int Nb = N / 64;
  dim3 g2(ceil_div(Nb, kTile), ceil_div(Nb, kTile), B * Hh);
  PRISM_LAUNCH("proxy_logits", proxy_logits, g2, dim3(kThreads), 0, stream, q_mean,
                     k_mean, Nb, d, sqrt((double)d), proxy);
  st = check_launch("proxy_logits");
  if (st != PRISM_OK) return st;

  const unsigned rows = (unsigned)((long long)B * Hh * Nb);
  if (Nb <= 4 * kThreads)
    PRISM_LAUNCH("row_softmax", row_softmax<4>, dim3(rows), dim3(kThreads), 0, stream, proxy, Nb);
  else if (Nb <= 8 * kThreads)
    PRISM_LAUNCH("row_softmax", row_softmax<8>, dim3(rows), dim3(kThreads), 0, stream, proxy, Nb);
  else if (Nb <= 16 * kThreads)
    PRISM_LAUNCH("row_softmax", row_softmax<16>, dim3(rows), dim3(kThreads), 0, stream, proxy, Nb);
  else
    PRISM_LAUNCH("row_softmax", row_softmax<32>, dim3(rows), dim3(kThreads), 0, stream, proxy, Nb);
  return check_launch("row_softmax");
}

}  // namespace prism
