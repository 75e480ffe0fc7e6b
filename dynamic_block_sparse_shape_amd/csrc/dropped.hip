// Stage 4 variant (forward only): a pooled stand-in for the KV blocks a
// query block did not keep.
//
// The Sol-Attn abstract (listed on the Prism paper page) reuses the proxy
// scores of unselected blocks to approximate their contribution inside the
// online softmax instead of dropping them.  Reading used here: block j
// counts, for every query row of block i, as its 64 keys all scoring the
// stage-2 logit z_ij = <qbar_i, kbar_j> / sqrt(d) and all carrying the
// block's mean value vbar_j.  The stage-2 probabilities are reused as they
// are: with p_ij = exp(z_ij - L_i),
//   weight_i = sum_{j dropped} 64 exp(z_ij) = 64 exp(L_i) s_i,
//   s_i      = sum_{j dropped} p_ij,
//   value_i  = sum_{j dropped} p_ij vbar_j / s_i,
// and L_i = z_ij* - ln p_ij* at the row's largest probability (one fp64 dot
// product per row instead of the whole row of logits).
//
//   pool_values    one workgroup per (b, h, block): fp64 sum of the block's
//                  64 gathered value rows (exact for bf16), fp32 mean.
//   dropped_terms  one workgroup per (b, h, 64 query blocks): streams the 64
//                  proxy rows in slices of 32 columns (each slice is one word
//                  of the query->KV row bitmap), zeroes the kept columns,
//                  sums s_i in fp64, tracks the row maximum, and multiplies
//                  the slice by the 32 matching vbar rows on
//                  v_mfma_f32_32x32x2_f32 (fp32 operands, fp32 accumulation).
//                  HBM traffic is the proxy itself (8 Nb^2 bytes per head);
//                  vbar (Nb d 4 bytes per head) is re-read from L2.
// The forward kernel folds (drop_lse, drop_v) into its final normalisation.
#include <math.h>

#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kThreads = 256;

template <typename E>
__device__ __forceinline__ double widen(const unsigned char* p);
template <>
__device__ __forceinline__ double widen<uint16_t>(const unsigned char* p) {
  return (double)bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}
template <>
__device__ __forceinline__ double widen<float>(const unsigned char* p) {
  return (double)*reinterpret_cast<const float*>(p);
}

// vbar[bh][i][:] = mean of the 64 value rows of block i (through perm).
template <typename E, int D>
__global__ __launch_bounds__(kThreads) void pool_values(
    const unsigned char* __restrict__ v, const int32_t* __restrict__ perm,
    int Hh, int N, float* __restrict__ vbar) {
  constexpr int RB = D * (int)sizeof(E);     // bytes per row
  constexpr int TPR = RB / 16;               // threads per row (16 B each)
  constexpr int RPP = kThreads / TPR;        // rows per pass
  constexpr int EPV = 16 / (int)sizeof(E);   // elements per 16 B
  __shared__ double part[RPP][D];
  __shared__ int rows[64];
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  if (threadIdx.x < 64) rows[threadIdx.x] = perm[(long long)b * N + 64 * i + threadIdx.x];
  __syncthreads();
  const int piece = threadIdx.x % TPR, rg = threadIdx.x / TPR;
  const long long head = ((long long)b * Hh + h) * N;
  double acc[EPV];
#pragma unroll
  for (int e = 0; e < EPV; ++e) acc[e] = 0.0;
#pragma unroll
  for (int r = rg; r < 64; r += RPP) {
    const uint4 x = *reinterpret_cast<const uint4*>(v + (head + rows[r]) * RB + piece * 16);
    const unsigned char* px = reinterpret_cast<const unsigned char*>(&x);
#pragma unroll
    for (int e = 0; e < EPV; ++e) acc[e] += widen<E>(px + e * sizeof(E));
  }
#pragma unroll
  for (int e = 0; e < EPV; ++e) part[rg][piece * EPV + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    double s = 0.0;
    for (int g = 0; g < RPP; ++g) s += part[g][threadIdx.x];
    vbar[(((long long)b * Hh + h) * Nb + i) * D + threadIdx.x] = (float)(s * (1.0 / 64.0));
  }
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int kRows = 64;          // query blocks per workgroup
constexpr int kCols = 32;          // proxy columns per slice (one bitmap word)
constexpr int kRowsPerThread = kRows * kCols / kThreads;   // 8

// v_mfma_f32_32x32x2_f32 layouts (lane l, c = l % 32, h = l / 32): A[i][k]
// holds i = c, k = h; B[k][j] holds j = c, k = h; C[i][j] holds j = c and
// rows i = 8a + 4h + b in register 4a + b.
template <int D>
__global__ __launch_bounds__(kThreads) void dropped_terms(
    const double* __restrict__ proxy, const double* __restrict__ q_mean,
    const double* __restrict__ k_mean, const float* __restrict__ vbar,
    const uint32_t* __restrict__ rowbits, int Nb, int words, double sqrt_d,
    float* __restrict__ drop_lse, float* __restrict__ drop_v) {
  constexpr int TN = D / 64;                 // 32-column C tiles per wave
  constexpr int V4 = kCols * D / 4 / kThreads;   // float4 of vbar per thread
  __shared__ float As[kRows][kCols + 1];
  __shared__ __align__(16) float Bs[kCols][D + 32];
  __shared__ double s_sum[kRows], s_pmax[kRows];
  __shared__ int s_jmax[kRows];

  const long long bh = blockIdx.y;
  const int i0 = blockIdx.x * kRows;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int col = tid % kCols;               // this thread's slice column
  const int rbase = tid / kCols;             // rows rbase + 8 u
  const double* P = proxy + bh * Nb * (long long)Nb;
  const uint32_t* bits = rowbits + bh * words * (long long)Nb;
  const float* Vb = vbar + bh * Nb * (long long)D;

  double pr[kRowsPerThread];
  uint32_t wr[kRowsPerThread];
  float4 vr[V4];
  double sum[kRowsPerThread], pmax[kRowsPerThread];
  int jmax[kRowsPerThread];
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    sum[u] = 0.0;
    pmax[u] = -1.0;
    jmax[u] = 0;
  }
  auto load = [&](int sl) __attribute__((always_inline)) {
    const int j = sl * kCols + col;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const int i = i0 + rbase + 8 * u;
      const bool ok = i < Nb && j < Nb;
      pr[u] = ok ? P[(long long)i * Nb + j] : 0.0;
      wr[u] = i < Nb ? bits[(long long)sl * Nb + i] : 0u;
    }
#pragma unroll
    for (int t = 0; t < V4; ++t) {
      const int f = tid + kThreads * t;
      const int jr = sl * kCols + f / (D / 4);
      vr[t] = jr < Nb ? reinterpret_cast<const float4*>(Vb + (long long)jr * D)[f % (D / 4)]
                      : float4{0.f, 0.f, 0.f, 0.f};
    }
  };

  const int wr0 = 32 * (wave & 1), wc0 = (D / 2) * (wave >> 1);
  f32x16 acc[TN];
#pragma unroll
  for (int t = 0; t < TN; ++t) acc[t] = f32x16{};

  load(0);
  for (int sl = 0; sl < words; ++sl) {
    __syncthreads();                         // the last slice's products are done
    const int j = sl * kCols + col;
#pragma unroll
    for (int u = 0; u < kRowsPerThread; ++u) {
      const double p = pr[u];
      if (p > pmax[u]) {                     // ascending j: ties keep the first
        pmax[u] = p;
        jmax[u] = j;
      }
      const double pd = ((wr[u] >> col) & 1u) ? 0.0 : p;
      sum[u] += pd;
      As[rbase + 8 * u][col] = (float)pd;
    }
#pragma unroll
    for (int t = 0; t < V4; ++t) {
      const int f = tid + kThreads * t;
      *reinterpret_cast<float4*>(&Bs[f / (D / 4)][4 * (f % (D / 4))]) = vr[t];
    }
    __syncthreads();
    if (sl + 1 < words) load(sl + 1);        // in flight during the products
#pragma unroll
    for (int kk = 0; kk < kCols / 2; ++kk) {
      const float a = As[wr0 + (lane & 31)][2 * kk + (lane >> 5)];
#pragma unroll
      for (int t = 0; t < TN; ++t) {
        const float bv = Bs[2 * kk + (lane >> 5)][wc0 + 32 * t + (lane & 31)];
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x2f32(a, bv, acc[t], 0, 0, 0);
      }
    }
  }

  // per-row totals: the 32 threads of a row are 32 consecutive lanes
#pragma unroll
  for (int u = 0; u < kRowsPerThread; ++u) {
    double s = sum[u], pm = pmax[u];
    int jm = jmax[u];
#pragma unroll
    for (int off = 1; off < 32; off <<= 1) {
      s += __shfl_xor(s, off, 64);
      const double po = __shfl_xor(pm, off, 64);
      const int jo = __shfl_xor(jm, off, 64);
      if (po > pm || (po == pm && jo < jm)) {
        pm = po;
        jm = jo;
      }
    }
    if (col == 0) {
      s_sum[rbase + 8 * u] = s;
      s_pmax[rbase + 8 * u] = pm;
      s_jmax[rbase + 8 * u] = jm;
    }
  }
  __syncthreads();

  // drop_lse: 4 threads per row share the fp64 dot product <qbar_i, kbar_j*>
  {
    const int r = tid >> 2, part = tid & 3;
    const int i = i0 + r;
    const int ic = i < Nb ? i : Nb - 1;
    const double* qa = q_mean + (bh * Nb + ic) * (long long)D;
    const double* ka = k_mean + (bh * Nb + min(s_jmax[r], Nb - 1)) * (long long)D;
    double z = 0.0;
#pragma unroll 8
    for (int e = part; e < D; e += 4) z += qa[e] * ka[e];
    z += __shfl_xor(z, 1, 64);
    z += __shfl_xor(z, 2, 64);
    if (part == 0 && i < Nb) {
      const double s = s_sum[r];
      const double L = z / sqrt_d - log(s_pmax[r]);
      drop_lse[bh * Nb + i] = s > 0.0 ? (float)(log(64.0) + L + log(s)) : -INFINITY;
    }
  }

  // drop_v = (sum_j p_ij vbar_j) / s_i
#pragma unroll
  for (int t = 0; t < TN; ++t)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int lr = wr0 + 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
      const int i = i0 + lr;
      if (i < Nb) {
        const double s = s_sum[lr];
        drop_v[(bh * Nb + i) * (long long)D + wc0 + 32 * t + (lane & 31)] =
            s > 0.0 ? (float)((double)acc[t][r] / s) : 0.f;
      }
    }
}

template <typename E, int D>
prism_status run(const double* proxy, const double* q_mean,
                 const double* k_mean, const void* v, const int32_t* perm,
                 const int32_t* counts, const int32_t* kv_idx, int capacity,
                 int B, int Hh, int N, float* drop_lse, float* drop_v,
                 void* ws, hipStream_t stream) {
  const int Nb = N / 64;
  const int words = (Nb + 31) / 32;
  char* w8 = static_cast<char*>(ws);
  float* vbar = reinterpret_cast<float*>(w8);
  uint32_t* colbits = reinterpret_cast<uint32_t*>(
      w8 + align256((size_t)B * Hh * Nb * D * sizeof(float)));
  uint32_t* rowbits = reinterpret_cast<uint32_t*>(
      reinterpret_cast<char*>(colbits) + bitmap_bytes(B, Hh, Nb));
  PRISM_LAUNCH("pool_values", (pool_values<E, D>), dim3(Nb, Hh, B), dim3(kThreads), 0,
               stream, static_cast<const unsigned char*>(v), perm, Hh, N, vbar);
  prism_status st = check_launch("pool_values");
  if (st != PRISM_OK) return st;
  if ((st = launch_column_bitmap(counts, kv_idx, capacity, B, Hh, Nb, colbits,
                                 stream)) != PRISM_OK)
    return st;
  if ((st = launch_bitmap_transpose(colbits, B, Hh, Nb, rowbits, stream)) != PRISM_OK)
    return st;
  PRISM_LAUNCH("dropped_terms", dropped_terms<D>,
               dim3((unsigned)ceil_div(Nb, kRows), (unsigned)(B * Hh)),
               dim3(kThreads), 0, stream, proxy, q_mean, k_mean, vbar, rowbits,
               Nb, words, sqrt((double)D), drop_lse, drop_v);
  return check_launch("dropped_terms");
}

}  // namespace

size_t dropped_terms_ws_bytes(int B, int Hh, int N, int d) {
  const int Nb = N / 64;
  return align256((size_t)B * Hh * Nb * d * sizeof(float)) +
         2 * bitmap_bytes(B, Hh, Nb);
}

prism_status launch_dropped_terms(const double* proxy, const double* q_mean,
                                  const double* k_mean, const void* v,
                                  int dtype, const int32_t* perm,
                                  const int32_t* counts, const int32_t* kv_idx,
                                  int capacity, int B, int Hh, int N, int d,
                                  float* drop_lse, float* drop_v, void* ws,
                                  hipStream_t stream) {
  if (dtype == PRISM_BF16)
    return d == 128 ? run<uint16_t, 128>(proxy, q_mean, k_mean, v, perm, counts, kv_idx,
                                         capacity, B, Hh, N, drop_lse, drop_v, ws, stream)
                    : run<uint16_t, 64>(proxy, q_mean, k_mean, v, perm, counts, kv_idx,
                                        capacity, B, Hh, N, drop_lse, drop_v, ws, stream);
  return d == 128 ? run<float, 128>(proxy, q_mean, k_mean, v, perm, counts, kv_idx,
                                    capacity, B, Hh, N, drop_lse, drop_v, ws, stream)
                  : run<float, 64>(proxy, q_mean, k_mean, v, perm, counts, kv_idx,
                                   capacity, B, Hh, N, drop_lse, drop_v, ws, stream);
}

}  // namespace prism
