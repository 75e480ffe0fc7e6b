// Fused routing: block proxy scores and the hybrid top-k + top-p selection
// in one kernel, without the [B, Hh, Nb, Nb] proxy matrix.
//
// The Sol-Attn abstract on the Prism paper page names computing and
// materialising proxy scores as an overhead and thresholds blocks without
// materialising the proxy map; the walk-through ("三者如何协同") runs top-k
// then the CDF rule in one gating kernel.
//
//   kbar_pairs   kbar [bh][Nb][d] -> [bh][d/2][Nb][2] (workspace): a
//                column's d-pair is then one 16-byte load whose neighbours
//                in the wave are the neighbouring columns (fully coalesced).
//   route_rows   one workgroup of 1024 threads per R query blocks of a
//                head (R = 8 up to 5120 blocks, 4 above):
//     1. logits z_ij = <qbar_i, kbar_j> / sqrt(d) for its R rows and every
//        column j, in fp64: thread t owns columns t + 1024 e and streams
//        their kbar pairs straight from memory (L2: the workgroups of an
//        XCD walk the same head), qbar comes from LDS (broadcast reads);
//        R * NPT accumulators per thread, one FMA chain each;
//     2. per row: softmax in fp64 exactly as the stage-2 kernel writes it
//        (max, exp(z - max), sum, times the reciprocal), and the stage-3
//        selection (select_core.h) on the probabilities in registers.
//   kbar of a head (4.6 MB at the 2K grid) is read once per R rows; the
//   logits never leave the chip.  Counts and lists
//   equal those of the unfused calls except where a decision lies within
//   fp64 rounding of a tie (the logits are summed in another order than
//   the stage-2 GEMM's).
#include "select_core.h"

namespace prism {
namespace {

constexpr int kNT = 1024;

__global__ __launch_bounds__(256) void kbar_pairs(const double* __restrict__ km,
                                                  int Nb, int d,
                                                  double* __restrict__ kt) {
  const long long bh = blockIdx.y;
  const long long idx = (long long)blockIdx.x * 256 + threadIdx.x;   // (j, m)
  const int half = d / 2;
  if (idx >= (long long)Nb * half) return;
  const int j = (int)(idx / half), m = (int)(idx % half);
  const double2 v = *reinterpret_cast<const double2*>(km + (bh * Nb + j) * d + 2 * m);
  *reinterpret_cast<double2*>(kt + ((bh * half + m) * Nb + j) * 2) = v;
}

template <int NPT, int R>
__global__ __launch_bounds__(kNT, 1) void route_rows(
    const double* __restrict__ qm, const double* __restrict__ kt, int Nb,
    int d, double sqrt_d, int top_k, double tau, int32_t* __restrict__ counts,
    int32_t* __restrict__ kv_idx, int capacity) {
  __shared__ sel::SelShared<kNT> sh;
  __shared__ double red[kNT / 64];
  __shared__ __align__(16) double sq[R][128];
  const long long bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = d / 2;
  const double* Q = qm + bh * Nb * (long long)d;
  const double2* KT = reinterpret_cast<const double2*>(kt) + bh * half * (long long)Nb;

  double z[R][NPT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < NPT; ++e) z[r][e] = 0.0;
  // the R query rows in LDS (rows past Nb repeat the last one, never
  // written out); every lane reads the same address (broadcast)
  for (int t = tid; t < R * d; t += kNT) {
    const int r = t / d, c = t % d;
    sq[r][c] = Q[(long long)min(i0 + r, Nb - 1) * d + c];
  }
  __syncthreads();

#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = tid + kNT * e;
    if (j < Nb) {
      const double2* col = KT + j;
#pragma unroll 4
      for (int m = 0; m < half; ++m) {
        const double2 kv = col[(long long)m * Nb];
#pragma unroll
        for (int r = 0; r < R; ++r) {
          const double2 q2 = *reinterpret_cast<const double2*>(&sq[r][2 * m]);
          z[r][e] = fma(q2.x, kv.x, z[r][e]);
          z[r][e] = fma(q2.y, kv.y, z[r][e]);
        }
      }
    }
  }

  for (int r = 0; r < R; ++r) {
    const int i = i0 + r;
    if (i >= Nb) break;                        // uniform across the group
    // softmax of row i, as the stage-2 row kernel computes it
    double x[NPT];
    double m = -INFINITY;
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int j = tid + kNT * e;
      x[e] = j < Nb ? z[r][e] / sqrt_d : -INFINITY;
      m = fmax(m, x[e]);
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) m = fmax(m, __shfl_xor(m, off, 64));
    __syncthreads();
    if (lane == 0) red[wave] = m;
    __syncthreads();
    m = red[0];
#pragma unroll
    for (int w = 1; w < kNT / 64; ++w) m = fmax(m, red[w]);
    double s = 0.0;
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int j = tid + kNT * e;
      x[e] = j < Nb ? exp(x[e] - m) : 0.0;
      s += x[e];
    }
    s = sel::wave_sum(s);
    __syncthreads();
    if (lane == 0) red[wave] = s;
    __syncthreads();
    s = sel::tree_sum<kNT / 64>(red);
    const double inv_s = 1.0 / s;
    unsigned long long key[NPT];
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int j = tid + kNT * e;
      const double p = j < Nb ? x[e] * inv_s : 0.0;
      key[e] = (unsigned long long)__double_as_longlong(p > 0.0 ? p : 0.0);
    }
    const long long row = bh * Nb + i;
    sel::select_from_keys<NPT, kNT>(key, Nb, top_k, tau, sh,
                                    kv_idx + row * (long long)capacity,
                                    counts + row);
    __syncthreads();     // sh is reused by the next row's selection
  }
}

template <int NPT, int R>
prism_status launch_rows(const double* qm, const double* kt, int B, int Hh,
                         int Nb, int d, int top_k, double tau, int32_t* counts,
                         int32_t* kv_idx, int capacity, hipStream_t stream) {
  const dim3 grid((unsigned)((Nb + R - 1) / R), (unsigned)(B * Hh));
  PRISM_LAUNCH("route_rows", (route_rows<NPT, R>), grid, dim3(kNT), 0, stream,
               qm, kt, Nb, d, sqrt((double)d), top_k, tau, counts, kv_idx,
               capacity);
  return check_launch("route_rows");
}

}  // namespace

size_t route_fused_ws_bytes(int B, int Hh, int Nb, int d) {
  return align256((size_t)B * Hh * Nb * d * sizeof(double));
}

prism_status launch_route_fused(const double* q_mean, const double* k_mean,
                                int B, int Hh, int Nb, int d, int top_k,
                                double tau, int32_t* counts, int32_t* kv_idx,
                                int capacity, void* ws, hipStream_t stream) {
  double* kt = static_cast<double*>(ws);
  const long long pairs = (long long)Nb * (d / 2);
  PRISM_LAUNCH("kbar_pairs", kbar_pairs,
               dim3((unsigned)((pairs + 255) / 256), (unsigned)(B * Hh)),
               dim3(256), 0, stream, k_mean, Nb, d, kt);
  prism_status st = check_launch("kbar_pairs");
  if (st != PRISM_OK) return st;
  // R rows per workgroup: as many as the registers hold (R * NPT fp64
  // accumulators per thread); kbar is read Nb / R times per head
  const int npt = (Nb + kNT - 1) / kNT;
#define PRISM_ROUTE(NPT_, R_)                                                  \
  return launch_rows<NPT_, R_>(q_mean, kt, B, Hh, Nb, d, top_k, tau, counts,  \
                               kv_idx, capacity, stream)
  if (npt <= 1) PRISM_ROUTE(1, 8);
  if (npt <= 2) PRISM_ROUTE(2, 8);
  if (npt <= 3) PRISM_ROUTE(3, 8);
  if (npt <= 5) PRISM_ROUTE(5, 8);
  if (npt <= 6) PRISM_ROUTE(6, 4);
  PRISM_ROUTE(8, 4);
#undef PRISM_ROUTE
}

}  // namespace prism
