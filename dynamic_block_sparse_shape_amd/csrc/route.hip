// Fused routing: block proxy scores and the hybrid top-k + top-p selection
// in one kernel, without the [B, Hh, Nb, Nb] proxy matrix.
//
// The Sol-Attn abstract on the Prism paper page names computing and
// materialising proxy scores as an overhead and thresholds blocks without
// materialising the proxy map; the walk-through ("三者如何协同") runs top-k
// then the CDF rule in one gating kernel.  Here one workgroup of 1024
// threads takes R query blocks of one head:
//   1. logits z_ij = <qbar_i, kbar_j> / sqrt(d) for its R rows and every
//      column j, in fp64: thread t owns columns t + 1024 e; kbar is staged
//      through LDS in 16-deep slices of 1024 columns (128-byte rows, XOR
//      swizzle), qbar is read with wave-uniform (scalar) loads; R * NPT
//      accumulators per thread, one fp64 FMA chain each;
//   2. per row: softmax in fp64 exactly as the stage-2 kernel writes it
//      (max, exp(z - max), sum, times the reciprocal), and the stage-3
//      selection (select_core.h) on the probabilities held in registers.
// kbar of a head (4.6 MB at the 2K grid) is read once per R rows, from L2
// (the workgroups of an XCD sweep the same columns in the same order); the
// logits never leave the chip.  Counts and lists equal those of the unfused
// calls except where a decision lies within fp64 rounding of a tie: the
// logits are summed in another order than the stage-2 GEMM's.
#include "select_core.h"

namespace prism {
namespace {

constexpr int kNT = 1024;
constexpr int kSlice = 16;                     // d per LDS slice (128 B)

template <int NPT, int R>
__global__ __launch_bounds__(kNT, 1) void route_rows(
    const double* __restrict__ qm, const double* __restrict__ km, int Nb,
    int d, double sqrt_d, int top_k, double tau, int32_t* __restrict__ counts,
    int32_t* __restrict__ kv_idx, int capacity) {
  // phase 1: the kbar slice (1024 rows x 128 B); phase 2: the selection
  extern __shared__ __align__(16) unsigned char dyn[];
  __shared__ double red[kNT / 64];
  sel::SelShared<kNT>& sh = *reinterpret_cast<sel::SelShared<kNT>*>(dyn);
  const long long bh = blockIdx.y;
  const int i0 = blockIdx.x * R;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const double* Q = qm + bh * Nb * (long long)d;
  const double* K = km + bh * Nb * (long long)d;

  double z[R][NPT];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < NPT; ++e) z[r][e] = 0.0;
  // query rows past Nb repeat the last row (never written out)
  int qrow[R];
#pragma unroll
  for (int r = 0; r < R; ++r) qrow[r] = min(i0 + r, Nb - 1);

  // this thread's 16-byte pieces of a slice: column (tid + 1024 i) / 8,
  // piece tid % 8; stored at the column's 128-byte row, piece slot XORed
  // with bits 2-4 of the column so that a wave's reads of one piece from
  // 8 consecutive columns hit 8 different slots
  const int piece = tid & 7;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int c0 = kNT * e;
    for (int ds = 0; ds < d; ds += kSlice) {
      __syncthreads();
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int cl = (tid + kNT * i) >> 3;
        const int col = c0 + cl;
        double2 v = {0.0, 0.0};
        if (col < Nb)
          v = *reinterpret_cast<const double2*>(K + (long long)col * d + ds + 2 * piece);
        *reinterpret_cast<double2*>(dyn + cl * 128 + ((piece ^ ((cl >> 2) & 7)) << 4)) = v;
      }
      __syncthreads();
      const unsigned char* mine = dyn + tid * 128;
      const int sw = (tid >> 2) & 7;
      double2 kv[8];
#pragma unroll
      for (int p = 0; p < 8; ++p)
        kv[p] = *reinterpret_cast<const double2*>(mine + ((p ^ sw) << 4));
      // row by row, so only one row's 16 qbar values (scalar registers)
      // are live at a time
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const double* qr = Q + (long long)qrow[r] * d + ds;
        double acc = z[r][e];
#pragma unroll
        for (int p = 0; p < 8; ++p) {
          acc = fma(qr[2 * p], kv[p].x, acc);
          acc = fma(qr[2 * p + 1], kv[p].y, acc);
        }
        z[r][e] = acc;
        __builtin_amdgcn_sched_barrier(0);
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
  }
}

template <int NPT, int R>
prism_status launch_rows(const double* qm, const double* km, int B, int Hh,
                         int Nb, int d, int top_k, double tau, int32_t* counts,
                         int32_t* kv_idx, int capacity, hipStream_t stream) {
  const size_t lds = sizeof(sel::SelShared<kNT>) > (size_t)kNT * 128
                         ? sizeof(sel::SelShared<kNT>) : (size_t)kNT * 128;
  const dim3 grid((unsigned)((Nb + R - 1) / R), (unsigned)(B * Hh));
  PRISM_LAUNCH("route_rows", (route_rows<NPT, R>), grid, dim3(kNT), lds,
               stream, qm, km, Nb, d, sqrt((double)d), top_k, tau, counts,
               kv_idx, capacity);
  return check_launch("route_rows");
}

}  // namespace

prism_status launch_route_fused(const double* q_mean, const double* k_mean,
                                int B, int Hh, int Nb, int d, int top_k,
                                double tau, int32_t* counts, int32_t* kv_idx,
                                int capacity, hipStream_t stream) {
  // R rows per workgroup: as many as the registers hold (R * NPT fp64
  // accumulators per thread), so kbar is re-read Nb / R times per head
  const int npt = (Nb + kNT - 1) / kNT;
#define PRISM_ROUTE(NPT_, R_)                                                  \
  return launch_rows<NPT_, R_>(q_mean, k_mean, B, Hh, Nb, d, top_k, tau,      \
                               counts, kv_idx, capacity, stream)
  if (npt <= 1) PRISM_ROUTE(1, 8);
  if (npt <= 2) PRISM_ROUTE(2, 8);
  if (npt <= 3) PRISM_ROUTE(3, 8);
  if (npt <= 4) PRISM_ROUTE(4, 8);
  if (npt <= 5) PRISM_ROUTE(5, 8);
  if (npt <= 6) PRISM_ROUTE(6, 4);
  PRISM_ROUTE(8, 4);
#undef PRISM_ROUTE
}

}  // namespace prism
