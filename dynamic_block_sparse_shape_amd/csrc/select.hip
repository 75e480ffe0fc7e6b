// Stage 3: hybrid top-k + top-p (CDF) KV-block selection.
//
// One workgroup of 256 threads per proxy row; the row (<= 8192 fp64) lives
// in registers and select_core.h decides the selection.
#include "select_core.h"

namespace prism {
namespace {

using namespace sel;
constexpr int kThreads = 256;     // select_rows' workgroup

template <int NPT>
__global__ __launch_bounds__(kThreads, 4) void select_rows(
    const double* __restrict__ proxy, int Nb, int top_k, double tau,
    int32_t* __restrict__ counts, int32_t* __restrict__ kv_idx,
    int capacity) {
  __shared__ SelShared<kThreads> sh;
  const int tid = threadIdx.x;
  const long long row = blockIdx.x;
  const double* prow = proxy + row * Nb;
  // every load in flight at once: a clamped index instead of a branch per
  // load (a branch lets the compiler wait for each load before the next)
  double pv[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) pv[e] = prow[min(tid + e * kThreads, Nb - 1)];
  unsigned long long key[NPT];
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = tid + e * kThreads;
    const double p = pv[e] > 0.0 ? pv[e] : 0.0;  // probabilities; clamp -0 / NaN
    key[e] = j < Nb ? (unsigned long long)__double_as_longlong(p) : 0ull;
  }
  select_from_keys<NPT, kThreads>(key, Nb, top_k, tau, sh,
                                  kv_idx + row * (long long)capacity,
                                  counts + row);
}

}  // namespace

prism_status launch_select(const double* proxy, int B, int Hh, int Nb,
                           int top_k, double tau, int32_t* counts,
                           int32_t* kv_idx, int capacity, hipStream_t stream) {
  const unsigned rows = (unsigned)((long long)B * Hh * Nb);
  // keys per thread: the smallest instantiated count covering the row (the
  // 720p, 1080p and 2K grids need 5, 10 and 18: unused key slots still cost
  // a compare in every pass)
  const int per = (Nb + kThreads - 1) / kThreads;
#define PRISM_SELECT(NPT_)                                                     \
  PRISM_LAUNCH("select_rows", select_rows<NPT_>, dim3(rows), dim3(kThreads), 0, \
               stream, proxy, Nb, top_k, tau, counts, kv_idx, capacity)
  if (per <= 4) PRISM_SELECT(4);
  else if (per <= 6) PRISM_SELECT(6);
  else if (per <= 8) PRISM_SELECT(8);
  else if (per <= 10) PRISM_SELECT(10);
  else if (per <= 12) PRISM_SELECT(12);
  else if (per <= 16) PRISM_SELECT(16);
  else if (per <= 18) PRISM_SELECT(18);
  else if (per <= 20) PRISM_SELECT(20);
  else if (per <= 24) PRISM_SELECT(24);
  else PRISM_SELECT(32);
#undef PRISM_SELECT
  return check_launch("select_rows");
}

}  // namespace prism
