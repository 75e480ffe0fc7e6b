// Stage 3: hybrid top-k + top-p (CDF) KV-block selection.
//
// Walk-through section "三者如何协同": first the k highest-scoring KV blocks,
// then more blocks in descending score order until the cumulative proxy
// mass reaches cdf_threshold (default 0.20), giving every query block its
// own budget.  Order: descending score, equal scores by lower block index.
// The mass is the running fp64 sum in that order.
//
// One workgroup per proxy row; the row (<= 8192 fp64) lives in registers.
//  1. Radix refinement on the fp64 bit patterns (non-negative doubles order
//     like unsigned integers), 8 bits per pass, with per-bucket counts and
//     approximate masses in LDS, narrows the candidates to the smallest
//     prefix of buckets whose count reaches max(k, 1) and whose mass exceeds
//     the threshold by a safety margin far above any summation-order error.
//     That set is a prefix of the sorted order and holds the answer.
//  2. The <= 2048 candidates are bitonic-sorted in LDS by (score desc,
//     index asc).
//  3. A parallel scan of the sorted scores locates where the mass crosses
//     the threshold; only when the crossing is within the scan's rounding
//     bound of a tie does one lane redo the running sum one block at a time,
//     so the count always equals that of the sequential definition.
//  4. The first c sorted blocks are marked in an LDS bitmap and written in
//     ascending index order with ballot / popcount compaction.
// Rows whose candidates do not fit the sort buffer, or whose whole mass
// lies within rounding of the threshold, take an exact slow path that
// extracts blocks one at a time in sorted order.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / 64;
constexpr int kSortCap = 2048;
constexpr double kMassMargin = 1e-11;  // >> (n + 64) * 2^-53 for n <= 8192

struct SelShared {
  int hcnt[256];
  double hmass[256];
  unsigned long long ckey[kSortCap];
  int cidx[kSortCap];
  unsigned bits[8192 / 32];
  double wsum[kWaves];
  int wcnt[kWaves];
  int s_int[8];
  double s_dbl[8];
  unsigned long long s_u64[2];
};

__device__ __forceinline__ bool before(unsigned long long ka, int ia,
                                       unsigned long long kb, int ib) {
  return ka > kb || (ka == kb && ia < ib);
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <int NPT>
__global__ __launch_bounds__(kThreads) void select_rows(
    const double* __restrict__ proxy, int Nb, int top_k, double tau,
    int32_t* __restrict__ counts, int32_t* __restrict__ kv_idx,
    int capacity) {
  __shared__ SelShared sh;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  const long long row = blockIdx.x;
  const double* prow = proxy + row * Nb;
  int32_t* out = kv_idx + row * (long long)capacity;

  unsigned long long key[NPT];
  double total = 0.0;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    const int j = tid + e * kThreads;
    double p = j < Nb ? prow[j] : 0.0;
    p = p > 0.0 ? p : 0.0;  // scores are probabilities; clamp -0 / NaN
    key[e] = j < Nb ? (unsigned long long)__double_as_longlong(p) : 0ull;
    total += p;
  }
  total = wave_sum(total);
  if (lane == 0) sh.wsum[wave] = total;
  for (int w = tid; w < (Nb + 31) / 32; w += kThreads) sh.bits[w] = 0u;
  __syncthreads();
  total = (sh.wsum[0] + sh.wsum[1]) + (sh.wsum[2] + sh.wsum[3]);

  const int kk = min(top_k, Nb);
  const int kneed = max(kk, 1);
  // mode: 0 = all blocks, 1 = sort candidates, 2 = exact slow path
  int mode;
  unsigned long long theta = 0ull;
  int ncand = 0;
  if (kk >= Nb || total < tau - kMassMargin) {
    mode = 0;
  } else if (total < tau + kMassMargin) {
    mode = 2;
  } else {
    // ---------------------------------------------- radix refinement
    unsigned long long prefix = 0ull, mask = 0ull;
    int cnt_above = 0;
    double mass_above = 0.0;
    mode = 2;
    for (int shift = 56; shift >= 0; shift -= 8) {
      sh.hcnt[tid] = 0;
      sh.hmass[tid] = 0.0;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < NPT; ++e) {
        const int j = tid + e * kThreads;
        if (j < Nb && (key[e] & mask) == prefix) {
          const int dg = (int)((key[e] >> shift) & 0xffull);
          atomicAdd(&sh.hcnt[dg], 1);
          atomicAdd(&sh.hmass[dg], __longlong_as_double((long long)key[e]));
        }
      }
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending)
        int c4[4];
        double m4[4];
        int lc = 0;
        double lm = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c4[q] = sh.hcnt[255 - 4 * lane - q];
          m4[q] = sh.hmass[255 - 4 * lane - q];
          lc += c4[q];
          lm += m4[q];
        }
        // exclusive prefix over lanes (higher digits first)
        int ic = lc;
        double im = lm;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const int oc = __shfl_up(ic, off, 64);
          const double om = __shfl_up(im, off, 64);
          if (lane >= off) {
            ic += oc;
            im += om;
          }
        }
        int cc = cnt_above + ic - lc;
        double cm = mass_above + (im - lm);
        int hit = -1;
        int hit_cum = 0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          cc += c4[q];
          cm += m4[q];
          if (hit < 0 && c4[q] > 0 && cc >= kneed && cm >= tau + kMassMargin) {
            hit = 255 - 4 * lane - q;
            hit_cum = cc;
          }
        }
        const unsigned long long bal = __ballot(hit >= 0);
        const int first = bal ? __ffsll((long long)bal) - 1 : -1;
        if (lane == first) {
          sh.s_int[0] = hit;
          sh.s_int[1] = hit_cum;
        }
        if (first < 0 && lane == 0) sh.s_int[0] = -1;
      }
      __syncthreads();
      const int D = sh.s_int[0];
      const int cum = sh.s_int[1];
      __syncthreads();
      if (D < 0) {  // cannot happen when total >= tau + margin; be safe
        mode = 2;
        break;
      }
      if (cum <= kSortCap) {
        theta = prefix | ((unsigned long long)D << shift);
        ncand = cum;
        mode = 1;
        break;
      }
      if (shift == 0) {  // more than kSortCap identical keys
        mode = 2;
        break;
      }
      // refine inside bucket D: everything above it is in for good
      if (tid == 0) {
        int ca = 0;
        double ma = 0.0;
        for (int dg = 255; dg > D; --dg) {
          ca += sh.hcnt[dg];
          ma += sh.hmass[dg];
        }
        sh.s_int[2] = ca;
        sh.s_dbl[0] = ma;
      }
      __syncthreads();
      cnt_above += sh.s_int[2];
      mass_above += sh.s_dbl[0];
      prefix |= (unsigned long long)D << shift;
      mask |= 0xffull << shift;
      __syncthreads();
    }
  }

  int c = 0;
  if (mode == 0) {
    c = Nb;
    for (int w = tid; w < (Nb + 31) / 32; w += kThreads) {
      const int lo = w * 32;
      const int nbit = min(32, Nb - lo);
      sh.bits[w] = nbit == 32 ? 0xffffffffu : ((1u << nbit) - 1u);
    }
  } else if (mode == 1) {
    // ------------------------------------------------ gather candidates
    if (tid == 0) sh.s_int[3] = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < NPT; ++e) {
      const int j = tid + e * kThreads;
      if (j < Nb && key[e] >= theta) {
        const int pos = atomicAdd(&sh.s_int[3], 1);
        sh.ckey[pos] = key[e];
        sh.cidx[pos] = j;
      }
    }
    __syncthreads();
    int n2 = 1;
    while (n2 < ncand) n2 <<= 1;
    for (int i = ncand + tid; i < n2; i += kThreads) {
      sh.ckey[i] = 0ull;
      sh.cidx[i] = 0x7fffffff;
    }
    __syncthreads();
    // ---------------------------------------------------- bitonic sort
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (n2 >> 1); t += kThreads) {
          const int i = 2 * t - (t & (stride - 1));
          const int j = i + stride;
          const unsigned long long ka = sh.ckey[i], kb = sh.ckey[j];
          const int ia = sh.cidx[i], ib = sh.cidx[j];
          const bool up = (i & size) == 0;
          const bool sw = up ? before(kb, ib, ka, ia) : before(ka, ia, kb, ib);
          if (sw) {
            sh.ckey[i] = kb; sh.ckey[j] = ka;
            sh.cidx[i] = ib; sh.cidx[j] = ia;
          }
        }
        __syncthreads();
      }
    }
    // --------------------------------------- locate the CDF crossing
    const int per = (n2 + kThreads - 1) / kThreads;
    const int lo = tid * per;
    double local = 0.0;
    for (int i = lo; i < min(lo + per, ncand); ++i)
      local += __longlong_as_double((long long)sh.ckey[i]);
    double incl = local;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) sh.wsum[wave] = incl;
    if (tid == 0) {
      sh.s_int[4] = 0x7fffffff;
      sh.s_int[5] = 0;  // ambiguous flag
    }
    __syncthreads();
    double excl = incl - local;
    for (int w = 0; w < wave; ++w) excl += sh.wsum[w];
    if (excl < tau) {  // only the thread holding the first crossing looks
      double run = excl;
      for (int i = lo; i < min(lo + per, ncand); ++i) {
        const double prev = run;
        run += __longlong_as_double((long long)sh.ckey[i]);
        if (run >= tau) {
          atomicMin(&sh.s_int[4], i + 1);
          // too close to call from the scan?  (either side of the crossing)
          if (run - tau <= kMassMargin || tau - prev <= kMassMargin)
            sh.s_int[5] = 1;
          break;
        }
      }
    }
    __syncthreads();
    int mstar = sh.s_int[4];
    // crossing within rounding reach of the threshold: recount exactly
    if (mstar == 0x7fffffff || sh.s_int[5]) {
      if (tid == 0) {
        double S = 0.0;
        int m = 0x7fffffff;
        for (int i = 0; i < ncand; ++i) {
          S += __longlong_as_double((long long)sh.ckey[i]);
          if (S >= tau) {
            m = i + 1;
            break;
          }
        }
        sh.s_int[6] = m;
      }
      __syncthreads();
      mstar = sh.s_int[6];
    }
    if (mstar == 0x7fffffff) {
      mode = 2;  // candidates did not reach the threshold: exact slow path
    } else {
      c = min(Nb, max(kk, mstar));
      for (int i = tid; i < c; i += kThreads)
        atomicOr(&sh.bits[sh.cidx[i] >> 5], 1u << (sh.cidx[i] & 31));
    }
  }

  if (mode == 2) {
    // ------------------------------------------- exact slow extraction
    unsigned taken = 0u;
    double S = 0.0;
    int cnt = 0;
    while (cnt < Nb) {
      unsigned long long bk = 0ull;
      int bi = 0x7fffffff;
#pragma unroll
      for (int e = 0; e < NPT; ++e) {
        const int j = tid + e * kThreads;
        if (j < Nb && !((taken >> e) & 1u) && before(key[e], j, bk, bi)) {
          bk = key[e];
          bi = j;
        }
      }
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) {
        const unsigned long long ok = __shfl_xor(bk, off, 64);
        const int oi = __shfl_xor(bi, off, 64);
        if (before(ok, oi, bk, bi)) {
          bk = ok;
          bi = oi;
        }
      }
      if (lane == 0) {
        sh.ckey[wave] = bk;
        sh.cidx[wave] = bi;
      }
      __syncthreads();
      bk = sh.ckey[0];
      bi = sh.cidx[0];
      for (int w = 1; w < kWaves; ++w)
        if (before(sh.ckey[w], sh.cidx[w], bk, bi)) {
          bk = sh.ckey[w];
          bi = sh.cidx[w];
        }
      __syncthreads();
      if ((bi % kThreads) == tid) taken |= 1u << (bi / kThreads);
      S += __longlong_as_double((long long)bk);
      ++cnt;
      if (cnt >= kneed && S >= tau) break;
    }
    c = cnt;
#pragma unroll
    for (int e = 0; e < NPT; ++e)
      if ((taken >> e) & 1u) {
        const int j = tid + e * kThreads;
        atomicOr(&sh.bits[j >> 5], 1u << (j & 31));
      }
  }
  __syncthreads();

  // ------------------------------------------ ascending compaction
  int base = 0;
  for (int j0 = 0; j0 < Nb; j0 += kThreads) {
    const int j = j0 + tid;
    const bool f = j < Nb && ((sh.bits[j >> 5] >> (j & 31)) & 1u);
    const unsigned long long bal = __ballot(f);
    const int before_in_wave = __popcll(bal & ((1ull << lane) - 1ull));
    if (lane == 0) sh.wcnt[wave] = __popcll(bal);
    __syncthreads();
    int off = base;
    for (int w = 0; w < wave; ++w) off += sh.wcnt[w];
    if (f) out[off + before_in_wave] = j;
    base += (sh.wcnt[0] + sh.wcnt[1]) + (sh.wcnt[2] + sh.wcnt[3]);
    __syncthreads();
  }
  if (tid == 0) counts[row] = c;
}

}  // namespace

prism_status launch_select(const double* proxy, int B, int Hh, int Nb,
                           int top_k, double tau, int32_t* counts,
                           int32_t* kv_idx, int capacity, hipStream_t stream) {
  const unsigned rows = (unsigned)((long long)B * Hh * Nb);
  if (Nb <= 4 * kThreads)
    PRISM_LAUNCH("select_rows", select_rows<4>, dim3(rows), dim3(kThreads), 0, stream,
                       proxy, Nb, top_k, tau, counts, kv_idx, capacity);
  else if (Nb <= 8 * kThreads)
    PRISM_LAUNCH("select_rows", select_rows<8>, dim3(rows), dim3(kThreads), 0, stream,
                       proxy, Nb, top_k, tau, counts, kv_idx, capacity);
  else if (Nb <= 16 * kThreads)
    PRISM_LAUNCH("select_rows", select_rows<16>, dim3(rows), dim3(kThreads), 0, stream,
                       proxy, Nb, top_k, tau, counts, kv_idx, capacity);
  else
    PRISM_LAUNCH("select_rows", select_rows<32>, dim3(rows), dim3(kThreads), 0, stream,
                       proxy, Nb, top_k, tau, counts, kv_idx, capacity);
  return check_launch("select_rows");
}

}  // namespace prism
