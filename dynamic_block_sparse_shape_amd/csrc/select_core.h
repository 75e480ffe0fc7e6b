// Hybrid top-k + top-p selection of one row by one workgroup, shared by the
// stage-3 kernel (select.hip: scores read from the proxy matrix) and the
// fused routing kernel (route.hip: scores computed in registers).
//
// Walk-through section "三者如何协同": first the k highest-scoring KV blocks,
// then more blocks in descending score order until the cumulative proxy
// mass reaches cdf_threshold (default 0.20), giving every query block its
// own budget.  Order: descending score, equal scores by lower block index.
// The mass is the running fp64 sum in that order.
//
// The row (<= 8192 fp64 scores) is spread over the workgroup's registers.
//  1. Windowed radix refinement on the fp64 bit patterns (non-negative
//     doubles order like unsigned integers).  Each pass buckets the keys of
//     a window at the top of the current band into 256 buckets of 2^s keys:
//     the first window is an eighth of an octave around the row mean (a
//     near-flat softmax row keeps most keys there); when the crossing lies
//     outside it the search continues with 16 buckets per octave below the
//     band's largest key, and each later pass takes 8 more bits.  Per-bucket
//     counts and approximate masses in LDS locate the
//     bucket where the count reaches max(k, 1) and the mass exceeds the
//     threshold by a safety margin far above any summation-order error;
//     everything above it is selected, the search continues inside it.
//  2. Fast path: once that band holds <= 64 keys and the mass above it is
//     clearly below the threshold, one wave sorts the band by (score desc,
//     index asc) in registers and a scan locates where the mass crosses the
//     threshold.  The count equals the sequential definition's whenever the
//     crossing is not within rounding reach of the threshold.
//  3. Otherwise the whole candidate prefix (<= 2048 keys) is bitonic-sorted
//     in LDS and scanned; only when the crossing is within the scan's
//     rounding bound of a tie does one lane redo the running sum one block
//     at a time.
//  4. The selection is kept as an LDS bitmap and written in ascending index
//     order (one bitmap word per thread of the first 256, prefix sum of
//     popcounts).
// Rows whose candidates do not fit the sort buffer, or whose whole mass
// lies within rounding of the threshold, take an exact slow path that
// extracts blocks one at a time in sorted order.
#pragma once

#include "prism_internal.h"

namespace prism {
namespace sel {

constexpr int kSortCap = 2048;
constexpr int kBand = 64;          // band size for the one-wave fast path
constexpr double kMassMargin = 1e-11;  // >> (n + 64) * 2^-53 for n <= 8192

// LDS state of one row's selection by a workgroup of NT threads.
template <int NT>
struct SelShared {
  static constexpr int kWaves = NT / 64;
  int hcnt[2][256];          // two histograms: one is cleared while the
  double hmass[2][256];      // other is filled
  unsigned long long ckey[kSortCap];
  int cidx[kSortCap];
  unsigned bits[256];        // 8192 bits (Nb <= 8192)
  double wsum[kWaves];
  unsigned long long wmax[kWaves];
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

// Pairwise sum / max of the per-wave partials a[0 .. n) (n a power of two):
// ((a0 + a1) + (a2 + a3)) + ... -- a fixed order.
template <int N, typename T>
__device__ __forceinline__ T tree_sum(const T* a) {
  if constexpr (N == 1) return a[0];
  else return tree_sum<N / 2>(a) + tree_sum<N / 2>(a + N / 2);
}
template <int N>
__device__ __forceinline__ unsigned long long tree_max(const unsigned long long* a) {
  if constexpr (N == 1) return a[0];
  else {
    const unsigned long long x = tree_max<N / 2>(a), y = tree_max<N / 2>(a + N / 2);
    return x > y ? x : y;
  }
}

// Selection of one row by a workgroup of NT threads: thread tid holds the
// scores of blocks tid + NT * e (e < NPT) as the bit patterns of
// non-negative doubles in key[] (0 beyond Nb).  Writes the ascending list
// to out and the count to *count_out.  Every thread of the workgroup calls
// it.  It reuses sh from its first instruction on: a caller that calls it
// again (or reads sh) in the same workgroup puts a barrier in between.
template <int NPT, int NT>
__device__ __forceinline__ void select_from_keys(
    const unsigned long long (&key)[NPT], int Nb, int top_k, double tau,
    SelShared<NT>& sh, int32_t* __restrict__ out, int32_t* count_out) {
  constexpr int kWaves = NT / 64;
  const int tid = threadIdx.x;
  const int wave = tid / 64, lane = tid % 64;
  double total = 0.0;
  unsigned long long kmax = 0ull;
#pragma unroll
  for (int e = 0; e < NPT; ++e) {
    total += __longlong_as_double((long long)key[e]);
    kmax = key[e] > kmax ? key[e] : kmax;
  }
  total = wave_sum(total);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) {
    const unsigned long long o = __shfl_xor(kmax, off, 64);
    kmax = o > kmax ? o : kmax;
  }
  if (lane == 0) {
    sh.wsum[wave] = total;
    sh.wmax[wave] = kmax;
  }
  if (NT == 256 || tid < 256) {
    sh.bits[tid] = 0u;
    sh.hcnt[0][tid] = 0;
    sh.hmass[0][tid] = 0.0;
  }
  __syncthreads();
  total = tree_sum<kWaves>(sh.wsum);
  kmax = tree_max<kWaves>(sh.wmax);

  const int kk = min(top_k, Nb);
  const int kneed = max(kk, 1);
  // mode: 0 = all blocks, 1 = sort candidates, 2 = exact slow path,
  //       3 = selection decided by the band fast path
  int mode;
  unsigned long long theta = 0ull;
  int ncand = 0;
  int c = 0;
  if (kk >= Nb || total < tau - kMassMargin) {
    mode = 0;
  } else if (total < tau + kMassMargin) {
    mode = 2;
  } else {
    // ------------------------------------- windowed radix refinement
    // The band [lo, hi] holds the crossing; keys above hi are selected
    // (cnt_above, mass_above) and keys below lo are not.  Each pass
    // histograms the window [wlo, whi] at the band's top, 256 buckets of
    // 2^s keys, counts keys in (whi, hi] without atomics and ignores keys
    // below the window.  The first window is an eighth of an octave around
    // the row mean at 1/2048 octave per bucket: a near-flat softmax row keeps
    // most of its keys there, spread over many buckets, and the crossing
    // usually falls in a bucket of <= 64 keys after this one pass.
    unsigned long long lo = 0ull, hi = kmax;
    unsigned long long whi;
    {
      const double anchor = total / (double)Nb * 1.0442737824274138;  // 2^(1/16)
      const unsigned long long ka = (unsigned long long)__double_as_longlong(anchor);
      whi = ka < hi ? ka : hi;
    }
    int s = 41;
    int cnt_above = 0, cnt_ge_lo = Nb, band_cnt = Nb;
    double mass_above = 0.0;
    mode = 2;
    for (int pass = 0; pass < 64; ++pass) {
      // histogram hb was cleared before the previous pass's last barrier;
      // clear the other one for the next pass
      const int hb = pass & 1;
      int* hcnt = sh.hcnt[hb];
      double* hmass = sh.hmass[hb];
      if (NT == 256 || tid < 256) {
        sh.hcnt[hb ^ 1][tid] = 0;
        sh.hmass[hb ^ 1][tid] = 0.0;
      }
      const unsigned long long top = whi >> s;
      const unsigned long long wraw = top >= 255ull ? ((top - 255ull) << s) : 0ull;
      const unsigned long long wlo = wraw > lo ? wraw : lo;
      const bool split = whi < hi;     // keys in (whi, hi] are counted apart
      int acnt = 0;
      double amass = 0.0;
#pragma unroll
      for (int e = 0; e < NPT; ++e) {
        const int j = tid + e * NT;
        if (j < Nb && key[e] >= wlo && key[e] <= hi) {
          const double x = __longlong_as_double((long long)key[e]);
          if (key[e] > whi) {
            ++acnt;
            amass += x;
          } else {
            const int dg = 255 - (int)(top - (key[e] >> s));
            atomicAdd(&hcnt[dg], 1);
            atomicAdd(&hmass[dg], x);
          }
        }
      }
      if (split) {
        amass = wave_sum(amass);
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) acnt += __shfl_xor(acnt, off, 64);
        if (lane == 0) {
          sh.wcnt[wave] = acnt;
          sh.wsum[wave] = amass;
        }
      }
      __syncthreads();
      if (wave == 0) {
        int c0 = cnt_above;
        double m0 = mass_above;
        if (split) {
          c0 += tree_sum<kWaves>(sh.wcnt);
          m0 += tree_sum<kWaves>(sh.wsum);
        }
        // lane l owns digits 255-4l .. 252-4l (descending)
        int c4[4];
        double m4[4];
        int lc = 0;
        double lm = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          c4[q] = hcnt[255 - 4 * lane - q];
          m4[q] = hmass[255 - 4 * lane - q];
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
        int cc = c0 + ic - lc;
        double cm = m0 + (im - lm);
        int hit = -1, hit_cum = 0, hit_above = 0;
        double hit_mabove = 0.0;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int cb = cc;
          const double mb = cm;
          cc += c4[q];
          cm += m4[q];
          if (hit < 0 && c4[q] > 0 && cc >= kneed && cm >= tau + kMassMargin) {
            hit = 255 - 4 * lane - q;
            hit_cum = cc;
            hit_above = cb;
            hit_mabove = mb;
          }
        }
        const unsigned long long bal = __ballot(hit >= 0);
        const int first = bal ? __ffsll((long long)bal) - 1 : -1;
        if (lane == 0) sh.s_int[3] = 0;   // band gather counter
        if (c0 >= kneed && m0 >= tau + kMassMargin) {
          // the crossing lies above the window, in (whi, hi]
          if (lane == 0) {
            sh.s_int[0] = 256;
            sh.s_int[1] = c0;
          }
        } else if (first >= 0) {
          if (lane == first) {
            sh.s_int[0] = hit;
            sh.s_int[1] = hit_cum;
            sh.s_int[2] = hit_above;
            sh.s_dbl[0] = hit_mabove;
          }
        } else if (lane == 63) {
          // below the window: everything down to wlo is selected
          sh.s_int[0] = -1;
          sh.s_int[2] = cc;
          sh.s_dbl[0] = cm;
        }
      }
      __syncthreads();
      const int D = sh.s_int[0];
      if (D == 256) {
        lo = whi + 1ull;
        cnt_ge_lo = sh.s_int[1];
        whi = hi;
        s = 48;
      } else if (D >= 0) {
        const unsigned long long base = top - (unsigned long long)(255 - D);
        const unsigned long long nlo = base << s;
        const unsigned long long nhi = nlo + ((1ull << s) - 1ull);
        lo = nlo > lo ? nlo : lo;
        hi = nhi < whi ? nhi : whi;
        whi = hi;
        cnt_ge_lo = sh.s_int[1];
        cnt_above = sh.s_int[2];
        mass_above = sh.s_dbl[0];
      } else {
        if (wlo <= lo) break;   // cannot happen when total >= tau + margin
        cnt_above = sh.s_int[2];
        mass_above = sh.s_dbl[0];
        // next window starts at the largest key left below this one
        const unsigned long long cap = wlo - 1ull;
        unsigned long long mk = 0ull;
#pragma unroll
        for (int e = 0; e < NPT; ++e) {
          const int j = tid + e * NT;
          if (j < Nb && key[e] >= lo && key[e] <= cap && key[e] > mk) mk = key[e];
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
          const unsigned long long o = __shfl_xor(mk, off, 64);
          mk = o > mk ? o : mk;
        }
        if (lane == 0) sh.wmax[wave] = mk;
        __syncthreads();
        hi = tree_max<kWaves>(sh.wmax);
        whi = hi;
        s = 48;
      }
      band_cnt = cnt_ge_lo - cnt_above;
      // mass above the band clearly below the threshold (the crossing lies
      // in the band) or clearly above it (the count k decides)
      const bool clear = mass_above < tau - kMassMargin ||
                         mass_above > tau + kMassMargin;
      if (!clear) break;
      if (band_cnt <= kBand) {
        mode = 3;
        break;
      }
      if (D >= 0 && D < 256) {
        if (s == 0) break;   // a run of identical keys
        s = s > 8 ? s - 8 : 0;
      }
    }
    if (mode == 3) {
      // ------------------------------------------------ band fast path
      // (the gather counter was reset by the last scan)
#pragma unroll
      for (int e = 0; e < NPT; ++e) {
        const int j = tid + e * NT;
        if (j < Nb && key[e] >= lo && key[e] <= hi) {
          const int pos = atomicAdd(&sh.s_int[3], 1);
          if (pos < kBand) {
            sh.ckey[pos] = key[e];
            sh.cidx[pos] = j;
          }
        }
      }
      __syncthreads();
      if (wave == 0) {
        unsigned long long bk = lane < band_cnt ? sh.ckey[lane] : 0ull;
        int bi = lane < band_cnt ? sh.cidx[lane] : 0x7fffffff;
        // bitonic sort over the 64 lanes: lane order = (score desc, index asc)
        for (int size = 2; size <= 64; size <<= 1) {
          for (int stride = size >> 1; stride > 0; stride >>= 1) {
            const unsigned long long ok = __shfl_xor(bk, stride, 64);
            const int oi = __shfl_xor(bi, stride, 64);
            // ascending runs (lane & size == 0) put the element that comes
            // first in the lower lane of each pair, descending runs in the
            // upper one
            const bool want_first = ((lane & stride) == 0) == ((lane & size) == 0);
            const bool take = want_first ? before(ok, oi, bk, bi) : before(bk, bi, ok, oi);
            if (take) {
              bk = ok;
              bi = oi;
            }
          }
        }
        const double x = __longlong_as_double((long long)bk);
        double incl = x;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const double o = __shfl_up(incl, off, 64);
          if (lane >= off) incl += o;
        }
        bool ok;
        int m;
        if (mass_above > tau + kMassMargin) {
          // the mass was reached above the band: only the count k is open
          ok = true;
          m = cnt_above;
        } else {
          const double run = mass_above + incl;
          const double prev = run - x;
          const unsigned long long crossed = __ballot(lane < band_cnt && run >= tau);
          const int t = crossed ? __ffsll((long long)crossed) - 1 : -1;
          const double run_t = __shfl(run, t < 0 ? 0 : t, 64);
          const double prev_t = __shfl(prev, t < 0 ? 0 : t, 64);
          ok = t >= 0 && run_t - tau > kMassMargin && tau - prev_t > kMassMargin;
          m = cnt_above + t + 1;
        }
        int take_n = 0;
        if (ok) {
          const int cc = min(Nb, max(kk, m));
          take_n = cc - cnt_above;
          if (lane == 0) sh.s_int[4] = cc;
        }
        if (lane == 0) sh.s_int[5] = ok ? 1 : 0;
        if (ok && lane < take_n && lane < band_cnt)
          atomicOr(&sh.bits[bi >> 5], 1u << (bi & 31));
      }
      __syncthreads();
      if (sh.s_int[5]) {
        c = sh.s_int[4];
        // every key above the band is selected: one bitmap word per
        // (slot, wave, half-wave), written from a ballot
#pragma unroll
        for (int e = 0; e < NPT; ++e) {
          const int j = tid + e * NT;
          const unsigned long long bal = __ballot(j < Nb && key[e] > hi);
          const int w = (e * NT + wave * 64) >> 5;
          if (lane == 0 && (unsigned)bal) atomicOr(&sh.bits[w], (unsigned)bal);
          if (lane == 32 && (unsigned)(bal >> 32))
            atomicOr(&sh.bits[w + 1], (unsigned)(bal >> 32));
        }
      } else {
        mode = 2;
      }
    }
    if (mode == 2 && cnt_ge_lo <= kSortCap) {
      theta = lo;
      ncand = cnt_ge_lo;
      mode = 1;
    }
  }

  if (mode == 0) {
    c = Nb;
    for (int w = tid; w < (Nb + 31) / 32; w += NT) {
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
      const int j = tid + e * NT;
      if (j < Nb && key[e] >= theta) {
        const int pos = atomicAdd(&sh.s_int[3], 1);
        sh.ckey[pos] = key[e];
        sh.cidx[pos] = j;
      }
    }
    __syncthreads();
    int n2 = 1;
    while (n2 < ncand) n2 <<= 1;
    for (int i = ncand + tid; i < n2; i += NT) {
      sh.ckey[i] = 0ull;
      sh.cidx[i] = 0x7fffffff;
    }
    __syncthreads();
    // ---------------------------------------------------- bitonic sort
    for (int size = 2; size <= n2; size <<= 1) {
      for (int stride = size >> 1; stride > 0; stride >>= 1) {
        for (int t = tid; t < (n2 >> 1); t += NT) {
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
    const int per = (n2 + NT - 1) / NT;
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
      for (int i = tid; i < c; i += NT)
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
        const int j = tid + e * NT;
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
      if ((bi % NT) == tid) taken |= 1u << (bi / NT);
      S += __longlong_as_double((long long)bk);
      ++cnt;
      if (cnt >= kneed && S >= tau) break;
    }
    c = cnt;
#pragma unroll
    for (int e = 0; e < NPT; ++e)
      if ((taken >> e) & 1u) {
        const int j = tid + e * NT;
        atomicOr(&sh.bits[j >> 5], 1u << (j & 31));
      }
  }
  __syncthreads();

  // ------------------------------------------ ascending compaction
  // thread w < 256 owns bitmap word w (Nb <= 8192)
  {
    const int words = (Nb + 31) / 32;
    const unsigned wd = tid < words ? sh.bits[tid] : 0u;
    const int n = __popc(wd);
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int o = __shfl_up(incl, off, 64);
      if (lane >= off) incl += o;
    }
    if (lane == 63) sh.wcnt[wave] = incl;
    __syncthreads();
    int pos = incl - n;
    for (int w = 0; w < wave; ++w) pos += sh.wcnt[w];
    unsigned rest = wd;
    while (rest) {
      out[pos++] = tid * 32 + __ffs(rest) - 1;
      rest &= rest - 1u;
    }
  }
  if (tid == 0) *count_out = c;
}

}  // namespace sel
}  // namespace prism
