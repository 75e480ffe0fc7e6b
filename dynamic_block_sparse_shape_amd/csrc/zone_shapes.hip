// Stage 1: macro-zone statistics, block-shape choice and token permutation.
//
// README "Overview" (Tencent-Hunyuan/Prism): per macro-zone, the video
// feature variance along the channel says how content varies directionally
// and the audio-to-video feature norms say how strongly audio drives the
// region; the zone gets finer blocks along axes of rapid variation and
// strong coupling.  Walk-through section "一个巧妙的联动": the audio signal is
// the per-token L2 norm of the unscaled a2v bridge residual.  Walk-through
// "三者如何协同": one of 13 candidate shapes per zone.
//
// Kernels (all HBM-streaming except the tiny finaliser):
//   zone_feat_dev   one workgroup per (zone, 64-byte channel slice): stages
//                   the zone's slice (<= 512 tokens x 64 B = 32 KB) in LDS
//                   with 16-byte loads, then sums squared deviations from
//                   the line mean along T, H and W lines in fp64 (bf16:
//                   exact per-line sums and sums of squares, two channels
//                   per LDS read).  32 KB of LDS lets four workgroups share
//                   a CU, so one's loads overlap the others' arithmetic.
//   token_rms       one wave per token: ||dh||_2 / sqrt(C) in fp64.
//   zone_finalize   one workgroup per zone: reduces the slices in a fixed
//                   order, adds the a2v-norm term, takes the cost argmin and
//                   writes the zone's part of perm / inv_perm.
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kThreads = 256;
constexpr int kRowBytes = 64;         // bytes of one token's channel slice
constexpr int kMaxZoneTokens = 512;   // zone extents <= 8

struct ZoneBox {
  int t0, h0, w0, Lt, Lh, Lw;
};

__device__ __forceinline__ ZoneBox zone_box(const ZoneGeom& g, int z) {
  int zw = z % g.nzw;
  int zh = (z / g.nzw) % g.nzh;
  int zt = z / (g.nzw * g.nzh);
  ZoneBox b;
  b.t0 = zt * g.zt; b.h0 = zh * g.zh; b.w0 = zw * g.zw;
  b.Lt = min(g.zt, g.T - b.t0);
  b.Lh = min(g.zh, g.H - b.h0);
  b.Lw = min(g.zw, g.W - b.w0);
  return b;
}

// Slot of the zone's first token: zones before it in raster order cover
// whole T-slabs, then whole H-rows of its slab, then whole W-runs.
__device__ __forceinline__ long long zone_slot0(const ZoneGeom& g,
                                                const ZoneBox& b) {
  return (long long)b.t0 * g.H * g.W + (long long)b.Lt * b.h0 * g.W +
         (long long)b.Lt * b.Lh * b.w0;
}

template <typename E>
__device__ __forceinline__ double load_elem(const unsigned char* p);
template <>
__device__ __forceinline__ double load_elem<uint16_t>(const unsigned char* p) {
  return (double)bf16_to_f32(*reinterpret_cast<const uint16_t*>(p));
}
template <>
__device__ __forceinline__ double load_elem<float>(const unsigned char* p) {
  return (double)*reinterpret_cast<const float*>(p);
}

// Sum over the lines of one axis of sum_i (x_i - mean)^2 for a channel whose
// zone values sit in LDS at base + token * kRowBytes.
template <typename E>
__device__ __forceinline__ double line_dev(const unsigned char* base, int L,
                                           int first_tok, int stride) {
  double x[8];
  double s = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < L) {
      x[i] = load_elem<E>(base + (first_tok + i * stride) * kRowBytes);
      s += x[i];
    }
  }
  const double m = s / (double)L;
  double dv = 0.0;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    if (i < L) {
      const double e = x[i] - m;
      dv += e * e;
    }
  }
  return dv;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

template <typename E>
__global__ __launch_bounds__(kThreads) void zone_feat_dev(
    const unsigned char* __restrict__ feat, ZoneGeom g, int C,
    int n_slices, double* __restrict__ partial) {
  constexpr int CH = kRowBytes / (int)sizeof(E);  // channels per slice
  __shared__ __align__(16) unsigned char tile[kMaxZoneTokens * kRowBytes];
  __shared__ double red[3][kThreads / 64];

  // the two 64-byte halves of a 128-byte line go to workgroups 8 apart in
  // launch order (workgroups are dealt round-robin to the 8 XCDs): the same
  // XCD at about the same time, so the second half is an L2 hit and every
  // line is fetched once
  const int bx = blockIdx.x;
  const int slice = (bx / 16) * 16 + 15 < n_slices
                        ? (bx / 16) * 16 + 2 * (bx % 8) + (bx / 8) % 2
                        : bx;
  const int z = blockIdx.y;
  const int b = blockIdx.z;
  const ZoneBox zb = zone_box(g, z);
  const int nt = zb.Lt * zb.Lh * zb.Lw;
  const long long N = (long long)g.T * g.H * g.W;
  const long long rowB = (long long)C * sizeof(E);
  const int c0 = slice * CH;
  const int valid_bytes = min(CH, C - c0) * (int)sizeof(E);  // multiple of 16

  // stage: kPieces threads per token row, 16 bytes each; every load of the
  // thread is issued before the first LDS store, so a workgroup keeps its
  // whole slice (up to 32 KB) in flight
  constexpr int kPieces = kRowBytes / 16;
  constexpr int kIter = kMaxZoneTokens * kPieces / kThreads;
  const unsigned char* fb = feat + (long long)b * N * rowB + (long long)c0 * sizeof(E);
  // thread tid covers piece tid % kPieces of tokens tid / kPieces + kStep * it.
  // The token's (h, w) place in the zone and its byte offset in the feature
  // map are computed once and then advanced by kStep tokens in the zone's
  // mixed radix (Lt, Lh, Lw), with carries: no division or multiplication
  // per load.
  constexpr int kStep = kThreads / kPieces;
  const int piece = threadIdx.x % kPieces;
  const int plane = zb.Lh * zb.Lw;
  int tok = threadIdx.x / kPieces;
  const int lt0 = tok / plane;
  int lh = (tok - lt0 * plane) / zb.Lw;
  int lw = tok - lt0 * plane - lh * zb.Lw;
  const int dt = kStep / plane;
  const int dh = (kStep - dt * plane) / zb.Lw;
  const int dw = kStep - dt * plane - dh * zb.Lw;
  const long long RW = rowB, RH = (long long)g.W * rowB, RT = (long long)g.H * RH;
  const long long step = dw * RW + dh * RH + dt * RT;   // kStep tokens, no carry
  const long long carry_w = RH - zb.Lw * RW;            // w wraps: next h
  const long long carry_h = RT - zb.Lh * RH;            // h wraps: next t
  long long gofs = (((long long)(zb.t0 + lt0) * g.H + (zb.h0 + lh)) * g.W + zb.w0 + lw) * rowB +
                   piece * 16;
  uint4 v[kIter];
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    v[it] = make_uint4(0, 0, 0, 0);
    if (tok < nt && piece * 16 < valid_bytes)
      v[it] = *reinterpret_cast<const uint4*>(fb + gofs);
    tok += kStep;
    lw += dw;
    const bool cw = lw >= zb.Lw;
    lw -= cw ? zb.Lw : 0;
    lh += dh + (cw ? 1 : 0);
    const bool ch = lh >= zb.Lh;
    lh -= ch ? zb.Lh : 0;
    gofs += step + (cw ? carry_w : 0ll) + (ch ? carry_h : 0ll);
  }
#pragma unroll
  for (int it = 0; it < kIter; ++it) {
    const int i = threadIdx.x + it * kThreads;
    if (i / kPieces < nt)
      *reinterpret_cast<uint4*>(tile + (i / kPieces) * kRowBytes + (i % kPieces) * 16) = v[it];
  }
  __syncthreads();

  // Sums of squared deviations along T, H, W lines, summed over the
  // slice's channels, reduced over the workgroup.
  double dT = 0.0, dH = 0.0, dW = 0.0;
  if constexpr (sizeof(E) == 2) {
    // bf16: the squared deviation of a line of L <= 8 values is
    // (L q - s^2) / L with s the sum and q the sum of squares.  With 8-bit
    // significands, s, q, L q and s^2 are exact in fp64 whenever the line's
    // values lie within 2^17 of each other in magnitude -- the near-constant
    // lines where the subtraction cancels -- so each numerator is exact and
    // rounding enters only where numerators are summed and in one division
    // per axis (all lines along an axis of a zone share L), for any L (also
    // where 1 / L is not a power of two); a line with a wider spread has a
    // deviation of the order of q itself.  One LDS read per value and axis,
    // two channels per 32-bit read.
    constexpr int CP = kRowBytes / 4;          // channel pairs per slice
    constexpr int G = kThreads / CP;           // line groups
    const int cp = threadIdx.x % CP, grp = threadIdx.x / CP;
    const unsigned char* base = tile + cp * 4;
    auto line = [&](int tok0, int stride, int L) __attribute__((always_inline)) -> double {
      double s0 = 0.0, s1 = 0.0, q0 = 0.0, q1 = 0.0;
      for (int i = 0; i < L; ++i) {
        const uint32_t u =
            *reinterpret_cast<const uint32_t*>(base + (tok0 + i * stride) * kRowBytes);
        const double x0 = (double)__uint_as_float(u << 16);
        const double x1 = (double)__uint_as_float(u & 0xffff0000u);
        s0 += x0;
        s1 += x1;
        q0 = fma(x0, x0, q0);
        q1 = fma(x1, x1, q1);
      }
      const double Ld = (double)L;
      return (Ld * q0 - s0 * s0) + (Ld * q1 - s1 * s1);   // L x deviation
    };
    for (int l = grp; l < zb.Lt * zb.Lh; l += G)          // W lines (lt, lh)
      dW += line(l * zb.Lw, 1, zb.Lw);
    for (int l = grp; l < zb.Lt * zb.Lw; l += G)          // H lines (lt, lw)
      dH += line((l / zb.Lw) * zb.Lh * zb.Lw + l % zb.Lw, zb.Lw, zb.Lh);
    for (int l = grp; l < zb.Lh * zb.Lw; l += G)          // T lines (lh, lw)
      dT += line(l, zb.Lh * zb.Lw, zb.Lt);
    dW /= (double)zb.Lw;
    dH /= (double)zb.Lh;
    dT /= (double)zb.Lt;
  } else {
    // fp32: two passes per line (mean, then squared deviations): wider
    // inputs do not have exact squares
    constexpr int G = kThreads / CH;
    const int c = threadIdx.x % CH;
    const int grp = threadIdx.x / CH;
    const unsigned char* base = tile + c * sizeof(E);
    for (int l = grp; l < zb.Lt * zb.Lh; l += G)          // W lines (lt, lh)
      dW += line_dev<E>(base, zb.Lw, l * zb.Lw, 1);
    for (int l = grp; l < zb.Lt * zb.Lw; l += G) {        // H lines (lt, lw)
      const int lt = l / zb.Lw, lw = l % zb.Lw;
      dH += line_dev<E>(base, zb.Lh, lt * zb.Lh * zb.Lw + lw, zb.Lw);
    }
    for (int l = grp; l < zb.Lh * zb.Lw; l += G)          // T lines (lh, lw)
      dT += line_dev<E>(base, zb.Lt, l, zb.Lh * zb.Lw);
  }

  dT = wave_sum(dT);
  dH = wave_sum(dH);
  dW = wave_sum(dW);
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  if (lane == 0) {
    red[0][wave] = dT;
    red[1][wave] = dH;
    red[2][wave] = dW;
  }
  __syncthreads();
  if (threadIdx.x < 3) {
    double s = 0.0;
    for (int w = 0; w < kThreads / 64; ++w) s += red[threadIdx.x][w];
    partial[(((long long)b * g.nZ + z) * n_slices + slice) * 3 + threadIdx.x] = s;
  }
}

// ||dh_p||_2 / sqrt(C), one wave per token, 16-byte loads.
template <typename E>
__global__ __launch_bounds__(kThreads) void token_rms(
    const unsigned char* __restrict__ a2v, long long n_tokens, int C,
    double* __restrict__ out) {
  constexpr int EPV = 16 / (int)sizeof(E);  // elements per 16-byte load
  const long long tok = (long long)blockIdx.x * (kThreads / 64) + threadIdx.x / 64;
  const int lane = threadIdx.x % 64;
  if (tok >= n_tokens) return;
  const unsigned char* row = a2v + tok * (long long)C * sizeof(E);
  const int nvec = C / EPV;
  double s = 0.0;
  for (int i = lane; i < nvec; i += 64) {
    uint4 v = *reinterpret_cast<const uint4*>(row + (long long)i * 16);
    const unsigned char* pv = reinterpret_cast<const unsigned char*>(&v);
#pragma unroll
    for (int e = 0; e < EPV; ++e) {
      const double x = load_elem<E>(pv + e * sizeof(E));
      s += x * x;
    }
  }
  s = wave_sum(s);
  if (lane == 0) out[tok] = sqrt(s) / sqrt((double)C);
}

// Cost of a shape: sum_a w_a (e_a^2 - 1) / (L_a^2 - 1), the three terms
// added smallest first so that costs equal as real numbers compare equal.
__device__ __forceinline__ double shape_cost(const double w[3], const int L[3],
                                             const Shape& s) {
  const int e[3] = {s.t, s.h, s.w};
  double t[3];
#pragma unroll
  for (int a = 0; a < 3; ++a)
    t[a] = L[a] > 1 ? w[a] * ((double)(e[a] * e[a] - 1) / (double)(L[a] * L[a] - 1))
                    : 0.0;
  // sort three values ascending
  double lo = fmin(t[0], t[1]), hi = fmax(t[0], t[1]);
  double a0 = fmin(lo, t[2]);
  double mid = fmax(lo, fmin(hi, t[2]));
  double a2 = fmax(hi, t[2]);
  return (a0 + mid) + a2;
}

__global__ __launch_bounds__(kThreads) void zone_finalize(
    ZoneGeom g, int C, int n_slices, const double* __restrict__ partial,
    const double* __restrict__ rms, double lam, int fixed_shape,
    int32_t* __restrict__ zone_shape, int32_t* __restrict__ perm,
    int32_t* __restrict__ inv_perm, double* __restrict__ zone_stats) {
  __shared__ double nrm[kMaxZoneTokens];
  __shared__ double red[3][kThreads / 64];
  __shared__ int s_sid;
  const int z = blockIdx.x;
  const int b = blockIdx.y;
  const ZoneBox zb = zone_box(g, z);
  const int nt = zb.Lt * zb.Lh * zb.Lw;
  const long long N = (long long)g.T * g.H * g.W;

  if (fixed_shape >= 0) {
    if (threadIdx.x == 0) {
      s_sid = fixed_shape;
      zone_shape[(long long)b * g.nZ + z] = fixed_shape;
    }
  } else {
    // audio term: directional variance of the RMS norm over the zone
    double uT = 0.0, uH = 0.0, uW = 0.0;
    if (rms != nullptr) {
      for (int i = threadIdx.x; i < nt; i += kThreads) {
        const int lw = i % zb.Lw, lh = (i / zb.Lw) % zb.Lh, lt = i / (zb.Lw * zb.Lh);
        const long long gtok = ((long long)(zb.t0 + lt) * g.H + (zb.h0 + lh)) * g.W + zb.w0 + lw;
        nrm[i] = rms[(long long)b * N + gtok];
      }
      __syncthreads();
      auto dev = [&](int L, int first, int stride) {
        double s = 0.0;
        for (int i = 0; i < L; ++i) s += nrm[first + i * stride];
        const double m = s / (double)L;
        double d = 0.0;
        for (int i = 0; i < L; ++i) {
          const double e = nrm[first + i * stride] - m;
          d += e * e;
        }
        return d;
      };
      for (int l = threadIdx.x; l < zb.Lt * zb.Lh; l += kThreads)
        uW += dev(zb.Lw, l * zb.Lw, 1);
      for (int l = threadIdx.x; l < zb.Lt * zb.Lw; l += kThreads)
        uH += dev(zb.Lh, (l / zb.Lw) * zb.Lh * zb.Lw + l % zb.Lw, zb.Lw);
      for (int l = threadIdx.x; l < zb.Lh * zb.Lw; l += kThreads)
        uT += dev(zb.Lt, l, zb.Lh * zb.Lw);
    }
    uT = wave_sum(uT);
    uH = wave_sum(uH);
    uW = wave_sum(uW);
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
    if (lane == 0) {
      red[0][wave] = uT;
      red[1][wave] = uH;
      red[2][wave] = uW;
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      double u[3], v[3];
      for (int a = 0; a < 3; ++a) {
        double s = 0.0;
        for (int w = 0; w < kThreads / 64; ++w) s += red[a][w];
        u[a] = s / (double)nt;
        double d = 0.0;
        const double* pp = partial + ((long long)b * g.nZ + z) * n_slices * 3;
        for (int sl = 0; sl < n_slices; ++sl) d += pp[sl * 3 + a];
        v[a] = d / ((double)C * (double)nt);
      }
      double w[3];
      for (int a = 0; a < 3; ++a) w[a] = v[a] + lam * u[a];
      const int L[3] = {zb.Lt, zb.Lh, zb.Lw};
      int best = -1;
      double bestJ = 0.0;
      for (int s = 0; s < kNumShapes; ++s) {
        if (!shape_fits(s, zb.Lt, zb.Lh, zb.Lw)) continue;
        const double J = shape_cost(w, L, shape_of(s));
        if (best < 0 || J < bestJ) {
          best = s;
          bestJ = J;
        }
      }
      s_sid = best;
      zone_shape[(long long)b * g.nZ + z] = best;
      if (zone_stats) {
        double* st = zone_stats + ((long long)b * g.nZ + z) * 6;
        st[0] = v[0]; st[1] = v[1]; st[2] = v[2];
        st[3] = u[0]; st[4] = u[1]; st[5] = u[2];
      }
    }
  }
  __syncthreads();

  // permutation of this zone's tokens into its blocks
  const Shape sh = shape_of(s_sid);
  const int nbh = zb.Lh / sh.h, nbw = zb.Lw / sh.w;
  const long long slot0 = zone_slot0(g, zb);
  for (int s = threadIdx.x; s < nt; s += kThreads) {
    const int blk = s >> 6, r = s & 63;
    const int bw = blk % nbw, bh = (blk / nbw) % nbh, bt = blk / (nbw * nbh);
    const int dw = r % sh.w, dh = (r / sh.w) % sh.h, dt = r / (sh.w * sh.h);
    const long long tok = ((long long)(zb.t0 + bt * sh.t + dt) * g.H +
                           (zb.h0 + bh * sh.h + dh)) * g.W +
                          (zb.w0 + bw * sh.w + dw);
    perm[(long long)b * N + slot0 + s] = (int32_t)tok;
    if (inv_perm) inv_perm[(long long)b * N + tok] = (int32_t)(slot0 + s);
  }
}

inline int n_slices_for(int C, int dtype) {
  const int CH = kRowBytes / (dtype == PRISM_BF16 ? 2 : 4);
  return ceil_div(C, CH);
}

}  // namespace

size_t zone_shapes_ws_bytes(int B, const ZoneGeom& g, int C) {
  const size_t part = (size_t)B * g.nZ * n_slices_for(C, PRISM_FP32) * 3 * sizeof(double);
  const size_t rms = (size_t)B * g.T * g.H * g.W * sizeof(double);
  return ((part + 255) / 256) * 256 + rms;
}

prism_status launch_zone_shapes(const void* feat, const void* a2v, int dtype,
                                int B, const ZoneGeom& g, int C, double lam,
                                int fixed_shape, int32_t* zone_shape,
                                int32_t* perm, int32_t* inv_perm,
                                double* zone_stats, void* ws,
                                hipStream_t stream) {
  const long long N = (long long)g.T * g.H * g.W;
  double* partial = nullptr;
  double* rms = nullptr;
  int n_slices = 0;
  if (fixed_shape < 0) {
    n_slices = n_slices_for(C, dtype);
    partial = static_cast<double*>(ws);
    const size_t part = (size_t)B * g.nZ * n_slices_for(C, PRISM_FP32) * 3 * sizeof(double);
    rms = reinterpret_cast<double*>(static_cast<char*>(ws) + ((part + 255) / 256) * 256);
    dim3 grid(n_slices, g.nZ, B);
    if (dtype == PRISM_BF16)
      PRISM_LAUNCH("zone_feat_dev", zone_feat_dev<uint16_t>, grid, dim3(kThreads), 0, stream,
                         static_cast<const unsigned char*>(feat), g, C, n_slices, partial);
    else
      PRISM_LAUNCH("zone_feat_dev", zone_feat_dev<float>, grid, dim3(kThreads), 0, stream,
                         static_cast<const unsigned char*>(feat), g, C, n_slices, partial);
    prism_status st = check_launch("zone_feat_dev");
    if (st != PRISM_OK) return st;
    if (a2v) {
      const long long ntok = (long long)B * N;
      dim3 g2((unsigned)((ntok + 3) / 4));
      if (dtype == PRISM_BF16)
        PRISM_LAUNCH("token_rms", token_rms<uint16_t>, g2, dim3(kThreads), 0, stream,
                           static_cast<const unsigned char*>(a2v), ntok, C, rms);
      else
        PRISM_LAUNCH("token_rms", token_rms<float>, g2, dim3(kThreads), 0, stream,
                           static_cast<const unsigned char*>(a2v), ntok, C, rms);
      st = check_launch("token_rms");
      if (st != PRISM_OK) return st;
    } else {
      rms = nullptr;
    }
  }
  PRISM_LAUNCH("zone_finalize", zone_finalize, dim3(g.nZ, B), dim3(kThreads), 0, stream, g, C,
                     n_slices, partial, rms, lam, fixed_shape, zone_shape, perm,
                     inv_perm, zone_stats);
  return check_launch("zone_finalize");
}

}  // namespace prism
