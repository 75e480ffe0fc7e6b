// Stage 4, backward: gradients of the block-sparse attention over the same
// selected blocks (the selection itself is constant).
//
// README "Overview": the method is used for training, so the sparse
// attention needs its backward pass.  With P = exp(s * scale - lse) and
// D_r = <dO_r, O_r>: dV = P^T dO, dS = P * (dO V^T - D), dQ = dS K * scale,
// dK = dS^T Q * scale.
//
// Launch sequence (deterministic, no floating-point atomics):
//   bwd_delta       D_r per query row (fp32).
//   bitmap_clear /  column bitmaps: bit i of KV block j's word set when query
//   bitmap_build    block i selected j -- the KV->query lists, read in
//                   ascending i by the dK/dV kernel.
//   dkdv_bf16       one workgroup per KV block; wave w owns 16 KV rows whose
//                   K and V stay in registers; loops over the query blocks
//                   that selected it (Q, Q^T, dO, dO^T staged in LDS).
//   dq_bf16         one workgroup per query block; loops over its list
//                   (K, K^T, V staged in LDS).
// All products are v_mfma_f32_16x16x32_bf16 with fp32 accumulation; the
// fp32 dtype uses plain per-thread kernels with the same structure.
#include <algorithm>

#include "prism_internal.h"

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// row of a 64-row operand feeding M-row m of M-tile mt (see attn_fwd.hip):
// lane group g of the C layout then holds slots 32*(mt/2) + 8g + 4*(mt%2) + r
__device__ __forceinline__ int slot_of(int mt, int m) {
  return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

// pack the C-layout tiles (2*ks2, 2*ks2+1) into a bf16x8 B operand
__device__ __forceinline__ bf16x8 pack_b(const f32x4& a, const f32x4& b) {
  uint4 u;
  u.x = (uint32_t)f32_to_bf16(a[0]) | ((uint32_t)f32_to_bf16(a[1]) << 16);
  u.y = (uint32_t)f32_to_bf16(a[2]) | ((uint32_t)f32_to_bf16(a[3]) << 16);
  u.z = (uint32_t)f32_to_bf16(b[0]) | ((uint32_t)f32_to_bf16(b[1]) << 16);
  u.w = (uint32_t)f32_to_bf16(b[2]) | ((uint32_t)f32_to_bf16(b[3]) << 16);
  return as_bf16x8(u);
}

// 64 gathered rows of a [., D] bf16 tensor into row-major (ld = D + 8) and
// transposed (ld = 72) LDS copies; either destination may be null.
template <int D>
__device__ __forceinline__ void stage_rows(const uint16_t* __restrict__ src,
                                           long long head, const int* rows,
                                           uint16_t* rm, uint16_t* tr) {
  const int tid = threadIdx.x;
  if (rm) {
#pragma unroll
    for (int c = tid; c < 64 * (D / 8); c += 256) {
      const int r = c / (D / 8), piece = c % (D / 8);
      *reinterpret_cast<uint4*>(&rm[r * (D + 8) + piece * 8]) =
          *reinterpret_cast<const uint4*>(src + (head + rows[r]) * D + piece * 8);
    }
  }
  if (tr) {
    for (int c = tid; c < (D / 8) * 16; c += 256) {
      const int dc = c % (D / 8), rg = c / (D / 8);
      uint4 r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r4[e] = *reinterpret_cast<const uint4*>(src + (head + rows[4 * rg + e]) * D + dc * 8);
      const uint16_t* s0 = reinterpret_cast<const uint16_t*>(&r4[0]);
      const uint16_t* s1 = reinterpret_cast<const uint16_t*>(&r4[1]);
      const uint16_t* s2 = reinterpret_cast<const uint16_t*>(&r4[2]);
      const uint16_t* s3 = reinterpret_cast<const uint16_t*>(&r4[3]);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        uint2 pk;
        pk.x = (uint32_t)s0[e8] | ((uint32_t)s1[e8] << 16);
        pk.y = (uint32_t)s2[e8] | ((uint32_t)s3[e8] << 16);
        *reinterpret_cast<uint2*>(&tr[(dc * 8 + e8) * 72 + 4 * rg]) = pk;
      }
    }
  }
}

// ------------------------------------------------------------- helpers
template <typename E>
__device__ __forceinline__ float ld(const E* p);
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) {
  return bf16_to_f32(*p);
}
template <>
__device__ __forceinline__ float ld<float>(const float* p) {
  return *p;
}

// D_r = <dO_r, O_r>, one row per 16 lanes... generic: one thread-group of
// D/8 lanes per row for bf16, plain loop for fp32.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_delta(const E* __restrict__ o,
                                                 const E* __restrict__ d_o,
                                                 long long rows,
                                                 float* __restrict__ delta) {
  constexpr int TPR = 16;  // threads per row
  const long long r = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float s = 0.f;
  if (r < rows) {
    for (int e = part; e < D; e += TPR)
      s += ld<E>(o + r * D + e) * ld<E>(d_o + r * D + e);
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (r < rows && part == 0) delta[r] = s;
}

__global__ void bitmap_clear(uint32_t* __restrict__ bits, long long n) {
  for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i < n;
       i += (long long)gridDim.x * blockDim.x)
    bits[i] = 0u;
}

// bit i of word (j, i / 32) <- query block i selected KV block j
__global__ void bitmap_build(const int32_t* __restrict__ counts,
                             const int32_t* __restrict__ kv_idx, int capacity,
                             int Nb, int words, long long rows,
                             uint32_t* __restrict__ bits) {
  const long long row = (long long)blockIdx.x * 4 + threadIdx.x / 64;
  if (row >= rows) return;
  const int lane = threadIdx.x % 64;
  const long long bh = row / Nb;
  const int i = (int)(row % Nb);
  const int cnt = counts[row];
  const int32_t* lst = kv_idx + row * (long long)capacity;
  for (int t = lane; t < cnt; t += 64) {
    const int j = lst[t];
    atomicOr(&bits[(bh * Nb + j) * words + (i >> 5)], 1u << (i & 31));
  }
}

// ------------------------------------------------------- dK / dV (bf16)
template <int D>
struct DkdvSmem {
  uint16_t Q[64 * (D + 8)];
  uint16_t Qt[D * 72];
  uint16_t dO[64 * (D + 8)];
  uint16_t dOt[D * 72];
  float lse2[64];
  float delta[64];
  int rows[64];
};

template <int D>
__global__ __launch_bounds__(256) void dkdv_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const uint32_t* __restrict__ bits,
    int words, int Hh, int N, float scale, float* __restrict__ dk,
    float* __restrict__ dv) {
  constexpr int KS = D / 32, DT = D / 16, LD = D + 8;
  __shared__ __align__(16) DkdvSmem<D> sm;
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const long long head = ((long long)b * Hh + h) * N;
  const int32_t* pb = perm + (long long)b * N;
  const float sl2 = scale * kLog2e;

  const int kvrow = pb[64 * j + 16 * wave + c16];
  bf16x8 kreg[KS], vreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    kreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(k + (head + kvrow) * D + 32 * ks + 8 * g));
    vreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(v + (head + kvrow) * D + 32 * ks + 8 * g));
  }
  f32x4 dva[DT], dka[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    dva[t] = f32x4{0.f, 0.f, 0.f, 0.f};
    dka[t] = f32x4{0.f, 0.f, 0.f, 0.f};
  }
  const uint32_t* col = bits + (((long long)b * Hh + h) * Nb + j) * words;

  for (int w = 0; w < words; ++w) {
    uint32_t word = col[w];
    while (word) {
      const int i = w * 32 + __ffs(word) - 1;
      word &= word - 1;
      __syncthreads();
      if (tid < 64) {
        const int r = pb[64 * i + tid];
        sm.rows[tid] = r;
        sm.lse2[tid] = lse[head + r] * kLog2e;
        sm.delta[tid] = delta[head + r];
      }
      __syncthreads();
      stage_rows<D>(q, head, sm.rows, sm.Q, sm.Qt);
      stage_rows<D>(d_o, head, sm.rows, sm.dO, sm.dOt);
      __syncthreads();

      // S = Q K^T and dP = dO V^T: M = query slots, N = this wave's 16 kv
      f32x4 s[4], dp[4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
        const int qr = slot_of(mt, c16);
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Q[qr * LD + 32 * ks + 8 * g])),
              kreg[ks], s[mt], 0, 0, 0);
          dp[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(&sm.dO[qr * LD + 32 * ks + 8 * g])),
              vreg[ks], dp[mt], 0, 0, 0);
        }
      }
      // P and dS; lane holds query slots slot_of(mt, 4g + r), kv c16
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int qs = slot_of(mt, 4 * g + r);
          const float p = exp2f(s[mt][r] * sl2 - sm.lse2[qs]);
          s[mt][r] = p;
          dp[mt][r] = p * (dp[mt][r] - sm.delta[qs]);
        }
      bf16x8 pB[2], dsB[2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        pB[ks2] = pack_b(s[2 * ks2], s[2 * ks2 + 1]);
        dsB[ks2] = pack_b(dp[2 * ks2], dp[2 * ks2 + 1]);
      }
      // dV^T += dO^T P ; dK^T += Q^T dS   (M = d, N = kv, K = query slots)
#pragma unroll
      for (int mt = 0; mt < DT; ++mt) {
        const int dr = 16 * mt + c16;
#pragma unroll
        for (int ks2 = 0; ks2 < 2; ++ks2) {
          dva[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(&sm.dOt[dr * 72 + 32 * ks2 + 8 * g])),
              pB[ks2], dva[mt], 0, 0, 0);
          dka[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
              as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Qt[dr * 72 + 32 * ks2 + 8 * g])),
              dsB[ks2], dka[mt], 0, 0, 0);
        }
      }
    }
  }
  // dV[kv c16][16mt + 4g + r]
  float* dvr = dv + (head + kvrow) * D;
  float* dkr = dk + (head + kvrow) * D;
#pragma unroll
  for (int mt = 0; mt < DT; ++mt) {
    *reinterpret_cast<float4*>(dvr + 16 * mt + 4 * g) =
        make_float4(dva[mt][0], dva[mt][1], dva[mt][2], dva[mt][3]);
    *reinterpret_cast<float4*>(dkr + 16 * mt + 4 * g) =
        make_float4(dka[mt][0] * scale, dka[mt][1] * scale, dka[mt][2] * scale,
                    dka[mt][3] * scale);
  }
}

// ------------------------------------------------------------ dQ (bf16)
template <int D>
struct DqSmem {
  uint16_t K[64 * (D + 8)];
  uint16_t Kt[D * 72];
  uint16_t V[64 * (D + 8)];
  int rows[64];
};

template <int D>
__global__ __launch_bounds__(256) void dq_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ kv_idx, int capacity, int Hh, int N,
    float scale, float* __restrict__ dq) {
  constexpr int KS = D / 32, DT = D / 16, LD = D + 8;
  __shared__ __align__(16) DqSmem<D> sm;
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const long long head = ((long long)b * Hh + h) * N;
  const int32_t* pb = perm + (long long)b * N;
  const float sl2 = scale * kLog2e;

  const int qrow = pb[64 * i + 16 * wave + c16];
  bf16x8 qreg[KS], doreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(q + (head + qrow) * D + 32 * ks + 8 * g));
    doreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(d_o + (head + qrow) * D + 32 * ks + 8 * g));
  }
  const float lse2 = lse[head + qrow] * kLog2e;
  const float dlt = delta[head + qrow];
  f32x4 dqa[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dqa[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const long long rowid = ((long long)b * Hh + h) * Nb + i;
  const int cnt = counts[rowid];
  const int32_t* lst = kv_idx + rowid * (long long)capacity;
  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    __syncthreads();
    if (tid < 64) sm.rows[tid] = pb[64 * j + tid];
    __syncthreads();
    stage_rows<D>(k, head, sm.rows, sm.K, sm.Kt);
    stage_rows<D>(v, head, sm.rows, sm.V, nullptr);
    __syncthreads();
    // S^T = K Q^T, dP^T = V dO^T   (M = kv slots, N = this wave's queries)
    f32x4 s[4], dp[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      dp[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const int kr = slot_of(mt, c16);
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(&sm.K[kr * LD + 32 * ks + 8 * g])),
            qreg[ks], s[mt], 0, 0, 0);
        dp[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(&sm.V[kr * LD + 32 * ks + 8 * g])),
            doreg[ks], dp[mt], 0, 0, 0);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float p = exp2f(s[mt][r] * sl2 - lse2);
        dp[mt][r] = p * (dp[mt][r] - dlt);
      }
    bf16x8 dsB[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) dsB[ks2] = pack_b(dp[2 * ks2], dp[2 * ks2 + 1]);
    // dQ^T += K^T dS^T  (M = d, N = queries, K = kv slots)
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const int dr = 16 * mt + c16;
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
        dqa[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(&sm.Kt[dr * 72 + 32 * ks2 + 8 * g])),
            dsB[ks2], dqa[mt], 0, 0, 0);
    }
  }
  float* dqr = dq + (head + qrow) * D;
#pragma unroll
  for (int mt = 0; mt < DT; ++mt)
    *reinterpret_cast<float4*>(dqr + 16 * mt + 4 * g) =
        make_float4(dqa[mt][0] * scale, dqa[mt][1] * scale, dqa[mt][2] * scale,
                    dqa[mt][3] * scale);
}

// ------------------------------------------------------ fp32 reference
template <int D>
__global__ __launch_bounds__(64) void dq_f32(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ kv_idx, int capacity, int Hh, int N,
    float scale, float* __restrict__ dq) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const long long head = ((long long)b * Hh + h) * N;
  const int32_t* pb = perm + (long long)b * N;
  const long long qr = head + pb[64 * i + threadIdx.x];
  float acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) acc[e] = 0.f;
  const float L = lse[qr], Dl = delta[qr];
  const long long rowid = ((long long)b * Hh + h) * Nb + i;
  const int cnt = counts[rowid];
  const int32_t* lst = kv_idx + rowid * (long long)capacity;
  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    for (int r = 0; r < 64; ++r) {
      const long long kr = head + pb[64 * j + r];
      float s = 0.f, dpv = 0.f;
      for (int e = 0; e < D; ++e) {
        s = fmaf(q[qr * D + e], k[kr * D + e], s);
        dpv = fmaf(d_o[qr * D + e], v[kr * D + e], dpv);
      }
      const float p = expf(s * scale - L);
      const float ds = p * (dpv - Dl);
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = fmaf(ds, k[kr * D + e], acc[e]);
    }
  }
#pragma unroll
  for (int e = 0; e < D; ++e) dq[qr * D + e] = acc[e] * scale;
}

template <int D>
__global__ __launch_bounds__(64) void dkdv_f32(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const float* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const uint32_t* __restrict__ bits,
    int words, int Hh, int N, float scale, float* __restrict__ dk,
    float* __restrict__ dv) {
  const int j = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const long long head = ((long long)b * Hh + h) * N;
  const int32_t* pb = perm + (long long)b * N;
  const long long kr = head + pb[64 * j + threadIdx.x];
  float ak[D], av[D];
#pragma unroll
  for (int e = 0; e < D; ++e) ak[e] = av[e] = 0.f;
  const uint32_t* col = bits + (((long long)b * Hh + h) * Nb + j) * words;
  for (int w = 0; w < words; ++w) {
    uint32_t word = col[w];
    while (word) {
      const int i = w * 32 + __ffs(word) - 1;
      word &= word - 1;
      for (int r = 0; r < 64; ++r) {
        const long long qr = head + pb[64 * i + r];
        float s = 0.f, dpv = 0.f;
        for (int e = 0; e < D; ++e) {
          s = fmaf(q[qr * D + e], k[kr * D + e], s);
          dpv = fmaf(d_o[qr * D + e], v[kr * D + e], dpv);
        }
        const float p = expf(s * scale - lse[qr]);
        const float ds = p * (dpv - delta[qr]);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          av[e] = fmaf(p, d_o[qr * D + e], av[e]);
          ak[e] = fmaf(ds, q[qr * D + e], ak[e]);
        }
      }
    }
  }
#pragma unroll
  for (int e = 0; e < D; ++e) {
    dv[kr * D + e] = av[e];
    dk[kr * D + e] = ak[e] * scale;
  }
}

inline int bitmap_words(int Nb) { return (Nb + 31) / 32; }

template <int D>
prism_status run_bwd(const void* q, const void* k, const void* v,
                     const void* o, const void* d_o, const float* lse,
                     int dtype, const int32_t* perm, const int32_t* counts,
                     const int32_t* kv_idx, int capacity, int B, int Hh, int N,
                     float scale, float* dq, float* dk, float* dv, void* ws,
                     hipStream_t stream) {
  const int Nb = N / 64;
  const int words = bitmap_words(Nb);
  const long long rows = (long long)B * Hh * N;
  float* delta = static_cast<float*>(ws);
  const size_t dbytes = ((rows * sizeof(float) + 255) / 256) * 256;
  uint32_t* bits = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + dbytes);
  const long long nbits = (long long)B * Hh * Nb * words;

  if (dtype == PRISM_BF16)
    PRISM_LAUNCH("bwd_delta", (bwd_delta<uint16_t, D>), dim3((unsigned)((rows + 15) / 16)),
                       dim3(256), 0, stream, (const uint16_t*)o, (const uint16_t*)d_o,
                       rows, delta);
  else
    PRISM_LAUNCH("bwd_delta", (bwd_delta<float, D>), dim3((unsigned)((rows + 15) / 16)),
                       dim3(256), 0, stream, (const float*)o, (const float*)d_o, rows,
                       delta);
  prism_status st = check_launch("bwd_delta");
  if (st != PRISM_OK) return st;
  const unsigned cg = (unsigned)std::min<long long>((nbits + 255) / 256, 65535);
  PRISM_LAUNCH("bitmap_clear", bitmap_clear, dim3(cg), dim3(256), 0, stream, bits, nbits);
  if ((st = check_launch("bitmap_clear")) != PRISM_OK) return st;
  const long long qrows = (long long)B * Hh * Nb;
  PRISM_LAUNCH("bitmap_build", bitmap_build, dim3((unsigned)((qrows + 3) / 4)), dim3(256), 0,
                     stream, counts, kv_idx, capacity, Nb, words, qrows, bits);
  if ((st = check_launch("bitmap_build")) != PRISM_OK) return st;

  dim3 grid(Nb, Hh, B);
  if (dtype == PRISM_BF16) {
    PRISM_LAUNCH("dkdv_bf16", dkdv_bf16<D>, grid, dim3(256), 0, stream, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o,
                       lse, delta, perm, bits, words, Hh, N, scale, dk, dv);
    if ((st = check_launch("dkdv_bf16")) != PRISM_OK) return st;
    PRISM_LAUNCH("dq_bf16", dq_bf16<D>, grid, dim3(256), 0, stream, (const uint16_t*)q,
                       (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o,
                       lse, delta, perm, counts, kv_idx, capacity, Hh, N, scale, dq);
    return check_launch("dq_bf16");
  }
  PRISM_LAUNCH("dkdv_f32", dkdv_f32<D>, grid, dim3(64), 0, stream, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)d_o, lse, delta,
                     perm, bits, words, Hh, N, scale, dk, dv);
  if ((st = check_launch("dkdv_f32")) != PRISM_OK) return st;
  PRISM_LAUNCH("dq_f32", dq_f32<D>, grid, dim3(64), 0, stream, (const float*)q,
                     (const float*)k, (const float*)v, (const float*)d_o, lse, delta,
                     perm, counts, kv_idx, capacity, Hh, N, scale, dq);
  return check_launch("dq_f32");
}

}  // namespace

size_t attn_bwd_ws_bytes(int B, int Hh, int N, int d) {
  (void)d;
  const long long rows = (long long)B * Hh * N;
  const size_t dbytes = ((rows * sizeof(float) + 255) / 256) * 256;
  const int Nb = N / 64;
  return dbytes + (size_t)B * Hh * Nb * bitmap_words(Nb) * sizeof(uint32_t);
}

prism_status launch_attn_bwd(const void* q, const void* k, const void* v,
                             const void* o, const void* d_o, const float* lse,
                             int dtype, const int32_t* perm,
                             const int32_t* counts, const int32_t* kv_idx,
                             int capacity, int B, int Hh, int N, int d,
                             float scale, float* dq, float* dk, float* dv,
                             void* ws, hipStream_t stream) {
  if (d == 128)
    return run_bwd<128>(q, k, v, o, d_o, lse, dtype, perm, counts, kv_idx,
                        capacity, B, Hh, N, scale, dq, dk, dv, ws, stream);
  return run_bwd<64>(q, k, v, o, d_o, lse, dtype, perm, counts, kv_idx,
                     capacity, B, Hh, N, scale, dq, dk, dv, ws, stream);
}

}  // namespace prism
