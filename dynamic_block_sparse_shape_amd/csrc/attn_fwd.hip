// Stage 4, forward: block-sparse attention with online softmax over the
// selected KV blocks only.
//
// The abstract page ("Prism: Dynamic Sparse Attention ...") describes
// sparse attention that computes only the selected key/value blocks inside
// one online-softmax pass; README "Overview": each query block has its own
// budget of blocks.
//
// bf16 path (gfx950 MFMA, v_mfma_f32_16x16x32_bf16, fp32 accumulation):
//   one workgroup (4 waves) per (b, h, query block); wave w owns query rows
//   16w..16w+15, held in registers as the B operand.  For each listed KV
//   block the workgroup gathers K (row-major) and V (transposed) through
//   perm into LDS.  Each wave computes S^T = K Q^T (kv x q), so every lane
//   holds 16 scores of one query and the row statistics need only two
//   cross-lane steps; the KV rows feeding the M-tiles are ordered so that
//   the lane's scores are already the B operand of O^T += V^T P^T.
// fp32 path: one thread per query row, plain fp32 arithmetic (reference
//   precision for small problems).
#include "prism_internal.h"

namespace prism {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(uint4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

// KV row feeding M-row m of M-tile mt, chosen so that the C layout of the
// score tiles (lane group g holds M-rows 4g..4g+3) lands each lane's scores
// on kv slots 32*(mt/2) + 8g + 4*(mt%2) + r -- eight consecutive kv per
// lane group per 32-wide k-step of the P*V product.
__device__ __forceinline__ int kv_of(int mt, int m) {
  return 32 * (mt >> 1) + 8 * (m >> 2) + 4 * (mt & 1) + (m & 3);
}

template <int D>
struct FwdSmem {
  static constexpr int KLD = D + 8;   // K row stride (bf16 elements)
  static constexpr int VLD = 64 + 8;  // V^T row stride
  uint16_t K[64 * KLD];
  uint16_t Vt[D * VLD];
  int rows[64];
};

template <int D>
__global__ __launch_bounds__(256) void attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, int Hh, int N, float scale_log2, uint16_t* __restrict__ o,
    float* __restrict__ lse) {
  constexpr int KS = D / 32;   // k-steps of Q K^T
  constexpr int DT = D / 16;   // d tiles of O^T
  constexpr int KLD = FwdSmem<D>::KLD;
  constexpr int VLD = FwdSmem<D>::VLD;
  __shared__ __align__(16) FwdSmem<D> sm;

  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int g = lane >> 4, c16 = lane & 15;
  const long long head = ((long long)b * Hh + h) * N;   // row offset
  const int32_t* pb = perm + (long long)b * N;

  const int qrow = pb[64 * i + 16 * wave + c16];
  bf16x8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const uint4*>(
        q + (head + qrow) * D + 32 * ks + 8 * g));

  float m_run = -INFINITY, l_run = 0.f;
  f32x4 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x4{0.f, 0.f, 0.f, 0.f};

  const long long rowid = ((long long)b * Hh + h) * Nb + i;
  const int cnt = counts[rowid];
  const int32_t* lst = kv_idx + rowid * (long long)capacity;

  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    __syncthreads();
    if (tid < 64) sm.rows[tid] = pb[64 * j + tid];
    __syncthreads();
    // K: 64 rows x D bf16, 16-byte pieces
#pragma unroll
    for (int c = tid; c < 64 * (D / 8); c += 256) {
      const int r = c / (D / 8), piece = c % (D / 8);
      *reinterpret_cast<uint4*>(&sm.K[r * KLD + piece * 8]) =
          *reinterpret_cast<const uint4*>(k + (head + sm.rows[r]) * D + piece * 8);
    }
    // V^T: a thread takes 8 d-values of 4 consecutive kv rows
    for (int c = tid; c < (D / 8) * 16; c += 256) {
      const int dc = c % (D / 8), rg = c / (D / 8);
      uint4 r4[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        r4[e] = *reinterpret_cast<const uint4*>(v + (head + sm.rows[4 * rg + e]) * D + dc * 8);
      const uint16_t* s0 = reinterpret_cast<const uint16_t*>(&r4[0]);
      const uint16_t* s1 = reinterpret_cast<const uint16_t*>(&r4[1]);
      const uint16_t* s2 = reinterpret_cast<const uint16_t*>(&r4[2]);
      const uint16_t* s3 = reinterpret_cast<const uint16_t*>(&r4[3]);
#pragma unroll
      for (int e8 = 0; e8 < 8; ++e8) {
        uint2 pk;
        pk.x = (uint32_t)s0[e8] | ((uint32_t)s1[e8] << 16);
        pk.y = (uint32_t)s2[e8] | ((uint32_t)s3[e8] << 16);
        *reinterpret_cast<uint2*>(&sm.Vt[(dc * 8 + e8) * VLD + 4 * rg]) = pk;
      }
    }
    __syncthreads();

    // S^T = K Q^T
    f32x4 s[4];
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      s[mt] = f32x4{0.f, 0.f, 0.f, 0.f};
      const uint16_t* krow = &sm.K[kv_of(mt, c16) * KLD + 8 * g];
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        s[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(krow + 32 * ks)), qreg[ks],
            s[mt], 0, 0, 0);
    }
    // online softmax (log2 domain) for query c16
    float mx = -INFINITY;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[mt][r] *= scale_log2;
        mx = fmaxf(mx, s[mt][r]);
      }
    mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
    mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
    const float m_new = fmaxf(m_run, mx);
    const float alpha = exp2f(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        s[mt][r] = exp2f(s[mt][r] - m_new);
        rs += s[mt][r];
      }
    rs += __shfl_xor(rs, 16, 64);
    rs += __shfl_xor(rs, 32, 64);
    l_run = l_run * alpha + rs;
    m_run = m_new;
#pragma unroll
    for (int t2 = 0; t2 < DT; ++t2) oacc[t2] *= alpha;

    // P^T as the B operand: k-step ks2 covers kv 32*ks2 .. 32*ks2+31
    bf16x8 pbf[2];
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2) {
      uint4 u;
      uint32_t* uw = reinterpret_cast<uint32_t*>(&u);
#pragma unroll
      for (int r = 0; r < 4; r += 2) {
        uw[r / 2] = (uint32_t)f32_to_bf16(s[2 * ks2][r]) |
                    ((uint32_t)f32_to_bf16(s[2 * ks2][r + 1]) << 16);
        uw[2 + r / 2] = (uint32_t)f32_to_bf16(s[2 * ks2 + 1][r]) |
                        ((uint32_t)f32_to_bf16(s[2 * ks2 + 1][r + 1]) << 16);
      }
      pbf[ks2] = as_bf16x8(u);
    }
    // O^T += V^T P^T
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const uint16_t* vrow = &sm.Vt[(16 * mt + c16) * VLD + 8 * g];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
        oacc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
            as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 32 * ks2)), pbf[ks2],
            oacc[mt], 0, 0, 0);
    }
  }

  // O[q][16mt + 4g + r] = oacc[mt][r] / l
  const float inv_l = 1.f / l_run;
  uint16_t* orow = o + (head + qrow) * D;
#pragma unroll
  for (int mt = 0; mt < DT; ++mt) {
    uint2 pk;
    pk.x = (uint32_t)f32_to_bf16(oacc[mt][0] * inv_l) |
           ((uint32_t)f32_to_bf16(oacc[mt][1] * inv_l) << 16);
    pk.y = (uint32_t)f32_to_bf16(oacc[mt][2] * inv_l) |
           ((uint32_t)f32_to_bf16(oacc[mt][3] * inv_l) << 16);
    *reinterpret_cast<uint2*>(orow + 16 * mt + 4 * g) = pk;
  }
  if (g == 0) lse[head + qrow] = (m_run + log2f(l_run)) * kLn2;
}

// fp32 reference-precision path: one thread per query row.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, int Hh, int N, float scale, float* __restrict__ o,
    float* __restrict__ lse) {
  const int i = blockIdx.x, h = blockIdx.y, b = blockIdx.z;
  const int Nb = N / 64;
  const long long head = ((long long)b * Hh + h) * N;
  const int32_t* pb = perm + (long long)b * N;
  const int qrow = pb[64 * i + threadIdx.x];
  float qv[D], acc[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    qv[e] = q[(head + qrow) * D + e];
    acc[e] = 0.f;
  }
  float m_run = -INFINITY, l_run = 0.f;
  const long long rowid = ((long long)b * Hh + h) * Nb + i;
  const int cnt = counts[rowid];
  const int32_t* lst = kv_idx + rowid * (long long)capacity;
  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    for (int r = 0; r < 64; ++r) {
      const long long kr = head + pb[64 * j + r];
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) s = fmaf(qv[e], k[kr * D + e], s);
      s *= scale;
      const float m_new = fmaxf(m_run, s);
      const float alpha = expf(m_run - m_new);
      const float p = expf(s - m_new);
      l_run = l_run * alpha + p;
#pragma unroll
      for (int e = 0; e < D; ++e) acc[e] = acc[e] * alpha + p * v[kr * D + e];
      m_run = m_new;
    }
  }
  const float inv_l = 1.f / l_run;
#pragma unroll
  for (int e = 0; e < D; ++e) o[(head + qrow) * D + e] = acc[e] * inv_l;
  lse[head + qrow] = m_run + logf(l_run);
}

}  // namespace

prism_status launch_attn_fwd(const void* q, const void* k, const void* v,
                             int dtype, const int32_t* perm,
                             const int32_t* counts, const int32_t* kv_idx,
                             int capacity, int B, int Hh, int N, int d,
                             float scale, void* o, float* lse,
                             hipStream_t stream) {
  dim3 grid(N / 64, Hh, B);
  if (dtype == PRISM_BF16) {
    const float sl2 = scale * kLog2e;
    if (d == 128)
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<128>, grid, dim3(256), 0, stream,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                         perm, counts, kv_idx, capacity, Hh, N, sl2, (uint16_t*)o, lse);
    else
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<64>, grid, dim3(256), 0, stream,
                         (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                         perm, counts, kv_idx, capacity, Hh, N, sl2, (uint16_t*)o, lse);
  } else {
    if (d == 128)
      PRISM_LAUNCH("attn_fwd_f32", attn_fwd_f32<128>, grid, dim3(64), 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, perm,
                         counts, kv_idx, capacity, Hh, N, scale, (float*)o, lse);
    else
      PRISM_LAUNCH("attn_fwd_f32", attn_fwd_f32<64>, grid, dim3(64), 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, perm,
                         counts, kv_idx, capacity, Hh, N, scale, (float*)o, lse);
  }
  return check_launch("attn_fwd");
}

}  // namespace prism
