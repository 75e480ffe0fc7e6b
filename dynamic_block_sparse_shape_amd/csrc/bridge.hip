// The audio-to-video (a2v) bridge residual that stage 1 reads.
//
// Prism architecture walk-through (wmrh.cn), sections "a2v / v2a 条件桥" and
// "一个巧妙的联动：桥接残差反哺稀疏注意力": a conditional cross-attention
// block whose queries are the video tokens' 3072-wide hidden states and whose
// keys and values come from the audio tokens' 1536-wide hidden states; its
// output is added to the video tower as a residual, and the *unscaled*
// residual feeds the sparse attention's per-token norm.  Both directions
// support a rotary alignment of video frames and audio steps on one time
// axis.  The pages give no formula; the library computes multi-head
// scaled dot-product cross-attention with linear projections (weights
// [out, in], no bias, no normalisation), heads of 128, and an optional
// rotary rotation of q and k by caller-given time positions:
//   q = x_v Wq^T, k = x_a Wk^T, v = x_a Wv^T, rotated pairwise (2i, 2i+1) by
//   pos * base^(-2i / 128); o_h = softmax(q_h k_h^T / sqrt(128)) v_h;
//   dh = concat_h(o_h) Wo^T.
//
// Kernels:
//   gemm_nt_bf16   C[M, F] = X[M, K] W[F, K]^T, bf16 in, fp32 accumulation
//                  (v_mfma_f32_32x32x16_bf16), bf16 out, optional rotary
//                  epilogue.  256 x 256 tiles over 64-deep k-slabs, four
//                  waves of 128 x 128, two LDS stages; tiles dealt so that
//                  each XCD walks groups of 8 token tiles across the feature
//                  tiles (its L2 serves each k-slab to several workgroups).
//   bridge_attn    per (64 video tokens, head, batch): the audio keys in
//                  64-key tiles, online softmax, output over the queries in
//                  place (every workgroup reads its query rows before it
//                  writes the same rows and columns).
#include "attn_tiles.h"

namespace prism {
namespace {

using namespace tiles;

constexpr int kGM = 256;       // tokens per GEMM tile
constexpr int kGN = 256;       // output features per GEMM tile
constexpr int kGK = 64;        // k per LDS stage (128-byte rows)
using TK = Tile<64>;           // 128-byte rows, XOR-swizzled 16-byte pieces

// Work item of this workgroup: each XCD (workgroup L runs on XCD L % 8)
// takes a contiguous eighth of the item sequence; items run in groups of up
// to 8 token tiles, feature tile by feature tile, so the ~32 workgroups an
// XCD holds at once share 8 X slabs and 4 W slabs per k-step.
__device__ __forceinline__ bool gemm_item(int TT, int FT, int& tm, int& tf) {
  const long long total = (long long)TT * FT;
  const long long per = (total + 7) / 8;
  const long long q = (long long)(blockIdx.x & 7) * per + (blockIdx.x >> 3);
  if (q >= total) return false;
  constexpr int G = 8;
  const long long grp = q / ((long long)G * FT);
  const int rem = (int)(q % ((long long)G * FT));
  const int gsz = min(G, TT - (int)grp * G);
  tf = rem / gsz;
  tm = (int)grp * G + rem % gsz;
  return true;
}

// NT: 256 threads (four waves of 128 features x 128 tokens, one wave per
// SIMD) or 512 threads (eight waves of 128 x 64, two per SIMD).
template <int NT>
__global__ __launch_bounds__(NT, 1) void gemm_nt_bf16(
    const uint16_t* __restrict__ X, const uint16_t* __restrict__ Wt, int M,
    int F, int K, uint16_t* __restrict__ C, const float* __restrict__ pos,
    float log2_base) {
  extern __shared__ __align__(16) unsigned char dyn[];
  // stage s: X tile (256 rows) then W tile (256 rows), 128 bytes per row
  constexpr int kStage = (kGM + kGN) * kGK * 2;
  constexpr int kPieces = (kGM + kGN) * (kGK * 2 / 16) / NT;   // per thread
  constexpr int TW = NT == 256 ? 4 : 2;       // 32-token tiles per wave
  const int TT = (M + kGM - 1) / kGM, FT = F / kGN;
  int tm, tf;
  if (!gemm_item(TT, FT, tm, tf)) return;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int c = lane & 31, hf = lane >> 5;
  const int wf = wave & 1, wt = wave >> 1;
  const int tbase = 32 * TW * wt;             // first token row of the wave
  const int m0 = tm * kGM, f0 = tf * kGN;
  const int rows_x = min(kGM, M - m0);
  // one buffer resource per operand tile: rows past M read as zeros
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(X + (long long)m0 * K), (short)0, rows_x * K * 2,
      0x00020000);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(Wt + (long long)f0 * K), (short)0, kGN * K * 2,
      0x00020000);
  // piece i of this thread: row (tid + NT i) / 8 of the 512 stage rows
  // (X rows 0..255, then W rows), 16-byte piece tid % 8
  const int piece = tid & 7;
  const uint32_t goff0 = (uint32_t)((tid >> 3) * K * 2 + piece * 16);
  const uint32_t gstep = (uint32_t)((NT >> 3) * K * 2);
  u32x4 st[kPieces];
  auto load = [&](int kt) __attribute__((always_inline)) {
    const uint32_t kb = (uint32_t)(kt * kGK * 2);
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      constexpr int half = kPieces / 2;
      const int ii = i < half ? i : i - half;
      st[i] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(
                     i < half ? rx : rw, goff0 + ii * gstep + kb, 0, 0));
    }
  };
  auto store = [&](unsigned char* s) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < kPieces; ++i) {
      const int r = (tid + NT * i) >> 3;        // 0..511
      *reinterpret_cast<u32x4*>(s + TK::off(r, piece)) = st[i];
    }
  };

  f32x16 acc[4][TW];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < TW; ++b) acc[a][b] = f32x16{};

  const int KT = K / kGK;
  load(0);
  store(dyn);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    if (kt + 1 < KT) load(kt + 1);
    const unsigned char* sx = dyn + (kt & 1) * kStage;
    const unsigned char* sw = sx + kGM * kGK * 2;
#pragma unroll
    for (int ks = 0; ks < kGK / 16; ++ks) {
      bf16x8 fa[4], fb[TW];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        fa[i] = lds_row8<64>(sw, 128 * wf + 32 * i + c, 2 * ks + hf);
#pragma unroll
      for (int i = 0; i < TW; ++i)
        fb[i] = lds_row8<64>(sx, tbase + 32 * i + c, 2 * ks + hf);
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < TW; ++b) acc[a][b] = mfma32(fa[a], fb[b], acc[a][b]);
    }
    if (kt + 1 < KT) store(dyn + ((kt + 1) & 1) * kStage);
    __syncthreads();
  }

  // acc[a][b] holds C^T: register 4e + g of lane (c, hf) is feature
  // f0 + 128 wf + 32 a + 8 e + 4 hf + g, token m0 + tbase + 32 b + c
#pragma unroll
  for (int b = 0; b < TW; ++b) {
    const int tok = m0 + tbase + 32 * b + c;
    if (tok >= M) continue;
    const float p = pos ? pos[tok] : 0.f;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int f = f0 + 128 * wf + 32 * a + 8 * e + 4 * hf;
        float x[4];
#pragma unroll
        for (int g = 0; g < 4; ++g) x[g] = acc[a][b][4 * e + g];
        if (pos) {
          // pairs (f, f+1) and (f+2, f+3), f even; the pair's place in the
          // 128-wide head sets its frequency
#pragma unroll
          for (int g = 0; g < 4; g += 2) {
            const float fr = exp2f(-(float)((f + g) & 127) * (1.f / 128.f) * log2_base);
            float sn, cs;
            sincosf(p * fr, &sn, &cs);
            const float xe = x[g], xo = x[g + 1];
            x[g] = xe * cs - xo * sn;
            x[g + 1] = xe * sn + xo * cs;
          }
        }
        uint2 pk;
        pk.x = cvt2(x[0], x[1]);
        pk.y = cvt2(x[2], x[3]);
        *reinterpret_cast<uint2*>(C + (long long)tok * F + f) = pk;
      }
  }
}

// Cross-attention of 64 video tokens against every audio token of one head:
// wave (qh, kh) takes queries 32 qh .. +31 against keys 32 kh .. +31 of each
// 64-key tile (S^T = K Q^T on 32 x 32 MFMA tiles, P straight from the
// C layout into the B operand of O^T += V^T P^T); the two kh halves keep
// separate online-softmax states, merged at the end.  Keys past Na score
// -inf.  q and o may alias: each workgroup reads its own query rows into
// registers first and writes the same rows and columns after the merge.
__global__ __launch_bounds__(256, 2) void bridge_attn(
    const uint16_t* q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, uint16_t* o, int N, int Na, int Dtot,
    float scale_log2) {
  constexpr int D = 128, KS = D / 16, DT = D / 32;
  using TL = Tile<D>;
  using SH = Share<D, 256>;
  __shared__ __align__(16) unsigned char smem[2 * TL::kBytes];
  __shared__ float sm_m[2][32], sm_l[2][32];
  const int head = blockIdx.y, b = blockIdx.z;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int qh = wave & 1, kh = wave >> 1;
  const int c = lane & 31, hf = lane >> 5, j16 = lane & 15, grp = lane >> 4;
  const int qrow = 64 * blockIdx.x + 32 * qh + c;
  const long long qbase = ((long long)b * N + min(qrow, N - 1)) * Dtot + head * D;
  bf16x8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(q + qbase + 16 * ks + 8 * hf));
  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  const int krow = 32 * kh + slot_of(c);
  // key row of C-layout register 4e + g of this lane
  int kof[16];
#pragma unroll
  for (int r = 0; r < 16; ++r) kof[r] = 32 * kh + slot_of(8 * (r >> 2) + 4 * hf + (r & 3));
  const long long kvbase = (long long)b * Na * Dtot + head * D;
  const unsigned char* sk = smem;
  const unsigned char* sv = smem + TL::kBytes;
  const int tiles = (Na + 63) / 64;
  for (int t = 0; t < tiles; ++t) {
    __syncthreads();
#pragma unroll
    for (int i = 0; i < SH::kPerThread; ++i) {
      const int r = SH::row_of(tid, i), p = SH::piece_of(tid);
      const int key = 64 * t + r;
      u32x4 kv4 = u32x4{0u, 0u, 0u, 0u}, vv4 = u32x4{0u, 0u, 0u, 0u};
      if (key < Na) {
        kv4 = *reinterpret_cast<const u32x4*>(k + kvbase + (long long)key * Dtot + 8 * p);
        vv4 = *reinterpret_cast<const u32x4*>(v + kvbase + (long long)key * Dtot + 8 * p);
      }
      *reinterpret_cast<u32x4*>(smem + TL::off(r, p)) = kv4;
      *reinterpret_cast<u32x4*>(smem + TL::kBytes + TL::off(r, p)) = vv4;
    }
    __syncthreads();
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = mfma32(lds_row8<D>(sk, krow, 2 * ks + hf), qreg[ks], s);
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      if (64 * t + kof[r] >= Na) s[r] = -INFINITY;
      mx = fmax_prop(mx, s[r]);
    }
    mx = xor32_max(mx) * scale_log2;
    const float m_new = mx > m_run + 8.f ? mx : m_run;
    if (m_new == -INFINITY) continue;       // no valid key yet (whole wave)
    const float alpha = m_run == m_new ? 1.f : exp2_fast(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], scale_log2, -m_new));
      rs += s[r];
    }
    rs = xor32_sum(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) oacc[t2] *= alpha;
    }
    const bf16x8 p0 = pack8(s, 0), p1 = pack8(s, 1);
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const int d0 = 32 * mt + 16 * (grp & 1);
      const int r0 = 32 * kh + 8 * (grp >> 1);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0, d0, j16), p0, oacc[mt]);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0 + 16, d0, j16), p1, oacc[mt]);
    }
  }
  // merge the kh = 1 half into kh = 0 through LDS
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smem);
  if (kh == 1) {
    if (hf == 0) {
      sm_m[qh][c] = m_run;
      sm_l[qh][c] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xo[((qh * 64 + lane) * DT + mt) * 16 + r] = oacc[mt][r];
  }
  __syncthreads();
  if (kh == 0 && qrow < N) {
    const float m2 = sm_m[qh][c], l2 = sm_l[qh][c];
    const float m = fmaxf(m_run, m2);
    const bool none = m == -INFINITY;
    const float a1 = none ? 0.f : exp2_fast(m_run - m);
    const float a2 = none ? 0.f : exp2_fast(m2 - m);
    const float l = l_run * a1 + l2 * a2;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = o + qbase;
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float vals[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = 4 * a + bb;
          vals[bb] = (oacc[mt][r] * a1 + xo[((qh * 64 + lane) * DT + mt) * 16 + r] * a2) * inv_l;
        }
        uint2 pk;
        pk.x = cvt2(vals[0], vals[1]);
        pk.y = cvt2(vals[2], vals[3]);
        *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * a + 4 * hf) = pk;
      }
  }
}

prism_status gemm(const uint16_t* X, const uint16_t* Wt, int M, int F, int K,
                  uint16_t* C, const float* pos, float log2_base,
                  hipStream_t stream) {
  const long long TT = (M + kGM - 1) / kGM, FT = F / kGN;
  const unsigned grid = (unsigned)(8 * ((TT * FT + 7) / 8));
  const size_t lds = 2 * (size_t)(kGM + kGN) * kGK * 2;
  PRISM_LAUNCH("bridge_gemm", gemm_nt_bf16<512>, dim3(grid), dim3(512), lds,
               stream, X, Wt, M, F, K, C, pos, log2_base);
  return check_launch("bridge_gemm");
}

}  // namespace

size_t a2v_bridge_ws_bytes(int B, int N, int Na, int heads) {
  const size_t D = (size_t)heads * 128;
  return align256((size_t)B * N * D * 2) + 2 * align256((size_t)B * Na * D * 2);
}

prism_status launch_a2v_bridge(const void* x_v, const void* x_a,
                               const void* w_q, const void* w_k,
                               const void* w_v, const void* w_o,
                               const float* pos_v, const float* pos_a, int B,
                               int N, int Na, int Cv, int Ca, int heads,
                               float rope_base, void* dh, void* ws,
                               hipStream_t stream) {
  const int D = heads * 128;
  char* w8 = static_cast<char*>(ws);
  uint16_t* qp = reinterpret_cast<uint16_t*>(w8);
  w8 += align256((size_t)B * N * D * 2);
  uint16_t* kp = reinterpret_cast<uint16_t*>(w8);
  w8 += align256((size_t)B * Na * D * 2);
  uint16_t* vp = reinterpret_cast<uint16_t*>(w8);
  const float lb = log2f(rope_base);
  const uint16_t* xv = static_cast<const uint16_t*>(x_v);
  const uint16_t* xa = static_cast<const uint16_t*>(x_a);
  prism_status st;
  if ((st = gemm(xv, static_cast<const uint16_t*>(w_q), B * N, D, Cv, qp,
                 pos_v, lb, stream)) != PRISM_OK)
    return st;
  if ((st = gemm(xa, static_cast<const uint16_t*>(w_k), B * Na, D, Ca, kp,
                 pos_a, lb, stream)) != PRISM_OK)
    return st;
  if ((st = gemm(xa, static_cast<const uint16_t*>(w_v), B * Na, D, Ca, vp,
                 nullptr, lb, stream)) != PRISM_OK)
    return st;
  const float sl2 = tiles::kLog2e / sqrtf(128.f);
  PRISM_LAUNCH("bridge_attn", bridge_attn, dim3((N + 63) / 64, heads, B),
               dim3(256), 0, stream, qp, kp, vp, qp, N, Na, D, sl2);
  if ((st = check_launch("bridge_attn")) != PRISM_OK) return st;
  return gemm(qp, static_cast<const uint16_t*>(w_o), B * N, Cv, D,
              static_cast<uint16_t*>(dh), nullptr, lb, stream);
}

}  // namespace prism
