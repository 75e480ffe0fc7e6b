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
//   bitmap_build    word-major column bitmaps: bit i of KV block j's word
//                   set when query block i selected j -- the KV->query
//                   lists, read in ascending i by the dK/dV kernel.
//   pairing         pairs of KV blocks and pairs of query blocks whose
//                   lists overlap most (pairing.hip).
//   dkdv_bf16       one workgroup per pair of KV blocks; loops over the
//                   union of the query blocks that selected them.
//   dq_bf16         one workgroup per pair of query blocks; loops over the
//                   union of their lists.
// Both use v_mfma_f32_32x32x16_bf16 tiles with fp32 accumulation, row-major
// swizzled LDS tiles with transposed fragments from ds_read_b64_tr_b16, and
// register-staged gathers (see attn_tiles.h); the fp32 dtype uses plain
// per-thread kernels with the same structure.
#include <algorithm>

#include "attn_tiles.h"

namespace prism {
namespace {

// D_r = <dO_r, O_r>: each thread takes one 16-byte piece of the row of O and
// of dO (8 bf16 or 4 fp32), a group of D*sizeof(E)/16 lanes reduces a row.
template <typename E, int D>
__global__ __launch_bounds__(256) void bwd_delta(const E* __restrict__ o,
                                                 const E* __restrict__ d_o,
                                                 long long rows,
                                                 float* __restrict__ delta) {
  constexpr int PER = 16 / (int)sizeof(E);   // elements per 16-byte piece
  constexpr int TPR = D / PER;               // threads per row (<= 64)
  const long long r = (long long)blockIdx.x * (256 / TPR) + threadIdx.x / TPR;
  const int part = threadIdx.x % TPR;
  float s = 0.f;
  if (r < rows) {
    const uint4 a = *reinterpret_cast<const uint4*>(o + r * D + part * PER);
    const uint4 g = *reinterpret_cast<const uint4*>(d_o + r * D + part * PER);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w};
    const uint32_t gv[4] = {g.x, g.y, g.z, g.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      if constexpr (sizeof(E) == 2) {
        s += __uint_as_float(av[t] << 16) * __uint_as_float(gv[t] << 16);
        s += __uint_as_float(av[t] & 0xffff0000u) *
             __uint_as_float(gv[t] & 0xffff0000u);
      } else {
        s += __uint_as_float(av[t]) * __uint_as_float(gv[t]);
      }
    }
  }
#pragma unroll
  for (int off = TPR / 2; off >= 1; off >>= 1) s += __shfl_xor(s, off, 64);
  if (r < rows && part == 0) delta[r] = s;
}

// ------------------------------------------------------- dK / dV (bf16)
// One workgroup (8 waves) per pair of KV blocks (pairs[p]: neighbours in the
// permuted order selected by largely the same query blocks).  The two column
// bitmaps are merged into one ascending union of query blocks (entries
// id | (selects the first) << 13 | (selects the second) << 14, 16 bits
// each) and each query block's Q, dO, lse and D are gathered once for both.
// Waves 0-3 own the pair's first KV block and waves 4-7 its second; within
// a half, wave (kh, qh) computes KV rows 32*kh .. +31 (K, V of the block resident in LDS, B
// operands) against query rows 32*qh .. +31.  A half skips the query blocks
// that did not select its KV block.  Q and dO are copied straight from HBM
// into two LDS slots (buffer loads with the LDS modifier, no staging
// registers), one union entry ahead; Q^T / dO^T fragments come from
// ds_read_b64_tr_b16.  The two qh waves of a KV half sum their partial dK /
// dV at the end.
template <int D>
__global__ __launch_bounds__(512, 2) void dkdv_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const uint32_t* __restrict__ bits,
    int words, const int2* __restrict__ pairs, int Hh, int N, long long heads,
    float scale, float* __restrict__ dk, float* __restrict__ dv) {
  using namespace tiles;
  using TL = Tile<D>;
  using SH = Share<D, 512>;
  constexpr int KS = D / 16, DT = D / 32;
  constexpr int KP = SH::kPerThread;
  // Q, dO of one union entry per slot (separate arrays, so reads of one
  // slot never wait for copies into the other), K, V of both KV blocks, the
  // lse / D rows of the two slots; the union list in dynamic LDS
  __shared__ __align__(16) unsigned char qo0[2 * TL::kBytes];
  __shared__ __align__(16) unsigned char qo1[2 * TL::kBytes];
  __shared__ __align__(16) unsigned char skv[4 * TL::kBytes];   // half h: K, V
  __shared__ __align__(16) float sx[256];                        // slot u: lse, D
  extern __shared__ __align__(16) unsigned char dyn[];
  uint16_t* ulist = reinterpret_cast<uint16_t*>(dyn);
  __shared__ int s_cnt[8];

  const int Nb = N / 64;
  long long bh;
  int pr;
  if (!xcd_item((Nb + 1) / 2, heads, bh, pr)) return;
  const int b = (int)(bh / Hh);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int kh = wave & 1, qh = (wave >> 1) & 1;
  const int c = lane & 31, hf = lane >> 5;
  const long long head = bh * N;
  const int32_t* pb = perm + (long long)b * N;
  const float sl2 = scale * kLog2e;
  const int2 pk = pairs[bh * ((Nb + 1) / 2) + pr];
  const int j0 = pk.x;
  const bool has_second = pk.y >= 0;
  const int j1 = has_second ? pk.y : j0;

  // ---- ascending union of the two columns (thread w owns word w)
  int ucnt = 0;
  {
    const uint32_t* col0 = bits + (bh * words + tid) * (long long)Nb + j0;
    const uint32_t wa = tid < words ? col0[0] : 0u;
    const uint32_t wb = (tid < words && has_second) ? col0[j1 - j0] : 0u;
    uint32_t wu = wa | wb;
    const int n = __popc(wu);
    int incl = n;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int x = __shfl_up(incl, off, 64);
      if (lane >= off) incl += x;
    }
    if (lane == 63) s_cnt[wave] = incl;
    __syncthreads();
    int pos = incl - n;
#pragma unroll
    for (int w = 0; w < 8; ++w) {
      const int x = s_cnt[w];
      pos += w < wave ? x : 0;
      ucnt += x;
    }
    while (wu) {
      const int bit = __ffs(wu) - 1;
      ulist[pos++] = (uint16_t)((tid * 32 + bit) | (((wa >> bit) & 1u) << 13) |
                                (((wb >> bit) & 1u) << 14));
      wu &= wu - 1u;
    }
  }
  {
    // K and V of both KV blocks stay in LDS for the whole kernel
    uint32_t o0[SH::kPerThread];
    Stage<D, 512> ks0, vs0;
    const __amdgpu_buffer_rsrc_t rk = head_rsrc<D>(k, head, N);
    const __amdgpu_buffer_rsrc_t rv = head_rsrc<D>(v, head, N);
    stage_offsets<D, 512>(o0, pb, j0, tid);
    stage_load<D, 512>(ks0, rk, o0);
    stage_load<D, 512>(vs0, rv, o0);
    stage_store<D, 512>(ks0, skv, tid);
    stage_store<D, 512>(vs0, skv + TL::kBytes, tid);
    stage_offsets<D, 512>(o0, pb, j1, tid);
    stage_load<D, 512>(ks0, rk, o0);
    stage_load<D, 512>(vs0, rv, o0);
    stage_store<D, 512>(ks0, skv + 2 * TL::kBytes, tid);
    stage_store<D, 512>(vs0, skv + 3 * TL::kBytes, tid);
  }
  __syncthreads();
  if (ucnt == 0) {
    // no query block selected either KV block: zero gradients
    if (qh == 0 && (half == 0 || has_second)) {
      const int kvr = pb[64 * (half ? j1 : j0) + 32 * kh + c];
      float4* dvr = reinterpret_cast<float4*>(dv + (head + kvr) * D);
      float4* dkr = reinterpret_cast<float4*>(dk + (head + kvr) * D);
      for (int e = hf; e < D / 4; e += 2) {
        dvr[e] = float4{0.f, 0.f, 0.f, 0.f};
        dkr[e] = float4{0.f, 0.f, 0.f, 0.f};
      }
    }
    return;
  }

  const int kvrow = pb[64 * (half ? j1 : j0) + 32 * kh + c];
  const int brow = 32 * kh + c;               // K / V row of this lane's column
  const unsigned char* skt = skv + half * 2 * TL::kBytes;
  const unsigned char* svt = skt + TL::kBytes;
  f32x16 dva[DT], dka[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) {
    dva[t] = f32x16{};
    dka[t] = f32x16{};
  }
  // C-layout register 4a + b of this lane holds query row
  // qbase(a) + b, qbase(a) = 32 qh + 16 (a / 2) + 8 hf + 4 (a % 2)
  const int arow = 32 * qh + slot_of(c);      // Q / dO row of this lane's M-row
  const uint32_t mflag = 1u << (13 + half);
  RowAddr ra_q = row_addr<D>(arow, hf), ra_k = row_addr<D>(brow, hf);
  TrAddr ta = tr_addr<D>(32 * qh, lane);

  // Q / dO tiles are copied into the two slots one union entry ahead; one
  // lse (tid < 64) or D (64 <= tid < 128) value per thread is staged one
  // entry ahead in a register (its row two entries ahead) and published
  // into the slot's lse / D row, lse scaled to log2 units
  const float* xsrc = (tid < 64 ? lse : delta) + head;
  const float xscale = tid < 64 ? kLog2e : 1.f;
  const __amdgpu_buffer_rsrc_t rq = head_rsrc<D>(q, head, N);
  const __amdgpu_buffer_rsrc_t ro = head_rsrc<D>(d_o, head, N);
  float xS = 0.f;
  uint32_t offn[KP];
  int xrow_n = 0;
  const int last = ucnt - 1;
  auto uid = [&](int t) __attribute__((always_inline)) -> int {
    return (int)(ulist[min(t, last)] & 0x1fffu);
  };
  auto xload = [&](int blk) __attribute__((always_inline)) -> int {
    return pb[64 * blk + (tid & 63)];
  };
  {
    // entry 0 copied into slot 0 with its lse / D row, entry 1's offsets
    // and lse / D value, entry 2's lse / D row.  Past the end of the list
    // the last block is re-fetched.
    int rows[KP];
    int u = uid(0);
    stage_rows<D, 512>(rows, pb, u, tid);
    dma_offsets<D, 512>(offn, rows, tid);
    stage_dma<D, 512>(qo0, rq, offn, tid);
    stage_dma<D, 512>(qo0 + TL::kBytes, ro, offn, tid);
    const float x0 = xsrc[xload(u)];
    if (tid < 128) sx[tid] = x0 * xscale;
    u = uid(1);
    stage_rows<D, 512>(rows, pb, u, tid);
    dma_offsets<D, 512>(offn, rows, tid);
    xS = xsrc[xload(u)];
    xrow_n = xload(uid(2));
  }

  auto compute_block = [&](const unsigned char* sq, const float* s_lse)
                           __attribute__((always_inline)) {
    const unsigned char* sdo = sq + TL::kBytes;
    const float* s_dlt = s_lse + 64;
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(lds_row_at<D>(sq, ra_q, ks), lds_row_at<D>(skt, ra_k, ks), s);
      dp = mfma32(lds_row_at<D>(sdo, ra_q, ks), lds_row_at<D>(svt, ra_k, ks), dp);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int qb = 32 * qh + 16 * (a >> 1) + 8 * hf + 4 * (a & 1);
      const float4 l4 = *reinterpret_cast<const float4*>(&s_lse[qb]);
      const float4 d4 = *reinterpret_cast<const float4*>(&s_dlt[qb]);
      const float lv[4] = {l4.x, l4.y, l4.z, l4.w};
      const float dv4[4] = {d4.x, d4.y, d4.z, d4.w};
#pragma unroll
      for (int bb = 0; bb < 4; ++bb) {
        const int r = 4 * a + bb;
        const float p = exp2_fast(fmaf(s[r], sl2, -lv[bb]));
        s[r] = p;
        dp[r] = p * (dp[r] - dv4[bb]);
      }
    }
    const bf16x8 p0 = pack8(s, 0), p1 = pack8(s, 1);
    const bf16x8 g0 = pack8(dp, 0), g1 = pack8(dp, 1);
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      dva[mt] = mfma32(lds_tr_at<D>(sdo, ta, 0, mt), p0, dva[mt]);
      dva[mt] = mfma32(lds_tr_at<D>(sdo, ta, 1, mt), p1, dva[mt]);
      dka[mt] = mfma32(lds_tr_at<D>(sq, ta, 0, mt), g0, dka[mt]);
      dka[mt] = mfma32(lds_tr_at<D>(sq, ta, 1, mt), g1, dka[mt]);
    }
  };

// One union entry t (in slot SLOT_, lse / D row XB_): once every wave's
// copies into that slot have landed, publish entry t+1's lse / D into the
// other row, load entry t+2's lse / D and rows and entry t+3's lse / D row
// (issued first: the waits for them leave the copies in flight), start
// copying entry t+1 into the other slot, compute entry t if it selected
// this half's KV block, then turn the rows into offsets.
#define PRISM_DKDV_STEP(T_, SLOT_, OTHER_, XB_)                             \
  {                                                                         \
    const int tt = (T_);                                                    \
    wait_loads();                                                           \
    __syncthreads();                                                        \
    if (tid < 128) sx[(1 - (XB_)) * 128 + tid] = xS * xscale;               \
    const float x_n = xsrc[xrow_n];                                         \
    int rows_n[KP];                                                         \
    stage_rows<D, 512>(rows_n, pb, uid(tt + 2), tid);                       \
    const int xrow_nn = xload(uid(tt + 3));                                 \
    pin_order();                                                            \
    stage_dma<D, 512>(OTHER_, rq, offn, tid);                               \
    stage_dma<D, 512>(OTHER_ + TL::kBytes, ro, offn, tid);                  \
    pin_order();                                                            \
    const uint32_t e = __builtin_amdgcn_readfirstlane((uint32_t)ulist[tt]); \
    opaque(ra_q);                                                           \
    opaque(ra_k);                                                           \
    opaque(ta);                                                             \
    if (e & mflag) compute_block(SLOT_, sx + (XB_) * 128);                  \
    dma_offsets<D, 512>(offn, rows_n, tid);                                 \
    xS = x_n;                                                               \
    xrow_n = xrow_nn;                                                       \
  }

  int t = 0;
  for (; t + 1 < ucnt; t += 2) {
    PRISM_DKDV_STEP(t, qo0, qo1, 0)
    PRISM_DKDV_STEP(t + 1, qo1, qo0, 1)
  }
  if (t < ucnt) PRISM_DKDV_STEP(t, qo0, qo1, 0)
#undef PRISM_DKDV_STEP
  // the copies issued past the end of the list land before the slots are
  // reused below
  wait_loads();

  // sum the two qh partials of each KV half: qh = 1 hands over through LDS
  // (half h uses slot h), one tensor at a time (2 waves x 64 lanes x D/2
  // floats = 2 * kBytes per half)
  float* xch = reinterpret_cast<float*>(half ? qo1 : qo0);
  float* dvr = dv + (head + kvrow) * D;
  float* dkr = dk + (head + kvrow) * D;
  const bool write = half == 0 || has_second;
  for (int pass = 0; pass < 2; ++pass) {
    f32x16* acc = pass == 0 ? dva : dka;
    __syncthreads();
    if (qh == 1) {
#pragma unroll
      for (int mt = 0; mt < DT; ++mt)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          xch[((kh * 64 + lane) * DT + mt) * 16 + r] = acc[mt][r];
    }
    __syncthreads();
    if (qh == 0 && write) {
      float* out = pass == 0 ? dvr : dkr;
      const float f = pass == 0 ? 1.f : scale;
#pragma unroll
      for (int mt = 0; mt < DT; ++mt)
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          float4 o4;
          const float* x = &xch[((kh * 64 + lane) * DT + mt) * 16 + 4 * a];
          o4.x = (acc[mt][4 * a + 0] + x[0]) * f;
          o4.y = (acc[mt][4 * a + 1] + x[1]) * f;
          o4.z = (acc[mt][4 * a + 2] + x[2]) * f;
          o4.w = (acc[mt][4 * a + 3] + x[3]) * f;
          *reinterpret_cast<float4*>(out + 32 * mt + 8 * a + 4 * hf) = o4;
        }
    }
  }
}

// ------------------------------------------------------------ dQ (bf16)
// One workgroup (8 waves) per pair of query blocks, as in the forward: the
// union of the two lists is gathered once, waves 0-3 own the pair's first
// query block and waves 4-7 its second, wave (qh, kh) of a half computes S^T
// and dP^T per 32x32 tile and dQ^T += K^T dS^T with K^T fragments from
// ds_read_b64_tr_b16.  K and V go through two LDS buffers, staged two
// blocks ahead in registers.
template <int D>
__global__ __launch_bounds__(512, 2) void dq_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const uint16_t* __restrict__ d_o,
    const float* __restrict__ lse, const float* __restrict__ delta,
    const int32_t* __restrict__ perm, const int32_t* __restrict__ counts,
    const int32_t* __restrict__ kv_idx, int capacity,
    const int2* __restrict__ pairs, int Hh, int N, long long heads, float scale,
    float* __restrict__ dq) {
  using namespace tiles;
  using TL = Tile<D>;
  using SH = Share<D, 512>;
  constexpr int KS = D / 16, DT = D / 32;
  const int Nb = N / 64;
  extern __shared__ __align__(16) unsigned char dyn[];
  unsigned char* smem = dyn;                    // two (K, V) buffers
  uint16_t* ulist = reinterpret_cast<uint16_t*>(dyn + 4 * TL::kBytes);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ulist + ((Nb + 1) & ~1));
  __shared__ int s_cnt[8];

  long long bh;
  int pr;
  if (!xcd_item((Nb + 1) / 2, heads, bh, pr)) return;
  const int b = (int)(bh / Hh);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int qh = wave & 1, kh = (wave >> 1) & 1;
  const int c = lane & 31, hf = lane >> 5, j16 = lane & 15, grp = lane >> 4;
  const long long head = bh * N;
  const int32_t* pb = perm + (long long)b * N;
  const float sl2 = scale * kLog2e;
  const int2 pq = pairs[bh * ((Nb + 1) / 2) + pr];
  const int i0 = pq.x;
  const bool has_second = pq.y >= 0;
  const int i1 = has_second ? pq.y : i0;
  const long long row0 = bh * Nb + i0, row1 = bh * Nb + i1;
  const int cnt0 = counts[row0];
  const int cnt1 = has_second ? counts[row1] : 0;
  const int32_t* lst0 = kv_idx + row0 * (long long)capacity;
  const int32_t* lst1 = kv_idx + row1 * (long long)capacity;
  const int ucnt = pair_union(lst0, cnt0, lst1, cnt1, Nb, bits, ulist, s_cnt,
                              tid);

  const int iq = half == 1 ? i1 : i0;
  const int qrow = pb[64 * iq + 32 * qh + c];
  bf16x8 qreg[KS], doreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks) {
    qreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(q + (head + qrow) * D + 16 * ks + 8 * hf));
    doreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(d_o + (head + qrow) * D + 16 * ks + 8 * hf));
  }
  const float lse2 = lse[head + qrow] * kLog2e;
  const float dlt = delta[head + qrow];
  const uint32_t mflag = 1u << (13 + half);
  f32x16 dqa[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) dqa[t] = f32x16{};
  const int arow = 32 * kh + slot_of(c);

  Stage<D, 512> kA, vA, kB, vB;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc<D>(k, head, N);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc<D>(v, head, N);
  uint32_t offs_n[SH::kPerThread];
  // an empty union leaves ulist[0] = block 0 (pair_union): a safe id for
  // the prologue's loads, and the loop runs no step (dq = 0)
  const int last = max(ucnt - 1, 0);
  auto uid = [&](int t) __attribute__((always_inline)) -> int {
    return (int)(ulist[min(t, last)] & 0x1fffu);
  };
  int j_n = 0;
  {
    uint32_t o0[SH::kPerThread];
    stage_offsets<D, 512>(o0, pb, uid(0), tid);
    stage_load<D, 512>(kA, rk, o0);
    stage_load<D, 512>(vA, rv, o0);
    stage_offsets<D, 512>(o0, pb, uid(1), tid);
    stage_load<D, 512>(kB, rk, o0);
    stage_load<D, 512>(vB, rv, o0);
    stage_store<D, 512>(kA, smem, tid);
    stage_store<D, 512>(vA, smem + TL::kBytes, tid);
    stage_offsets<D, 512>(o0, pb, uid(2), tid);
    stage_load<D, 512>(kA, rk, o0);
    stage_load<D, 512>(vA, rv, o0);
    stage_offsets<D, 512>(offs_n, pb, uid(3), tid);
    j_n = uid(4);
  }

  auto compute_block = [&](const unsigned char* sk, const unsigned char* sv)
                           __attribute__((always_inline)) {
    f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s = mfma32(lds_row8<D>(sk, arow, 2 * ks + hf), qreg[ks], s);
      dp = mfma32(lds_row8<D>(sv, arow, 2 * ks + hf), doreg[ks], dp);
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const float p = exp2_fast(fmaf(s[r], sl2, -lse2));
      dp[r] = p * (dp[r] - dlt);
    }
    const bf16x8 g0 = pack8(dp, 0), g1 = pack8(dp, 1);
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const int d0 = 32 * mt + 16 * (grp & 1);
      const int r0 = 32 * kh + 8 * (grp >> 1);
      dqa[mt] = mfma32(lds_tr8<D>(sk, r0, d0, j16), g0, dqa[mt]);
      dqa[mt] = mfma32(lds_tr8<D>(sk, r0 + 16, d0, j16), g1, dqa[mt]);
    }
  };

#define PRISM_DQ_STEP(T_, BUF_, KS_, VS_)                                   \
  {                                                                         \
    const int tt = (T_);                                                    \
    __syncthreads();                                                        \
    stage_store<D, 512>(KS_, smem + (1 - (BUF_)) * 2 * TL::kBytes, tid);    \
    stage_store<D, 512>(VS_, smem + (1 - (BUF_)) * 2 * TL::kBytes +         \
                                 TL::kBytes, tid);                          \
    int rows_n[SH::kPerThread];                                             \
    stage_rows<D, 512>(rows_n, pb, j_n, tid);                               \
    pin_order();                                                            \
    stage_load<D, 512>(KS_, rk, offs_n);                                    \
    stage_load<D, 512>(VS_, rv, offs_n);                                    \
    pin_order();                                                            \
    j_n = uid(tt + 5);                                                      \
    const uint32_t e = __builtin_amdgcn_readfirstlane((uint32_t)ulist[tt]); \
    if (e & mflag)                                                          \
      compute_block(smem + (BUF_) * 2 * TL::kBytes,                         \
                    smem + (BUF_) * 2 * TL::kBytes + TL::kBytes);           \
    rows_to_offsets<D, 512>(offs_n, rows_n, tid);                           \
  }

  int t = 0;
  for (; t + 1 < ucnt; t += 2) {
    PRISM_DQ_STEP(t, 0, kB, vB)
    PRISM_DQ_STEP(t + 1, 1, kA, vA)
  }
  if (t < ucnt) PRISM_DQ_STEP(t, 0, kB, vB)
#undef PRISM_DQ_STEP

  // sum the two kh partials of each query half through LDS
  __syncthreads();
  float* xch = reinterpret_cast<float*>(smem + half * 2 * TL::kBytes);
  if (kh == 1) {
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xch[((qh * 64 + lane) * DT + mt) * 16 + r] = dqa[mt][r];
  }
  __syncthreads();
  if (kh == 0 && (half == 0 || has_second)) {
    float* dqr = dq + (head + qrow) * D;
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const float* x = &xch[((qh * 64 + lane) * DT + mt) * 16 + 4 * a];
        float4 o4;
        o4.x = (dqa[mt][4 * a + 0] + x[0]) * scale;
        o4.y = (dqa[mt][4 * a + 1] + x[1]) * scale;
        o4.z = (dqa[mt][4 * a + 2] + x[2]) * scale;
        o4.w = (dqa[mt][4 * a + 3] + x[3]) * scale;
        *reinterpret_cast<float4*>(dqr + 32 * mt + 8 * a + 4 * hf) = o4;
      }
  }
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
  // counts clamped to [0, Nb], ids outside [0, Nb) skipped, as the column
  // bitmap that dkdv_f32 reads does
  const int cnt = min(max(counts[rowid], 0), Nb);
  const int32_t* lst = kv_idx + rowid * (long long)capacity;
  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    if ((unsigned)j >= (unsigned)Nb) continue;
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
  const uint32_t* col = bits + ((long long)b * Hh + h) * words * (long long)Nb + j;
  for (int w = 0; w < words; ++w) {
    uint32_t word = col[(long long)w * Nb];
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


template <int D>
prism_status run_bwd(const void* q, const void* k, const void* v,
                     const void* o, const void* d_o, const float* lse,
                     int dtype, const int32_t* perm, const int32_t* counts,
                     const int32_t* kv_idx, int capacity, int B, int Hh, int N,
                     float scale, float* dq, float* dk, float* dv, void* ws,
                     hipStream_t stream) {
  const int Nb = N / 64;
  const int words = (Nb + 31) / 32;
  const long long rows = (long long)B * Hh * N;
  // workspace: D rows | column bitmap | row bitmap | pairing scratch |
  // query-block pairs | KV-block pairs
  char* w8 = static_cast<char*>(ws);
  float* delta = reinterpret_cast<float*>(w8);
  w8 += align256(rows * sizeof(float));
  uint32_t* bits = reinterpret_cast<uint32_t*>(w8);
  w8 += bitmap_bytes(B, Hh, Nb);
  uint32_t* rowbits = reinterpret_cast<uint32_t*>(w8);
  w8 += bitmap_bytes(B, Hh, Nb);
  void* pws = w8;
  w8 += block_pairs_ws_bytes(B, Hh, Nb);
  int2* qpairs = reinterpret_cast<int2*>(w8);
  w8 += block_pairs_bytes(B, Hh, Nb);
  int2* kpairs = reinterpret_cast<int2*>(w8);

  if (dtype == PRISM_BF16) {
    const long long rpb = 256 / (D / 8);      // rows per block
    PRISM_LAUNCH("bwd_delta", (bwd_delta<uint16_t, D>),
                 dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                 (const uint16_t*)o, (const uint16_t*)d_o, rows, delta);
  } else {
    const long long rpb = 256 / (D / 4);
    PRISM_LAUNCH("bwd_delta", (bwd_delta<float, D>),
                 dim3((unsigned)((rows + rpb - 1) / rpb)), dim3(256), 0, stream,
                 (const float*)o, (const float*)d_o, rows, delta);
  }
  prism_status st = check_launch("bwd_delta");
  if (st != PRISM_OK) return st;
  if ((st = launch_column_bitmap(counts, kv_idx, capacity, B, Hh, Nb, bits,
                                 stream)) != PRISM_OK)
    return st;

  dim3 grid(Nb, Hh, B);
  if (dtype == PRISM_BF16) {
    if ((st = launch_block_pairs(bits, B, Hh, Nb, pws, kpairs, stream)) != PRISM_OK)
      return st;
    if ((st = launch_bitmap_transpose(bits, B, Hh, Nb, rowbits, stream)) != PRISM_OK)
      return st;
    if ((st = launch_block_pairs(rowbits, B, Hh, Nb, pws, qpairs, stream)) != PRISM_OK)
      return st;
    const long long heads = (long long)B * Hh;
    const dim3 gp(tiles::xcd_grid((Nb + 1) / 2, heads));
    // the 16-bit union list (tiles and lse / D rows are static LDS)
    const size_t dyn = (size_t)Nb * sizeof(uint16_t);
    PRISM_LAUNCH("dkdv_bf16", dkdv_bf16<D>, gp, dim3(512), dyn, stream,
                 (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                 (const uint16_t*)d_o, lse, delta, perm, bits, words, kpairs, Hh, N,
                 heads, scale, dk, dv);
    if ((st = check_launch("dkdv_bf16")) != PRISM_OK) return st;
    const size_t dyn_q = 4 * tiles::Tile<D>::kBytes + 2 * (size_t)((Nb + 1) & ~1) +
                         8 * (size_t)((Nb + 31) / 32);
    PRISM_LAUNCH("dq_bf16", dq_bf16<D>, gp, dim3(512), dyn_q, stream, (const uint16_t*)q,
                 (const uint16_t*)k, (const uint16_t*)v, (const uint16_t*)d_o,
                 lse, delta, perm, counts, kv_idx, capacity, qpairs, Hh, N, heads,
                 scale, dq);
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
  const int Nb = N / 64;
  return align256(rows * sizeof(float)) + 2 * bitmap_bytes(B, Hh, Nb) +
         block_pairs_ws_bytes(B, Hh, Nb) + 2 * block_pairs_bytes(B, Hh, Nb);
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
