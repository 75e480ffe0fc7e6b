// Stage 4, forward: block-sparse attention with online softmax over the
// selected KV blocks only.
//
// The abstract page ("Prism: Dynamic Sparse Attention ...") describes
// sparse attention that computes only the selected key/value blocks inside
// one online-softmax pass; README "Overview": each query block has its own
// budget of blocks.
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16, fp32 accumulation):
//   every wave computes S^T = K Q^T (kv x q), so a lane holds 16 scores of
//   one query per 32-key tile and the row statistics need one cross-lane
//   step; the K rows
//   feeding the M-rows are ordered (tiles::slot_of) so that the lane's
//   probabilities are already the B operand of O^T += V^T P^T -- P never
//   goes through LDS.
// fp32 path: one thread per query row, plain fp32 arithmetic (reference
//   precision for small problems).
#include "attn_tiles.h"

namespace prism {
namespace {

// One workgroup of 4 waves per pair of query blocks (pairs[p]: neighbours
// in the permuted order whose lists overlap most, see pairing.hip), two
// workgroups per CU (64 KiB of tiles + 2 Nb bytes of list each: two fit for
// Nb below 8184).  The two lists are merged into one ascending union in
// LDS; each K/V block of the union is gathered from HBM once and serves both
// query blocks, so the gather traffic drops to the union's share.  Waves 0-1
// own the pair's first query block and waves 2-3 its second; wave qh of a
// half computes queries 32*qh .. +31 against all 64 KV rows of every block
// it holds (two 32x32 score tiles, each reused over a 128-deep
// contraction), so a query's whole row of a block lives in one wave and the
// online softmax needs no merge.  A half skips the union blocks its own list
// does not hold.  Each SIMD runs one wave of each of the CU's two
// workgroups: they wait at different barriers, so one's MFMA work can run
// beside the other's softmax.  K and V stay row-major in LDS (V^T fragments
// come from ds_read_b64_tr_b16), copied straight from HBM into two slots
// (buffer loads with the LDS modifier, no staging registers): the next
// union entry lands in one slot while the current one is read from the
// other.
template <int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, const int2* __restrict__ pairs, int Hh, int N,
    long long total /* B * Hh */, float scale_log2,
    const float* __restrict__ drop_lse, const float* __restrict__ drop_v,
    uint16_t* __restrict__ o, float* __restrict__ lse) {
  using namespace tiles;
  using TL = Tile<D>;
  using SH = Share<D, 256>;
  constexpr int KS = D / 16;     // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;     // 32-row d tiles of O^T
  constexpr int KP = SH::kPerThread;
  const int Nb = N / 64;
  // LDS: two K/V slots (K, then V of one block) as separate arrays, so the
  // compiler sees that reads of one slot never wait for copies into the
  // other; the union list in dynamic LDS.  The union's membership bitmaps
  // live in slot 0 while the list is built (before any tile is copied).
  __shared__ __align__(16) unsigned char slot0[2 * TL::kBytes];
  __shared__ __align__(16) unsigned char slot1[2 * TL::kBytes];
  extern __shared__ __align__(16) unsigned char dyn[];
  uint16_t* ulist = reinterpret_cast<uint16_t*>(dyn);
  uint32_t* bits = reinterpret_cast<uint32_t*>(slot0);
  __shared__ int s_cnt[4];

  long long bh;
  int pr;
  if (!xcd_item((Nb + 1) / 2, total, bh, pr)) return;
  const int b = (int)(bh / Hh);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(wave >> 1);
  const int qh = wave & 1;
  const int c = lane & 31, hf = lane >> 5, j16 = lane & 15, grp = lane >> 4;
  const long long head = bh * N;
  const int32_t* pb = perm + (long long)b * N;
  const int2 pq = pairs[bh * ((Nb + 1) / 2) + pr];
  const int i0 = pq.x;
  const bool has_second = pq.y >= 0;     // odd Nb: one pair is a single
  const int i1 = has_second ? pq.y : i0;
  const long long row0 = bh * Nb + i0;
  const int cnt0 = counts[row0];
  const int cnt1 = has_second ? counts[bh * Nb + i1] : 0;
  const int32_t* lst0 = kv_idx + row0 * (long long)capacity;
  const int32_t* lst1 = kv_idx + (bh * Nb + i1) * (long long)capacity;

  const int ucnt = pair_union<256>(lst0, cnt0, lst1, cnt1, Nb, bits, ulist, s_cnt, tid);

  // a missing second block borrows the first one's rows (never written)
  const int iq = half == 1 ? i1 : i0;
  const int qrow = pb[64 * iq + 32 * qh + c];
  bf16x8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(
        q + (head + qrow) * D + 16 * ks + 8 * hf));
  const uint32_t mflag = 1u << (13 + half);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  // K rows feeding this lane's M-rows of the two score tiles
  const int krow0 = slot_of(c), krow1 = 32 + slot_of(c);

  const __amdgpu_buffer_rsrc_t rk = head_rsrc<D>(k, head, N);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc<D>(v, head, N);
  uint32_t offn[KP];
  // an empty union leaves ulist[0] = block 0 (pair_union), a safe id for
  // the prologue's loads; the loop then runs no step
  const int last = max(ucnt - 1, 0);
  auto uid = [&](int t) __attribute__((always_inline)) -> int {
    return (int)(ulist[min(t, last)] & 0x1fffu);
  };
  // prologue: entry 0 copied into slot 0, offsets of entry 1.  Past the end
  // of the list the last block is re-fetched, so the loop body has no
  // branches around the loads and the wait counters stay exact.
  {
    int rows[KP];
    stage_rows<D, 256>(rows, pb, uid(0), tid);
    dma_offsets<D, 256>(offn, rows, tid);
    stage_dma<D, 256>(slot0, rk, offn, tid);
    stage_dma<D, 256>(slot0 + TL::kBytes, rv, offn, tid);
    stage_rows<D, 256>(rows, pb, uid(1), tid);
    dma_offsets<D, 256>(offn, rows, tid);
  }

  // one block: S^T (64 kv x 32 q, two tiles), online softmax over the 64
  // keys, O^T (d x 32 q) += V^T P^T
  auto compute_block = [&](const unsigned char* sk) __attribute__((always_inline)) {
    const unsigned char* sv = sk + TL::kBytes;
    f32x16 s0 = f32x16{}, s1 = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) {
      s0 = mfma32(lds_row8<D>(sk, krow0, 2 * ks + hf), qreg[ks], s0);
      s1 = mfma32(lds_row8<D>(sk, krow1, 2 * ks + hf), qreg[ks], s1);
    }
    // online softmax in the log2 domain (scale > 0, so the max of the raw
    // scores is the max of the scaled ones).  The exponent reference only
    // moves when a block's max exceeds it by more than 8: until then the
    // probabilities stay <= 2^8 (exact range in fp32 and bf16) and the
    // accumulator needs no rescale.
    float mx = fmax_prop(s0[0], s1[0]);
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmax_prop(mx, fmax_prop(s0[r], s1[r]));
    mx = xor32_max(mx) * scale_log2;
    const float m_new = mx > m_run + 8.f ? mx : m_run;
    const float alpha = exp2_fast(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = exp2_fast(fmaf(s0[r], scale_log2, -m_new));
      s1[r] = exp2_fast(fmaf(s1[r], scale_log2, -m_new));
      rs += s0[r] + s1[r];
    }
    rs = xor32_sum(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {      // the reference moved for some query
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) oacc[t2] *= alpha;
    }
    const bf16x8 p00 = pack8(s0, 0), p01 = pack8(s0, 1);
    const bf16x8 p10 = pack8(s1, 0), p11 = pack8(s1, 1);
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const int d0 = 32 * mt + 16 * (grp & 1);
      const int r0 = 8 * (grp >> 1);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0, d0, j16), p00, oacc[mt]);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0 + 16, d0, j16), p01, oacc[mt]);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0 + 32, d0, j16), p10, oacc[mt]);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0 + 48, d0, j16), p11, oacc[mt]);
    }
  };

// One union entry t (in slot SLOT_): once every wave's copies into that
// slot have landed, start copying entry t+1 into the other slot, load the
// rows of entry t+2 (issued first: the wait for them then leaves the copy
// in flight), compute entry t if this half's list holds it, then turn the
// rows into offsets.
#define PRISM_FWD_STEP(T_, SLOT_, OTHER_)                                   \
  {                                                                         \
    const int tt = (T_);                                                    \
    wait_loads();                                                           \
    __syncthreads();                                                        \
    int rows_n[KP];                                                         \
    stage_rows<D, 256>(rows_n, pb, uid(tt + 2), tid);                       \
    pin_order();                                                            \
    stage_dma<D, 256>(OTHER_, rk, offn, tid);                               \
    stage_dma<D, 256>(OTHER_ + TL::kBytes, rv, offn, tid);                  \
    pin_order();                                                            \
    const uint32_t e = __builtin_amdgcn_readfirstlane((uint32_t)ulist[tt]); \
    if (e & mflag) compute_block(SLOT_);                                    \
    dma_offsets<D, 256>(offn, rows_n, tid);                                 \
  }

  // slot 0 at even entries, slot 1 at odd ones
  int t = 0;
  for (; t + 1 < ucnt; t += 2) {
    PRISM_FWD_STEP(t, slot0, slot1)
    PRISM_FWD_STEP(t + 1, slot1, slot0)
  }
  if (t < ucnt) PRISM_FWD_STEP(t, slot0, slot1)
#undef PRISM_FWD_STEP
  // the copies issued past the end of the list land before the workgroup
  // ends (nothing reads them)
  wait_loads();

  if (half == 0 || has_second) {
    float m = m_run, l = l_run;
    // m = -inf: the query block's list is empty (no key at all)
    const bool none = m == -INFINITY;
    // optional stand-in of the blocks this query block did not keep: weight
    // exp(drop_lse) (natural log) with value drop_v, one more term of the
    // same softmax
    float b1 = 1.f, b2 = 0.f;
    const float* dvr = nullptr;
    if (drop_lse != nullptr) {
      const float dl = drop_lse[bh * Nb + iq] * kLog2e;
      const float mm = fmaxf(m, dl);
      b1 = none ? 0.f : exp2_fast(m - mm);
      b2 = dl == -INFINITY ? 0.f : exp2_fast(dl - mm);
      m = mm;
      l = l * b1 + b2;
      dvr = drop_v + (bh * Nb + iq) * D;
    }
    // no key and no stand-in: o = 0, lse = -inf
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
    uint16_t* orow = o + (head + qrow) * D;
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        float vals[4];
#pragma unroll
        for (int bb = 0; bb < 4; ++bb) {
          const int r = 4 * a + bb;
          const float x = oacc[mt][r];
          vals[bb] = dvr ? (x * b1 + b2 * dvr[32 * mt + 8 * a + 4 * hf + bb]) * inv_l
                         : x * inv_l;
        }
        uint2 pk;
        pk.x = cvt2(vals[0], vals[1]);
        pk.y = cvt2(vals[2], vals[3]);
        *reinterpret_cast<uint2*>(orow + 32 * mt + 8 * a + 4 * hf) = pk;
      }
    if (hf == 0) lse[head + qrow] = l > 0.f ? (m + log2f(l)) * kLn2 : -INFINITY;
  }
}

// fp32 reference-precision path: one thread per query row.
template <int D>
__global__ __launch_bounds__(64) void attn_fwd_f32(
    const float* __restrict__ q, const float* __restrict__ k,
    const float* __restrict__ v, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, int Hh, int N, float scale,
    const float* __restrict__ drop_lse, const float* __restrict__ drop_v,
    float* __restrict__ o, float* __restrict__ lse) {
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
  // counts are clamped to [0, Nb]; ids outside [0, Nb) are skipped
  const int cnt = min(max(counts[rowid], 0), Nb);
  const int32_t* lst = kv_idx + rowid * (long long)capacity;
  for (int t = 0; t < cnt; ++t) {
    const int j = lst[t];
    if ((unsigned)j >= (unsigned)Nb) continue;
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
  if (drop_lse != nullptr) {
    // stand-in of the blocks this query block did not keep
    const float dl = drop_lse[rowid];
    const float mm = fmaxf(m_run, dl);
    const float b1 = m_run == -INFINITY ? 0.f : expf(m_run - mm);
    const float b2 = dl == -INFINITY ? 0.f : expf(dl - mm);
    const float l = l_run * b1 + b2;
    const float* dvr = drop_v + rowid * D;
    const float inv_l = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e)
      o[(head + qrow) * D + e] = (acc[e] * b1 + b2 * dvr[e]) * inv_l;
    lse[head + qrow] = l > 0.f ? mm + logf(l) : -INFINITY;
    return;
  }
  // an empty list: o = 0, lse = -inf
  const float inv_l = l_run > 0.f ? 1.f / l_run : 0.f;
#pragma unroll
  for (int e = 0; e < D; ++e) o[(head + qrow) * D + e] = acc[e] * inv_l;
  lse[head + qrow] = l_run > 0.f ? m_run + logf(l_run) : -INFINITY;
}

}  // namespace

size_t attn_fwd_ws_bytes(int B, int Hh, int N, int d) {
  (void)d;
  const int Nb = N / 64;
  return 2 * bitmap_bytes(B, Hh, Nb) + block_pairs_ws_bytes(B, Hh, Nb) +
         block_pairs_bytes(B, Hh, Nb);
}

prism_status launch_attn_fwd(const void* q, const void* k, const void* v,
                             int dtype, const int32_t* perm,
                             const int32_t* counts, const int32_t* kv_idx,
                             int capacity, int B, int Hh, int N, int d,
                             float scale, const float* drop_lse,
                             const float* drop_v, void* o, float* lse,
                             void* ws, hipStream_t stream) {
  dim3 grid(N / 64, Hh, B);
  if (dtype == PRISM_BF16) {
    const float sl2 = scale * tiles::kLog2e;
    const long long total = (long long)B * Hh;   // (batch, head) pairs
    const int Nb = N / 64;
    // pair the query blocks: column bitmap -> row bitmap -> matching
    char* w8 = static_cast<char*>(ws);
    uint32_t* colbits = reinterpret_cast<uint32_t*>(w8);
    uint32_t* rowbits = reinterpret_cast<uint32_t*>(w8 + bitmap_bytes(B, Hh, Nb));
    void* pws = w8 + 2 * bitmap_bytes(B, Hh, Nb);
    int2* pairs = reinterpret_cast<int2*>(static_cast<char*>(pws) +
                                          block_pairs_ws_bytes(B, Hh, Nb));
    prism_status st = launch_column_bitmap(counts, kv_idx, capacity, B, Hh, Nb,
                                           colbits, stream);
    if (st != PRISM_OK) return st;
    if ((st = launch_bitmap_transpose(colbits, B, Hh, Nb, rowbits, stream)) != PRISM_OK)
      return st;
    if ((st = launch_block_pairs(rowbits, B, Hh, Nb, pws, pairs, stream)) != PRISM_OK)
      return st;
    const dim3 g1(tiles::xcd_grid((Nb + 1) / 2, total));
    if (d == 128) {
      // the 16-bit union list (the tiles are static LDS)
      const size_t dyn = 2 * (size_t)Nb;
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<128>, g1, dim3(256), dyn, stream,
                   (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                   perm, counts, kv_idx, capacity, pairs, Hh, N, total, sl2,
                   drop_lse, drop_v, (uint16_t*)o, lse);
    } else {
      const size_t dyn = 2 * (size_t)Nb;
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<64>, g1, dim3(256), dyn, stream,
                   (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                   perm, counts, kv_idx, capacity, pairs, Hh, N, total, sl2,
                   drop_lse, drop_v, (uint16_t*)o, lse);
    }
  } else {
    if (d == 128)
      PRISM_LAUNCH("attn_fwd_f32", attn_fwd_f32<128>, grid, dim3(64), 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, perm,
                         counts, kv_idx, capacity, Hh, N, scale, drop_lse, drop_v,
                         (float*)o, lse);
    else
      PRISM_LAUNCH("attn_fwd_f32", attn_fwd_f32<64>, grid, dim3(64), 0, stream,
                         (const float*)q, (const float*)k, (const float*)v, perm,
                         counts, kv_idx, capacity, Hh, N, scale, drop_lse, drop_v,
                         (float*)o, lse);
  }
  return check_launch("attn_fwd");
}

}  // namespace prism
