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
//   one query and the row statistics need one cross-lane step; the K rows
//   feeding the M-rows are ordered (tiles::slot_of) so that the lane's
//   probabilities are already the B operand of O^T += V^T P^T -- P never
//   goes through LDS.
// fp32 path: one thread per query row, plain fp32 arithmetic (reference
//   precision for small problems).
#include "attn_tiles.h"

namespace prism {
namespace {

// One workgroup (8 waves) per pair of query blocks (pairs[p]: neighbours in
// the permuted order whose lists overlap most, see pairing.hip).  The two
// lists are merged into one ascending union in LDS; each K/V block of the
// union is gathered from HBM once and serves both query blocks, so the
// gather traffic drops to the union's share.  Waves 0-3 own the pair's
// first query block and waves 4-7 its second; within a half, wave (qh, kh) computes queries 32*qh .. +31 against KV rows
// 32*kh .. +31 of every block, so each 32x32 MFMA tile is reused over a
// 128-deep (S) or 32-deep (P*V) contraction.  A half skips the union blocks
// its own list does not hold.  The two kh waves of a query half keep
// separate online-softmax states, merged once at the end (exactly as a
// split over KV).  K and V stay row-major in LDS; V^T fragments come from
// ds_read_b64_tr_b16.  Blocks are staged two ahead through registers.
template <int D>
__global__ __launch_bounds__(512, 2) void attn_fwd_bf16(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ perm,
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, const int2* __restrict__ pairs, int Hh, int N,
    long long total /* B * Hh */, float scale_log2,
    const float* __restrict__ drop_lse, const float* __restrict__ drop_v,
    uint16_t* __restrict__ o, float* __restrict__ lse) {
  using namespace tiles;
  using TL = Tile<D>;
  using SH = Share<D, 512>;
  constexpr int KS = D / 16;     // k-steps of S^T = K Q^T
  constexpr int DT = D / 32;     // 32-row d tiles of O^T
  const int Nb = N / 64;
  // two LDS buffers (K and V of one block each): block t+1 is published into
  // one while block t is read from the other -- one barrier per block.  Then
  // the union list (one entry per block: id | in-first << 16 |
  // in-second << 17) and the two membership bitmaps.
  extern __shared__ __align__(16) unsigned char dyn[];
  unsigned char* smem = dyn;
  uint32_t* ulist = reinterpret_cast<uint32_t*>(dyn + 4 * TL::kBytes);
  uint32_t* bits = ulist + Nb;
  __shared__ float sm_m[2][2][32], sm_l[2][2][32];
  __shared__ int s_cnt[8];

  long long bh;
  int pr;
  if (!xcd_item((Nb + 1) / 2, total, bh, pr)) return;
  const int b = (int)(bh / Hh);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int half = __builtin_amdgcn_readfirstlane(wave >> 2);
  const int qh = wave & 1, kh = (wave >> 1) & 1;
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

  const int ucnt = pair_union(lst0, cnt0, lst1, cnt1, Nb, bits, ulist, s_cnt, tid);

  // a missing second block borrows the first one's rows (never written)
  const int iq = half == 1 ? i1 : i0;
  const int qrow = pb[64 * iq + 32 * qh + c];
  bf16x8 qreg[KS];
#pragma unroll
  for (int ks = 0; ks < KS; ++ks)
    qreg[ks] = as_bf16x8(*reinterpret_cast<const u32x4*>(
        q + (head + qrow) * D + 16 * ks + 8 * hf));
  const uint32_t mflag = 1u << (16 + half);

  float m_run = -INFINITY, l_run = 0.f;
  f32x16 oacc[DT];
#pragma unroll
  for (int t = 0; t < DT; ++t) oacc[t] = f32x16{};
  const int krow = 32 * kh + slot_of(c);   // K row feeding this lane's M-row

  Stage<D, 512> kA, vA, kB, vB;
  const __amdgpu_buffer_rsrc_t rk = head_rsrc<D>(k, head, N);
  const __amdgpu_buffer_rsrc_t rv = head_rsrc<D>(v, head, N);
  uint32_t offs_n[SH::kPerThread];
  // an empty union leaves ulist[0] = block 0 (pair_union), a safe id for
  // the prologue's loads; the loop then runs no step
  const int last = max(ucnt - 1, 0);
  auto uid = [&](int t) __attribute__((always_inline)) -> int {
    return (int)(ulist[min(t, last)] & 0xffffu);
  };
  int j_n = 0;
  // prologue: block 0 published to buffer 0, block 1 staged, block 2 in
  // flight, offsets of block 3, id of block 4.  Past the end of the list the
  // last block is re-fetched, so the loop body has no branches around the
  // loads and the compiler's wait counters stay exact.
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

// One union block t (in buffer t % 2): publish staged block t+1 into the
// other buffer, load the rows of block t+4, refill the stage with block t+3,
// compute block t if this half's list holds it, then turn the rows into
// offsets.
#define PRISM_FWD_STEP(T_, BUF_, KS_, VS_)                                  \
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
    const uint32_t e = __builtin_amdgcn_readfirstlane(ulist[tt]);           \
    if (e & mflag)                                                          \
      compute_block(smem + (BUF_) * 2 * TL::kBytes,                         \
                    smem + (BUF_) * 2 * TL::kBytes + TL::kBytes);           \
    rows_to_offsets<D, 512>(offs_n, rows_n, tid);                           \
  }

  auto compute_block = [&](const unsigned char* sk, const unsigned char* sv)
                           __attribute__((always_inline)) {
    // S^T (32 kv x 32 q) = K_half Q_half^T
    f32x16 s = f32x16{};
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      s = mfma32(lds_row8<D>(sk, krow, 2 * ks + hf), qreg[ks], s);
    // online softmax in the log2 domain (scale > 0, so the max of the raw
    // scores is the max of the scaled ones).  The exponent reference m_run
    // only moves when a block's max exceeds it by more than 8: until then
    // the probabilities stay <= 2^8 (exact range in fp32 and bf16) and the
    // accumulator needs no rescale.
    float mx = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = xor32_max(mx) * scale_log2;
    const float m_new = mx > m_run + 8.f ? mx : m_run;
    const float alpha = exp2_fast(m_run - m_new);
    float rs = 0.f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = exp2_fast(fmaf(s[r], scale_log2, -m_new));
      rs += s[r];
    }
    rs = xor32_sum(rs);
    l_run = l_run * alpha + rs;
    m_run = m_new;
    if (__any(alpha != 1.f)) {      // the reference moved for some query
#pragma unroll
      for (int t2 = 0; t2 < DT; ++t2) oacc[t2] *= alpha;
    }
    const bf16x8 p0 = pack8(s, 0), p1 = pack8(s, 1);
    // O^T (d x 32 q) += V_half^T P^T
#pragma unroll
    for (int mt = 0; mt < DT; ++mt) {
      const int d0 = 32 * mt + 16 * (grp & 1);
      const int r0 = 32 * kh + 8 * (grp >> 1);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0, d0, j16), p0, oacc[mt]);
      oacc[mt] = mfma32(lds_tr8<D>(sv, r0 + 16, d0, j16), p1, oacc[mt]);
    }
  };

  // stage B holds block t+1 at even t, stage A at odd t
  int t = 0;
  for (; t + 1 < ucnt; t += 2) {
    PRISM_FWD_STEP(t, 0, kB, vB)
    PRISM_FWD_STEP(t + 1, 1, kA, vA)
  }
  if (t < ucnt) PRISM_FWD_STEP(t, 0, kB, vB)
#undef PRISM_FWD_STEP

  // merge the two KV halves of each query half: waves kh = 1 hand over
  // (m, l, O) through LDS (2 waves x 64 lanes x D/2 floats = 2 * kBytes per
  // query block)
  __syncthreads();
  float* xo = reinterpret_cast<float*>(smem + half * 2 * TL::kBytes);
  if (kh == 1) {
    if (hf == 0) {
      sm_m[half][qh][c] = m_run;
      sm_l[half][qh][c] = l_run;
    }
#pragma unroll
    for (int mt = 0; mt < DT; ++mt)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        xo[((qh * 64 + lane) * DT + mt) * 16 + r] = oacc[mt][r];
  }
  __syncthreads();
  if (kh == 0 && (half == 0 || has_second)) {
    const float m2 = sm_m[half][qh][c], l2 = sm_l[half][qh][c];
    float m = fmaxf(m_run, m2);
    // m = -inf: the query block's list is empty (no key at all)
    const bool none = m == -INFINITY;
    const float a1 = none ? 0.f : exp2_fast(m_run - m);
    const float a2 = none ? 0.f : exp2_fast(m2 - m);
    float l = l_run * a1 + l2 * a2;
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
          const float x = oacc[mt][r] * a1 +
                          xo[((qh * 64 + lane) * DT + mt) * 16 + r] * a2;
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
    const size_t words = (size_t)(Nb + 31) / 32;
    if (d == 128) {
      const size_t dyn = 4 * tiles::Tile<128>::kBytes + 4 * (size_t)Nb + 8 * words;
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<128>, g1, dim3(512), dyn, stream,
                   (const uint16_t*)q, (const uint16_t*)k, (const uint16_t*)v,
                   perm, counts, kv_idx, capacity, pairs, Hh, N, total, sl2,
                   drop_lse, drop_v, (uint16_t*)o, lse);
    } else {
      const size_t dyn = 4 * tiles::Tile<64>::kBytes + 4 * (size_t)Nb + 8 * words;
      PRISM_LAUNCH("attn_fwd_bf16", attn_fwd_bf16<64>, g1, dim3(512), dyn, stream,
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
