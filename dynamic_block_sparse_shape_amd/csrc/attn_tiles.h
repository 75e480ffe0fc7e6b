// Building blocks of the gfx950 block-sparse attention kernels.
//
// * 64-row bf16 tiles (one 64-token block of K, V, Q or dO) live row-major in
//   LDS with an XOR swizzle of their 16-byte pieces, so that both access
//   patterns below are free of bank conflicts:
//     - row-operand reads: ds_read_b128 of one 16-byte piece from each of
//       16 rows per 16 lanes;
//     - transposed-operand reads: ds_read_b64_tr_b16 (gfx950), where a
//       half-wave reads 8 bytes per lane from 4 consecutive rows x 32
//       columns and the hardware hands every lane 4 consecutive rows of one
//       column.
//   (The LDS bank-conflict counter reads zero for both patterns.)
// * A workgroup (256 or 512 threads) gathers a tile's rows through the
//   token permutation with 16-byte buffer loads held in registers one or two
//   blocks ahead, then publishes it with one ds_write_b128 per piece.
// * Blocks are processed in pairs over the union of their block lists
//   (pair_union); the pairs are neighbours whose lists overlap most
//   (pairing.hip).  Work items are ordered head by head across the 8 XCDs
//   (xcd_item).
// * MFMA v_mfma_f32_32x32x16_bf16 operand layouts (lane l, c = l % 32,
//   h = l / 32): A[i][k] holds i = c, k = 8h .. 8h+7; B[k][j] holds j = c,
//   k = 8h .. 8h+7; C[i][j] holds j = c and rows i = 8a + 4h + b in register
//   4a + b (a, b in 0..3).
#pragma once

#include "prism_internal.h"

namespace prism {
namespace tiles {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) bf16x4 lds_bf16x4;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ bf16x8 as_bf16x8(u32x4 v) {
  return __builtin_bit_cast(bf16x8, v);
}

__device__ __forceinline__ f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Row of the 32-row operand that feeds M-row i of a 32x32 tile.  With this
// order the C-layout registers 8s..8s+7 of a lane hold rows 16s + 8h + e
// (e = 0..7), i.e. exactly the B operand (k = 8h + e) of the next product
// over the same 32 rows, k-step s.
__device__ __forceinline__ int slot_of(int i) {
  const int a = i >> 3, hh = (i >> 2) & 1, b = i & 3;
  return 16 * (a >> 1) + 8 * hh + 4 * (a & 1) + b;
}

template <int D>
struct Tile {
  static constexpr int kRowBytes = D * 2;
  static constexpr int kPieces = kRowBytes / 16;          // 16-byte pieces per row
  static constexpr int kBytes = 64 * kRowBytes;

  // 16-byte slot of piece 0 of row r (the XOR key).  The LDS serves 256
  // bytes (64 banks) per pass.  Row-operand reads fetch one piece from each
  // of 16 consecutive rows: the key is a bijection on r mod 16 (D = 128;
  // for D = 64, two rows share a pass and the key is a bijection on r / 2
  // within each parity).  Transposed reads fetch 4 pieces (one aligned
  // group of 4 slots) from each of 4 consecutive rows: bits 2-3 of the slot
  // must differ between those rows, so the row's low bits go there.  The
  // key depends on r mod 16 only.
  __device__ static __forceinline__ int swz(int r) {
    if constexpr (kPieces == 16) return ((r & 3) << 2) | ((r >> 2) & 3);
    else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
  }
  // byte offset of (row r, 16-byte piece p)
  __device__ static __forceinline__ int off(int r, int p) {
    return r * kRowBytes + ((p ^ swz(r)) << 4);
  }
  // byte offset of the 8 bytes holding columns d .. d+3 of row r (d % 4 == 0)
  __device__ static __forceinline__ int off8(int r, int d) {
    return off(r, d >> 3) + ((d & 4) << 1);
  }
};

// How NT threads share the 16-byte pieces of one tile: thread tid owns
// piece tid % kPieces of rows (tid + NT * t) / kPieces, t < kPerThread.
template <int D, int NT = 256>
struct Share {
  static constexpr int kPerThread = 64 * Tile<D>::kPieces / NT;
  static_assert(kPerThread >= 1, "too many threads for one tile");
  __device__ static __forceinline__ int row_of(int tid, int t) {
    return (tid + NT * t) / Tile<D>::kPieces;
  }
  __device__ static __forceinline__ int piece_of(int tid) {
    return tid % Tile<D>::kPieces;
  }
};

// 16-byte piece of a row-operand fragment: ds_read_b128
template <int D>
__device__ __forceinline__ bf16x8 lds_row8(const unsigned char* tile, int r,
                                          int p) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(tile + Tile<D>::off(r, p)));
}

// Transposed fragment for an A or B operand over 8 consecutive tile rows:
// lane (quarter-wave lane j = l % 16) receives rows r0 .. r0+7 of column
// d0 + j.  Two ds_read_b64_tr_b16, each covering 4 rows.
template <int D>
__device__ __forceinline__ bf16x8 lds_tr8(const unsigned char* tile, int r0,
                                         int d0, int j) {
  const int r = r0 + (j >> 2);
  const int d = d0 + 4 * (j & 3);
  // generic -> LDS address space (the tile is a __shared__ array)
  lds_bf16x4* p0 = (lds_bf16x4*)(tile + Tile<D>::off8(r, d));
  lds_bf16x4* p1 = (lds_bf16x4*)(tile + Tile<D>::off8(r + 4, d));
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// Cheap per-lane addressing of the swizzled tiles.  With the XOR swizzle,
// the address of row r, piece 2ks + hf is  y + ((ks << 5) ^ x)  for two lane
// constants, and the transposed 4x4 reads of lds_tr8 at rows
// rbase + 8 (grp / 2) + 16 a + (j / 4) (+4) and columns 32 mt + ... are
// y_b + 16 a rows + ((mt << 6) ^ m_b)  (the swizzle of those rows does not
// depend on a or rbase).  Kernels keep these 2 + 4 constants live instead of
// one address register per fragment, and make them opaque once per loop
// iteration so the compiler recomputes (one VALU op) rather than hoists.
struct RowAddr {
  uint32_t y, x;
};
template <int D>
__device__ __forceinline__ RowAddr row_addr(int r, int hf) {
  const int sw = Tile<D>::swz(r);
  return {(uint32_t)(r * Tile<D>::kRowBytes + ((hf ^ (sw & 1)) << 4)),
          (uint32_t)((sw & ~1) << 4)};
}
template <int D>
__device__ __forceinline__ bf16x8 lds_row_at(const unsigned char* tile,
                                            RowAddr a, int ks) {
  return as_bf16x8(*reinterpret_cast<const u32x4*>(
      tile + (a.y + (((uint32_t)ks << 5) ^ a.x))));
}

struct TrAddr {
  uint32_t y0, y1, m0, m1;
};
// rbase: first row of the 32-row half (multiple of 32); lane = lane id
template <int D>
__device__ __forceinline__ TrAddr tr_addr(int rbase, int lane) {
  const int j = lane & 15, grp = lane >> 4;
  const int x = 2 * (grp & 1) + ((j & 3) >> 1);
  TrAddr t;
  {
    const int r = rbase + 8 * (grp >> 1) + (j >> 2);
    const int sw = Tile<D>::swz(r);
    t.y0 = (uint32_t)(r * Tile<D>::kRowBytes + (((x ^ sw) & 3) << 4) + 8 * (j & 1));
    t.m0 = (uint32_t)((sw >> 2) << 6);
  }
  {
    const int r = rbase + 8 * (grp >> 1) + (j >> 2) + 4;
    const int sw = Tile<D>::swz(r);
    t.y1 = (uint32_t)(r * Tile<D>::kRowBytes + (((x ^ sw) & 3) << 4) + 8 * (j & 1));
    t.m1 = (uint32_t)((sw >> 2) << 6);
  }
  return t;
}
// Same fragment as lds_tr8(tile, rbase + 8 (grp / 2) + 16 a, 32 mt + 16 (grp & 1), j)
template <int D>
__device__ __forceinline__ bf16x8 lds_tr_at(const unsigned char* tile, TrAddr t,
                                           int a, int mt) {
  const uint32_t ro = (uint32_t)(16 * a * Tile<D>::kRowBytes);
  lds_bf16x4* p0 = (lds_bf16x4*)(tile + (t.y0 + ro + (((uint32_t)mt << 6) ^ t.m0)));
  lds_bf16x4* p1 = (lds_bf16x4*)(tile + (t.y1 + ro + (((uint32_t)mt << 6) ^ t.m1)));
  const bf16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p0);
  const bf16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16(p1);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ void opaque(RowAddr& a) {
  asm volatile("" : "+v"(a.y), "+v"(a.x));
}
__device__ __forceinline__ void opaque(TrAddr& t) {
  asm volatile("" : "+v"(t.y0), "+v"(t.y1), "+v"(t.m0), "+v"(t.m1));
}

// Global -> register staging of one 64-row tile.  Rows are gathered with
// buffer loads: one resource per (tensor, head) and 32-bit byte offsets that
// the K and V (or Q and dO) tiles of a block share.
template <int D, int NT = 256>
struct Stage {
  u32x4 v[Share<D, NT>::kPerThread];   // clang vectors: promotable to registers
};

// Buffer resource over one head's [N, D] bf16 rows (loads past the end
// return zeros instead of faulting).
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t head_rsrc(
    const uint16_t* base, long long head_row0, int N) {
  return __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(base + head_row0 * D), (short)0, N * D * 2,
      0x00020000);
}

// Token rows of this thread's pieces of block j (plain loads of the
// permutation).  They are issued before a block's tile loads and turned into
// offsets only after them: wait counters retire loads in issue order, so a
// row load issued after a tile load would make its first use wait for that
// tile load too.
template <int D, int NT = 256>
__device__ __forceinline__ void stage_rows(int* rows,
                                           const int32_t* __restrict__ pb,
                                           int j, int tid) {
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t)
    rows[t] = pb[64 * j + Share<D, NT>::row_of(tid, t)];
}

// Byte offsets (within the head) of this thread's pieces, from its rows.
template <int D, int NT = 256>
__device__ __forceinline__ void rows_to_offsets(uint32_t* offs, const int* rows,
                                                int tid) {
  const uint32_t p16 = (uint32_t)Share<D, NT>::piece_of(tid) * 16u;
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t)
    offs[t] = (uint32_t)rows[t] * (uint32_t)(D * 2) + p16;
}

template <int D, int NT = 256>
__device__ __forceinline__ void stage_offsets(uint32_t* offs,
                                              const int32_t* __restrict__ pb,
                                              int j, int tid) {
  int rows[Share<D, NT>::kPerThread];
  stage_rows<D, NT>(rows, pb, j, tid);
  rows_to_offsets<D, NT>(offs, rows, tid);
}

// Keeps the compiler's scheduler from moving instructions across this point
// (used to pin the issue order of loads).
__device__ __forceinline__ void pin_order() { __builtin_amdgcn_sched_barrier(0); }

template <int D, int NT = 256>
__device__ __forceinline__ void stage_load(Stage<D, NT>& s, __amdgpu_buffer_rsrc_t r,
                                           const uint32_t* offs) {
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t)
    s.v[t] = __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, offs[t], 0, 0));
}

template <int D, int NT = 256>
__device__ __forceinline__ void stage_store(const Stage<D, NT>& s,
                                            unsigned char* tile, int tid) {
  const int p = Share<D, NT>::piece_of(tid);
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t)
    *reinterpret_cast<u32x4*>(tile + Tile<D>::off(Share<D, NT>::row_of(tid, t), p)) =
        s.v[t];
}

// Global -> LDS copy of one 64-row tile that bypasses registers
// (buffer_load_dwordx4 ... lds, gfx950).  One such load fills 1 KiB of LDS
// from a wave, lane l at byte 16 l, so each lane fetches the piece that the
// tile's swizzle places there: thread tid covers rows Share::row_of(tid, t)
// (the rows stage_rows reads) at LDS piece tid % kPieces.  dma_offsets turns
// those rows into the byte offsets of the pieces to fetch; stage_dma issues
// the loads.  They complete asynchronously and count in vmcnt: wait for
// them (vmcnt(0)) before the barrier that publishes the tile, and before
// the tile area is reused.
template <int D, int NT = 256>
__device__ __forceinline__ void dma_offsets(uint32_t* offs, const int* rows,
                                            int tid) {
  const int pos = Share<D, NT>::piece_of(tid);
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t) {
    const int piece = pos ^ Tile<D>::swz(Share<D, NT>::row_of(tid, t));
    offs[t] = (uint32_t)rows[t] * (uint32_t)(D * 2) + 16u * (uint32_t)piece;
  }
}

template <int D, int NT = 256>
__device__ __forceinline__ void stage_dma(unsigned char* tile,
                                          __amdgpu_buffer_rsrc_t r,
                                          const uint32_t* offs, int tid) {
  const int wave0 = tid & ~63;
#pragma unroll
  for (int t = 0; t < Share<D, NT>::kPerThread; ++t) {
    unsigned char* dst = tile + Share<D, NT>::row_of(wave0, t) * Tile<D>::kRowBytes;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)dst, 16, offs[t], 0, 0, 0);
  }
}

// Wait until every global load of this wave has landed (registers or LDS).
__device__ __forceinline__ void wait_loads() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

// Two floats -> packed bf16 pair (v_cvt_pk_bf16_f32, round to nearest even).
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
}

// Maximum that propagates NaN (IEEE 754-2019 maximum, v_maximum3_f32 on
// gfx950).  fmaxf drops a NaN operand, which in IEEE mode makes the compiler
// quiet every input first (one extra v_max_f32 x, x, x per score); for the
// finite scores of a row both give the same maximum, and a NaN score makes
// the row NaN either way (its exponential is NaN).
__device__ __forceinline__ float fmax_prop(float a, float b) {
  return __builtin_elementwise_maximum(a, b);
}

// Combine a value with the one held by lane l ^ 32: v_permlane32_swap
// (gfx950) hands every lane its partner's value without touching LDS.
__device__ __forceinline__ float xor32_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return fmax_prop(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float xor32_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x),
                                                  __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// 2^x with the hardware v_exp_f32 (inputs here are <= 0 or -inf).
__device__ __forceinline__ float exp2_fast(float x) {
  return __builtin_amdgcn_exp2f(x);
}

// Pack C-layout registers 8s .. 8s+7 into a bf16 B operand.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int s) {
  u32x4 u;
  u.x = cvt2(c[8 * s + 0], c[8 * s + 1]);
  u.y = cvt2(c[8 * s + 2], c[8 * s + 3]);
  u.z = cvt2(c[8 * s + 4], c[8 * s + 5]);
  u.w = cvt2(c[8 * s + 6], c[8 * s + 7]);
  return as_bf16x8(u);
}

// Ascending union of two blocks' KV lists, built by a workgroup of NT
// threads (NT = 256 or 512; thread w owns bitmap word w of the union).
// Each 16-bit entry is id | (in list 0) << 13 | (in list 1) << 14 (ids
// fit 13 bits: Nb <= 8192).  bits holds 2 * ceil(Nb / 32) words and ulist
// Nb entries (LDS); s_cnt 8 ints.  Counts are clamped to [0, Nb], ids outside [0, Nb) are
// skipped and duplicates merge, so any list gives a valid union.  Returns
// the union size; when it is 0, ulist[0] holds block 0 with no membership
// bits (a safe id for the gather prologue).  Ends with a barrier.
template <int NT = 512>
__device__ __forceinline__ int pair_union(const int32_t* __restrict__ lst0,
                                          int cnt0,
                                          const int32_t* __restrict__ lst1,
                                          int cnt1, int Nb, uint32_t* bits,
                                          uint16_t* ulist, int* s_cnt, int tid) {
  const int words = (Nb + 31) / 32;
  const int wave = tid >> 6, lane = tid & 63;
  for (int w = tid; w < 2 * words; w += NT) bits[w] = 0u;
  __syncthreads();
  cnt0 = min(max(cnt0, 0), Nb);
  cnt1 = min(max(cnt1, 0), Nb);
  for (int t = tid; t < cnt0; t += NT) {
    const int j = lst0[t];
    if ((unsigned)j < (unsigned)Nb) atomicOr(&bits[j >> 5], 1u << (j & 31));
  }
  for (int t = tid; t < cnt1; t += NT) {
    const int j = lst1[t];
    if ((unsigned)j < (unsigned)Nb)
      atomicOr(&bits[words + (j >> 5)], 1u << (j & 31));
  }
  __syncthreads();
  // thread w owns bitmap word w (words <= 256 <= NT)
  const uint32_t wa = tid < words ? bits[tid] : 0u;
  const uint32_t wb = tid < words ? bits[words + tid] : 0u;
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
  int pos = incl - n, ucnt = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) {
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
  if (ucnt == 0 && tid == 0) ulist[0] = 0;
  __syncthreads();
  return ucnt;
}

// Work item of this workgroup.  Workgroups are dealt round-robin to the 8
// XCDs, so workgroup L runs on XCD L % 8.  Every head's Nb items are split
// into 8 contiguous ranges of the item table, one per XCD, walked in order,
// and heads are visited in order: all XCDs work on the same head at the same
// time (one head's K / V, ~150 MB at the 2K grid, is the whole working set).
// The attention kernels' pair tables fill the ranges so that each XCD gets
// an equal, longest-first share (pairing.hip).  Returns false for padding
// items.
__device__ __forceinline__ bool xcd_item(int Nb, long long heads, long long& bh,
                                         int& i) {
  const long long L = blockIdx.x;
  const int c8 = (Nb + 7) / 8;
  const long long s = L >> 3;
  bh = s / c8;
  i = (int)(L & 7) * c8 + (int)(s % c8);
  return bh < heads && i < Nb;
}
inline unsigned xcd_grid(int Nb, long long heads) {
  return (unsigned)(8LL * ((Nb + 7) / 8) * heads);
}

}  // namespace tiles
}  // namespace prism
