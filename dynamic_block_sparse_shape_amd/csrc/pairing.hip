// Pairing of blocks for the attention kernels.
//
// The forward, dQ and dK/dV kernels take two blocks per workgroup and walk
// the union of their block lists: a tile is gathered once per union entry,
// so the gathered bytes are proportional to |A u B| = |A| + |B| - |A n B|.
// Pairing blocks whose lists overlap most cuts them.  Blocks are matched
// within a window of kWin blocks on either side (permuted order: the
// window stays inside or next to the block's zone) by the size of the
// intersection of their lists:
//   1. word-major bitmaps of the lists (the column bitmap of the selection
//      is built by the backward already; the row bitmap is its bit
//      transpose);
//   2. weights |A n B| for every block and its 2 kWin candidates;
//   3. rounds of mutual best choices (largest weight, ties to the lower
//      index, weight > 0) until no pair forms, then the blocks left over in
//      ascending order two by two;
//   4. the pairs of a head are ranked by their summed list length, longest
//      first, and dealt round-robin to the 8 ranges of the table that the 8
//      XCDs work through (tiles::xcd_item): every XCD gets an equal share of
//      long and short work, the longest starts first, and workgroups
//      running side by side walk lists of about the same length.
// The result is deterministic and every block appears in exactly one pair;
// the attention results do not depend on it (each block still walks its own
// list in ascending order).
#include "prism_internal.h"

namespace prism {
namespace {

constexpr int kWin = 16;          // candidates i - kWin .. i + kWin, i excluded
constexpr int kCand = 2 * kWin;

// Candidate c of block i: i - kWin + c below i, i + 1 + (c - kWin) above it
// (ascending in the candidate's index).
__device__ __forceinline__ int cand_of(int i, int c) {
  return c < kWin ? i - kWin + c : i + 1 + (c - kWin);
}

// Column bitmaps of the selection, word-major: bits[(bh * words + w) * Nb + j]
// holds bit i - 32 w for every query block i in [32 w, 32 w + 32) that
// selected KV block j.  One workgroup per (bh, w) ORs its 32 lists (any
// order) into an LDS row of Nb words and writes the row out whole (no
// global atomics, no clearing pass).  A count is clamped to [0, Nb] and an
// id outside [0, Nb) is skipped, so a list that breaks the caller contract
// cannot write outside the LDS row; duplicate ids set the same bit.
__global__ __launch_bounds__(256) void bitmap_build(
    const int32_t* __restrict__ counts, const int32_t* __restrict__ kv_idx,
    int capacity, int Nb, int words, uint32_t* __restrict__ bits) {
  extern __shared__ uint32_t srow[];                      // [Nb]
  const long long bh = blockIdx.y;
  const int w = blockIdx.x;
  for (int j = threadIdx.x; j < Nb; j += 256) srow[j] = 0u;
  __syncthreads();
  const int wave = threadIdx.x / 64, lane = threadIdx.x % 64;
  for (int r = wave; r < 32; r += 4) {
    const int i = 32 * w + r;
    if (i >= Nb) break;
    const long long row = bh * Nb + i;
    const int cnt = min(max(counts[row], 0), Nb);
    const int32_t* lst = kv_idx + row * (long long)capacity;
    for (int t = lane; t < cnt; t += 64) {
      const int j = lst[t];
      if ((unsigned)j < (unsigned)Nb) atomicOr(&srow[j], 1u << r);
    }
  }
  __syncthreads();
  uint32_t* out = bits + (bh * words + w) * (long long)Nb;
  for (int j = threadIdx.x; j < Nb; j += 256) out[j] = srow[j];
}

// Bit transpose of word-major bitmaps: in[(bh * words + w) * Nb + j] holds
// bit i - 32 w for rows i in [32 w, 32 w + 32) at column j; out[(bh * words
// + v) * Nb + i] holds bit j - 32 v for columns j in [32 v, 32 v + 32) at
// row i.  One wave per (bh, w, two consecutive v): each half-wave loads 32
// words of one 32 x 32 bit tile and 32 ballots hand out its columns.
__global__ __launch_bounds__(256) void bitmap_transpose(
    const uint32_t* __restrict__ in, int Nb, int words, long long heads,
    uint32_t* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const long long wid = (long long)blockIdx.x * 4 + (threadIdx.x >> 6);
  const int vpairs = (words + 1) / 2;
  const long long per_head = (long long)words * vpairs;
  if (wid >= heads * per_head) return;        // whole wave leaves together
  const long long bh = wid / per_head;
  const int w = (int)(wid % per_head) / vpairs;
  const int v = 2 * ((int)(wid % per_head) % vpairs) + (lane >> 5);
  const int l = lane & 31;
  const int j = 32 * v + l;
  const uint32_t x = (v < words && j < Nb)
                         ? in[(bh * words + w) * (long long)Nb + j] : 0u;
  uint32_t mine = 0u;
#pragma unroll
  for (int b = 0; b < 32; ++b) {
    const unsigned long long m = __ballot((x >> b) & 1u);
    const uint32_t half = (uint32_t)(lane < 32 ? m : m >> 32);
    if (l == b) mine = half;
  }
  const int i = 32 * w + l;
  if (v < words && i < Nb) out[(bh * words + v) * (long long)Nb + i] = mine;
}

// weight[(bh * Nb + i) * kCand + c] = |list(i) n list(cand_of(i, c))|, or -1
// when the candidate is outside [0, Nb); size[bh * Nb + i] = |list(i)|.
// Word-major bitmap input; a workgroup takes 256 consecutive blocks of one
// head and stages each bitmap word of them and of the kWin blocks on either
// side in LDS.
__global__ __launch_bounds__(256) void pair_weights(
    const uint32_t* __restrict__ bits, int Nb, int words,
    int32_t* __restrict__ weight, int32_t* __restrict__ size) {
  __shared__ uint32_t tile[256 + 2 * kWin];
  const long long bh = blockIdx.y;
  const int i0 = blockIdx.x * 256;
  const int t = threadIdx.x;
  const int i = i0 + t;
  int acc[kCand], own = 0;
#pragma unroll
  for (int c = 0; c < kCand; ++c) acc[c] = 0;
  for (int w = 0; w < words; ++w) {
    const uint32_t* row = bits + (bh * words + w) * (long long)Nb;
    for (int e = t; e < 256 + 2 * kWin; e += 256) {
      const int k = i0 - kWin + e;
      tile[e] = (k >= 0 && k < Nb) ? row[k] : 0u;
    }
    __syncthreads();
    const uint32_t a = tile[t + kWin];
    own += __popc(a);
#pragma unroll
    for (int c = 0; c < kCand; ++c)
      acc[c] += __popc(a & tile[t + (c < kWin ? c : c + 1)]);
    __syncthreads();
  }
  if (i >= Nb) return;
  size[bh * Nb + i] = own;
  int32_t* out = weight + (bh * Nb + i) * (long long)kCand;
#pragma unroll
  for (int c = 0; c < kCand; ++c) {
    const int k = cand_of(i, c);
    out[c] = (k >= 0 && k < Nb) ? acc[c] : -1;
  }
}

// Inclusive scan of one int per thread over a 1024-thread workgroup.
__device__ __forceinline__ int block_scan(int x, int* s_part) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int incl = x;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  __syncthreads();
  if (lane == 63) s_part[wave] = incl;
  __syncthreads();
  int before = 0;
  for (int w = 0; w < wave; ++w) before += s_part[w];
  return incl + before;
}

constexpr int kMatchThreads = 1024;
constexpr int kMaxRounds = 64;

// Sort keys padded to a power of two (P <= 4096).
__host__ __device__ inline int pow2_at_least(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}
// LDS bytes of pair_match: 3 int16 arrays of Nb, then P pairs and the
// padded sort keys.
__host__ __device__ inline size_t match_lds_bytes(int Nb) {
  const int P = (Nb + 1) / 2;
  return ((size_t)3 * Nb * sizeof(int16_t) + 7) / 8 * 8 +
         (size_t)P * sizeof(int2) + (size_t)pow2_at_least(P) * sizeof(uint32_t);
}

// One workgroup per head: mutual-best rounds, then the leftovers in
// ascending order; then the pairs ranked by summed list length, longest
// first (ties by first block), and dealt to the XCD ranges like cards:
// rank r to range r mod 8, position r / 8, skipping ranges that are
// already full (the last ranges are shorter when P is not a multiple of
// their length).  pairs[bh * P + p] = (a, b), a < b, or b = -1 (a single
// block when Nb is odd); P = (Nb + 1) / 2.  Nb <= 8192.
__global__ __launch_bounds__(kMatchThreads) void pair_match(
    const int32_t* __restrict__ weight, const int32_t* __restrict__ size,
    int Nb, int2* __restrict__ pairs) {
  extern __shared__ __align__(8) unsigned char smb[];
  int16_t* partner = reinterpret_cast<int16_t*>(smb);   // matched partner or -1
  int16_t* best = partner + Nb;                         // this round's choice or -1
  int16_t* urank = partner + 2 * Nb;                    // leftover rank -> block
  int2* sp = reinterpret_cast<int2*>(smb + ((size_t)3 * Nb * sizeof(int16_t) + 7) / 8 * 8);
  uint32_t* skey = reinterpret_cast<uint32_t*>(sp + (Nb + 1) / 2);
  __shared__ int s_changed, s_part[kMatchThreads / 64];
  const long long bh = blockIdx.x;
  const int32_t* wt = weight + bh * Nb * (long long)kCand;
  const int tid = threadIdx.x;
  for (int i = tid; i < Nb; i += kMatchThreads) partner[i] = -1;
  __syncthreads();
  for (int round = 0; round < kMaxRounds; ++round) {
    for (int i = tid; i < Nb; i += kMatchThreads) {
      int bk = -1, bw = 0;
      if (partner[i] < 0) {
        // the node's kCand weights: one 128-byte row, loaded as 16-byte vectors
        int wv[kCand];
        const int4* w4 = reinterpret_cast<const int4*>(wt + (long long)i * kCand);
#pragma unroll
        for (int q = 0; q < kCand / 4; ++q) {
          const int4 x = w4[q];
          wv[4 * q] = x.x;
          wv[4 * q + 1] = x.y;
          wv[4 * q + 2] = x.z;
          wv[4 * q + 3] = x.w;
        }
#pragma unroll
        for (int c = 0; c < kCand; ++c) {
          const int k = cand_of(i, c);
          if (wv[c] > bw && partner[k] < 0) {   // weight > 0: 0 <= k < Nb
            bw = wv[c];
            bk = k;
          }
        }
      }
      best[i] = (int16_t)bk;
    }
    if (tid == 0) s_changed = 0;
    __syncthreads();
    for (int i = tid; i < Nb; i += kMatchThreads) {
      const int k = best[i];
      if (k >= 0 && best[k] == i) {
        partner[i] = (int16_t)k;
        s_changed = 1;
      }
    }
    __syncthreads();
    const int changed = s_changed;
    __syncthreads();
    if (!changed) break;
  }

  // each thread owns a run of consecutive blocks [r0, r1)
  const int per = (Nb + kMatchThreads - 1) / kMatchThreads;
  const int r0 = min(Nb, tid * per), r1 = min(Nb, r0 + per);
  int nu = 0;
  for (int i = r0; i < r1; ++i) nu += partner[i] < 0;
  const int u_incl = block_scan(nu, s_part);
  int rank = u_incl - nu;
  for (int i = r0; i < r1; ++i)
    if (partner[i] < 0) urank[rank++] = (int16_t)i;
  if (tid == kMatchThreads - 1) s_changed = u_incl;   // number of leftovers
  __syncthreads();
  const int nleft = s_changed;
  // first members: matched blocks below their partner, leftovers of even
  // rank
  int nf = 0;
  rank = u_incl - nu;
  for (int i = r0; i < r1; ++i) {
    const int pk = partner[i];
    if (pk >= 0) nf += pk > i;
    else nf += (rank++ & 1) == 0;
  }
  const int f_incl = block_scan(nf, s_part);
  int p = f_incl - nf;
  rank = u_incl - nu;
  const int P = (Nb + 1) / 2, P2 = pow2_at_least(P);
  const int32_t* sz = size + bh * Nb;
  // sort key: (32767 - summed length) << 16 | pair index -- ascending order
  // is longest first, ties by pair index; padding sorts last
  auto key_of = [](int len, int idx) -> uint32_t {
    return ((uint32_t)(32767 - min(len, 32767)) << 16) | (uint32_t)idx;
  };
  // (the first members number exactly P; the bound only guards the table)
  for (int i = r0; i < r1; ++i) {
    const int pk = partner[i];
    if (pk >= 0) {
      if (pk > i && p < P) {
        skey[p] = key_of(sz[i] + sz[pk], p);
        sp[p++] = int2{i, pk};
      }
    } else {
      if ((rank & 1) == 0 && p < P) {
        const int nx = rank + 1 < nleft ? urank[rank + 1] : -1;
        skey[p] = key_of(sz[i] + (nx >= 0 ? sz[nx] : 0), p);
        sp[p++] = int2{i, nx};
      }
      ++rank;
    }
  }
  for (int e = P + tid; e < P2; e += kMatchThreads) skey[e] = 0xffffffffu;
  __syncthreads();
  // bitonic sort of the P2 keys
  for (int k = 2; k <= P2; k <<= 1) {
    for (int j = k >> 1; j > 0; j >>= 1) {
      for (int e = tid; e < P2; e += kMatchThreads) {
        const int f = e ^ j;
        if (f > e) {
          const uint32_t a = skey[e], b = skey[f];
          const bool up = (e & k) == 0;
          if ((a > b) == up) {
            skey[e] = b;
            skey[f] = a;
          }
        }
      }
      __syncthreads();
    }
  }
  // global rank, dealt round-robin to the XCD ranges (same split as
  // tiles::xcd_item: range x = [x c8, min(P, (x + 1) c8)))
  const int c8 = (P + 7) / 8;
  const int full = P / c8, rem = P % c8;
  int2* out = pairs + bh * P;
  for (int r = tid; r < P; r += kMatchThreads) {
    const int e = (int)(skey[r] & 0xffffu);
    int x, sidx;
    if (r < rem * (full + 1)) {
      sidx = r / (full + 1);
      x = r % (full + 1);
    } else {
      const int r2 = r - rem * (full + 1);
      sidx = rem + r2 / full;
      x = r2 % full;
    }
    out[x * c8 + sidx] = sp[e];
  }
}

}  // namespace

size_t bitmap_bytes(int B, int Hh, int Nb) {
  return align256((size_t)B * Hh * ((Nb + 31) / 32) * Nb * sizeof(uint32_t));
}

size_t block_pairs_ws_bytes(int B, int Hh, int Nb) {
  return align256((size_t)B * Hh * Nb * kCand * sizeof(int32_t)) +
         align256((size_t)B * Hh * Nb * sizeof(int32_t));
}

size_t block_pairs_bytes(int B, int Hh, int Nb) {
  return align256((size_t)B * Hh * ((Nb + 1) / 2) * sizeof(int2));
}

prism_status launch_block_pairs(const uint32_t* bits, int B, int Hh, int Nb,
                                void* ws, int2* pairs, hipStream_t stream) {
  const int words = (Nb + 31) / 32;
  const long long heads = (long long)B * Hh;
  int32_t* weight = static_cast<int32_t*>(ws);
  int32_t* size = reinterpret_cast<int32_t*>(
      static_cast<char*>(ws) + align256((size_t)heads * Nb * kCand * sizeof(int32_t)));
  PRISM_LAUNCH("pair_weights", pair_weights,
               dim3((unsigned)((Nb + 255) / 256), (unsigned)heads), dim3(256), 0,
               stream, bits, Nb, words, weight, size);
  prism_status st = check_launch("pair_weights");
  if (st != PRISM_OK) return st;
  PRISM_LAUNCH("pair_match", pair_match, dim3((unsigned)heads),
               dim3(kMatchThreads), match_lds_bytes(Nb), stream, weight, size,
               Nb, pairs);
  return check_launch("pair_match");
}

prism_status launch_column_bitmap(const int32_t* counts, const int32_t* kv_idx,
                                  int capacity, int B, int Hh, int Nb,
                                  uint32_t* bits, hipStream_t stream) {
  const int words = (Nb + 31) / 32;
  PRISM_LAUNCH("bitmap_build", bitmap_build,
               dim3((unsigned)words, (unsigned)(B * Hh)), dim3(256),
               (size_t)Nb * sizeof(uint32_t), stream, counts, kv_idx, capacity,
               Nb, words, bits);
  return check_launch("bitmap_build");
}

prism_status launch_bitmap_transpose(const uint32_t* in, int B, int Hh, int Nb,
                                     uint32_t* out, hipStream_t stream) {
  const int words = (Nb + 31) / 32;
  const long long heads = (long long)B * Hh;
  const long long waves = heads * words * ((words + 1) / 2);
  PRISM_LAUNCH("bitmap_transpose", bitmap_transpose,
               dim3((unsigned)((waves + 3) / 4)), dim3(256), 0, stream, in, Nb,
               words, heads, out);
  return check_launch("bitmap_transpose");
}

}  // namespace prism
