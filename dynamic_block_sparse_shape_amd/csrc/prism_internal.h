// Internal helpers shared by the gfx950 kernels and the C ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/prism.h"

namespace prism {

// ------------------------------------------------------------------ errors
prism_status fail(prism_status st, const char* fmt, ...);
void clear_error();
// Wraps the launch status of the most recent kernel.
prism_status check_launch(const char* what);

// Optional per-kernel timing (prism_profile_* in include/prism.h): when
// enabled, every launch is bracketed by two hipEvents on its stream.
struct ProfScope {
  int slot;
  hipStream_t stream;
  ProfScope(hipStream_t s, const char* name);
  ~ProfScope();
};

#define PRISM_LAUNCH(NAME, KERNEL, GRID, BLOCK, SHM, STREAM, ...)          \
  do {                                                                    \
    prism::ProfScope prism_prof_scope_((STREAM), (NAME));                 \
    hipLaunchKernelGGL(KERNEL, GRID, BLOCK, SHM, STREAM, __VA_ARGS__);    \
  } while (0)

#define PRISM_CHECK(cond, st, ...)            \
  do {                                        \
    if (!(cond)) return prism::fail(st, __VA_ARGS__); \
  } while (0)

// ------------------------------------------------------------ shape table
struct Shape { int t, h, w; };
constexpr int kNumShapes = 13;
// (t, h, w) per id; see prism_shape_table() in include/prism.h.
__host__ __device__ inline Shape shape_of(int id) {
  constexpr int tbl[kNumShapes][3] = {
      {4, 4, 4}, {2, 4, 8}, {2, 8, 4}, {4, 2, 8}, {4, 8, 2}, {8, 2, 4},
      {8, 4, 2}, {1, 8, 8}, {8, 1, 8}, {8, 8, 1}, {2, 2, 16}, {2, 16, 2},
      {16, 2, 2}};
  return Shape{tbl[id][0], tbl[id][1], tbl[id][2]};
}
__host__ __device__ inline bool shape_fits(int id, int Lt, int Lh, int Lw) {
  Shape s = shape_of(id);
  return Lt % s.t == 0 && Lh % s.h == 0 && Lw % s.w == 0;
}

// ------------------------------------------------------------- bf16 bits
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
  return __uint_as_float(static_cast<uint32_t>(h) << 16);
}
// round to nearest even; NaN stays NaN
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return 0x7fc0;
  u += 0x7fffu + ((u >> 16) & 1u);
  return static_cast<uint16_t>(u >> 16);
}

inline int ceil_div(int a, int b) { return (a + b - 1) / b; }
inline size_t align256(size_t n) { return (n + 255) / 256 * 256; }

// ------------------------------------------------------- stage launchers
struct ZoneGeom {
  int T, H, W, zt, zh, zw, nzt, nzh, nzw, nZ;
};
prism_status launch_zone_shapes(const void* feat, const void* a2v, int dtype,
                                int B, const ZoneGeom& g, int C, double lam,
                                int fixed_shape, int32_t* zone_shape,
                                int32_t* perm, int32_t* inv_perm,
                                double* zone_stats, void* ws,
                                hipStream_t stream);
size_t zone_shapes_ws_bytes(int B, const ZoneGeom& g, int C);

prism_status launch_pool_proxy(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               double* proxy, hipStream_t stream);

prism_status launch_pool_means(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               hipStream_t stream);

// Fused stages 2b-3 (route.hip): proxy scores and selection without the
// proxy matrix, from the pooled means.
size_t route_fused_ws_bytes(int B, int Hh, int Nb, int d);
prism_status launch_route_fused(const double* q_mean, const double* k_mean,
                                int B, int Hh, int Nb, int d, int top_k,
                                double tau, int32_t* counts, int32_t* kv_idx,
                                int capacity, void* ws, hipStream_t stream);

prism_status launch_select(const double* proxy, int B, int Hh, int Nb,
                           int top_k, double tau, int32_t* counts,
                           int32_t* kv_idx, int capacity, hipStream_t stream);

// Block pairing for the attention kernels (pairing.hip).  Bitmaps are
// word-major: bits[(bh * words + w) * Nb + x] holds 32 bits of block x's
// list (words = ceil(Nb / 32)).  Pairs: (Nb + 1) / 2 int2 per (b, h).
size_t bitmap_bytes(int B, int Hh, int Nb);
size_t block_pairs_ws_bytes(int B, int Hh, int Nb);
size_t block_pairs_bytes(int B, int Hh, int Nb);
prism_status launch_column_bitmap(const int32_t* counts, const int32_t* kv_idx,
                                  int capacity, int B, int Hh, int Nb,
                                  uint32_t* bits, hipStream_t stream);
prism_status launch_bitmap_transpose(const uint32_t* in, int B, int Hh, int Nb,
                                     uint32_t* out, hipStream_t stream);
prism_status launch_block_pairs(const uint32_t* bits, int B, int Hh, int Nb,
                                void* ws, int2* pairs, hipStream_t stream);

size_t attn_fwd_ws_bytes(int B, int Hh, int N, int d);
prism_status launch_attn_fwd(const void* q, const void* k, const void* v,
                             int dtype, const int32_t* perm,
                             const int32_t* counts, const int32_t* kv_idx,
                             int capacity, int B, int Hh, int N, int d,
                             float scale, const float* drop_lse,
                             const float* drop_v, void* o, float* lse,
                             void* ws, hipStream_t stream);

// Pooled stand-in for the unselected blocks (dropped.hip): per query block
// the log weight drop_lse [B,Hh,Nb] and mean value drop_v [B,Hh,Nb,d] (fp32).
size_t dropped_terms_ws_bytes(int B, int Hh, int N, int d);
prism_status launch_dropped_terms(const double* proxy, const double* q_mean,
                                  const double* k_mean, const void* v,
                                  int dtype, const int32_t* perm,
                                  const int32_t* counts, const int32_t* kv_idx,
                                  int capacity, int B, int Hh, int N, int d,
                                  float* drop_lse, float* drop_v, void* ws,
                                  hipStream_t stream);

// The a2v bridge residual (bridge.hip): projections on bf16 MFMA GEMMs,
// cross-attention over the audio tokens; heads of 128.
size_t a2v_bridge_ws_bytes(int B, int N, int Na, int heads);
prism_status launch_a2v_bridge(const void* x_v, const void* x_a,
                               const void* w_q, const void* w_k,
                               const void* w_v, const void* w_o,
                               const float* pos_v, const float* pos_a, int B,
                               int N, int Na, int Cv, int Ca, int heads,
                               float rope_base, void* dh, void* ws,
                               hipStream_t stream);

size_t attn_bwd_ws_bytes(int B, int Hh, int N, int d);
prism_status launch_attn_bwd(const void* q, const void* k, const void* v,
                             const void* o, const void* d_o, const float* lse,
                             int dtype, const int32_t* perm,
                             const int32_t* counts, const int32_t* kv_idx,
                             int capacity, int B, int Hh, int N, int d,
                             float scale, float* dq, float* dk, float* dv,
                             void* ws, hipStream_t stream);

}  // namespace prism
