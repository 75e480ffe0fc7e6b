// C ABI layer: host-side argument checks, workspace sizing, dispatch.
// Every check runs before the first HIP call, so a rejected call enqueues
// nothing and writes nothing.
#include <math.h>
#include <mutex>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "prism_internal.h"

namespace prism {

static thread_local char g_err[512] = "";

prism_status fail(prism_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return st;
}

void clear_error() { g_err[0] = '\0'; }

prism_status check_launch(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess)
    return fail(PRISM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PRISM_OK;
}

// ------------------------------------------------------ kernel timing
namespace {
constexpr int kProfMax = 4096;
std::mutex g_prof_mu;
bool g_prof_on = false;
int g_prof_dev = -1;
int g_prof_n = 0;
hipEvent_t g_prof_ev[kProfMax][2];
const char* g_prof_name[kProfMax];
}  // namespace

ProfScope::ProfScope(hipStream_t s, const char* name) : slot(-1), stream(s) {
  if (!g_prof_on) return;
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (!g_prof_on || g_prof_n >= kProfMax) return;
  slot = g_prof_n++;
  g_prof_name[slot] = name;
  (void)hipEventRecord(g_prof_ev[slot][0], stream);
}

ProfScope::~ProfScope() {
  if (slot >= 0) (void)hipEventRecord(g_prof_ev[slot][1], stream);
}

static bool dtype_ok(int dtype) {
  return dtype == PRISM_FP32 || dtype == PRISM_BF16;
}

static prism_status make_geom(int T, int H, int W, int zt, int zh, int zw,
                              ZoneGeom* g) {
  PRISM_CHECK(T >= 1 && H >= 1 && W >= 1, PRISM_ERR_INVALID_ARG,
              "grid extents must be >= 1 (T=%d H=%d W=%d)", T, H, W);
  PRISM_CHECK(zt >= 1 && zh >= 1 && zw >= 1, PRISM_ERR_INVALID_ARG,
              "zone extents must be >= 1 (%d,%d,%d)", zt, zh, zw);
  PRISM_CHECK(zt <= 8 && zh <= 8 && zw <= 8, PRISM_ERR_UNSUPPORTED,
              "zone extents above 8 are not supported (%d,%d,%d)", zt, zh,
              zw);
  PRISM_CHECK((long long)T * H * W <= (1LL << 30), PRISM_ERR_UNSUPPORTED,
              "grid too large");
  PRISM_CHECK(((long long)T * H * W) % PRISM_BLOCK_TOKENS == 0,
              PRISM_ERR_SHAPE, "token count T*H*W=%lld is not a multiple of 64",
              (long long)T * H * W);
  g->T = T; g->H = H; g->W = W;
  g->zt = zt; g->zh = zh; g->zw = zw;
  g->nzt = ceil_div(T, zt); g->nzh = ceil_div(H, zh); g->nzw = ceil_div(W, zw);
  g->nZ = g->nzt * g->nzh * g->nzw;
  return PRISM_OK;
}

// Every zone extent kind (full or remainder along each axis) must admit the
// requested shape (fixed) or at least one shape (dynamic).
static prism_status check_zone_kinds(const ZoneGeom& g, int fixed_shape) {
  int lt[2] = {g.zt, g.T % g.zt ? g.T % g.zt : g.zt};
  int lh[2] = {g.zh, g.H % g.zh ? g.H % g.zh : g.zh};
  int lw[2] = {g.zw, g.W % g.zw ? g.W % g.zw : g.zw};
  if (g.T < g.zt) lt[0] = lt[1] = g.T;
  if (g.H < g.zh) lh[0] = lh[1] = g.H;
  if (g.W < g.zw) lw[0] = lw[1] = g.W;
  for (int a = 0; a < 2; ++a)
    for (int b = 0; b < 2; ++b)
      for (int c = 0; c < 2; ++c) {
        int Lt = lt[a], Lh = lh[b], Lw = lw[c];
        if (fixed_shape >= 0) {
          PRISM_CHECK(shape_fits(fixed_shape, Lt, Lh, Lw), PRISM_ERR_SHAPE,
                      "shape %d does not fit zone %dx%dx%d", fixed_shape, Lt,
                      Lh, Lw);
        } else {
          bool any = false;
          for (int s = 0; s < kNumShapes; ++s) any |= shape_fits(s, Lt, Lh, Lw);
          PRISM_CHECK(any, PRISM_ERR_SHAPE,
                      "no candidate shape fits zone %dx%dx%d", Lt, Lh, Lw);
        }
      }
  return PRISM_OK;
}

// Tensors are read and written with 16-byte vector accesses; index arrays
// and lse with 4-byte ones.
static bool aligned(const void* p, uintptr_t a) {
  return p == nullptr || (reinterpret_cast<uintptr_t>(p) % a) == 0;
}
#define PRISM_CHECK_ALIGNED(p, a)                                         \
  PRISM_CHECK(aligned((p), (a)), PRISM_ERR_INVALID_ARG,                   \
              "%s must be %d-byte aligned", #p, (int)(a))

static prism_status check_heads(int B, int Hh, int N, int d) {
  PRISM_CHECK(B >= 1 && Hh >= 1 && N >= 1 && d >= 1, PRISM_ERR_INVALID_ARG,
              "sizes must be >= 1 (B=%d Hh=%d N=%d d=%d)", B, Hh, N, d);
  PRISM_CHECK(N % PRISM_BLOCK_TOKENS == 0, PRISM_ERR_SHAPE,
              "N=%d is not a multiple of 64", N);
  PRISM_CHECK(d == 64 || d == 128, PRISM_ERR_UNSUPPORTED,
              "head_dim %d not built (64 or 128)", d);
  PRISM_CHECK((long long)B * Hh * N * d < (1LL << 40), PRISM_ERR_UNSUPPORTED,
              "tensor too large");
  return PRISM_OK;
}

}  // namespace prism

using namespace prism;

extern "C" {

const char* prism_last_error(void) { return g_err; }

int prism_version(void) { return 100; }

int prism_profile_enable(int on) {
  clear_error();
  std::lock_guard<std::mutex> lk(g_prof_mu);
  if (on && !g_prof_on) {
    if (g_prof_dev < 0) {
      if (hipGetDevice(&g_prof_dev) != hipSuccess) {
        g_prof_dev = -1;
        return fail(PRISM_ERR_HIP, "hipGetDevice failed");
      }
      for (int i = 0; i < kProfMax; ++i)
        for (int e = 0; e < 2; ++e)
          if (hipEventCreate(&g_prof_ev[i][e]) != hipSuccess)
            return fail(PRISM_ERR_HIP, "hipEventCreate failed");
    }
    g_prof_n = 0;
  }
  g_prof_on = on != 0;
  return PRISM_OK;
}

void prism_profile_reset(void) {
  std::lock_guard<std::mutex> lk(g_prof_mu);
  g_prof_n = 0;
}

int prism_profile_count(void) { return g_prof_n; }

const char* prism_profile_name(int i) {
  return (i >= 0 && i < g_prof_n) ? g_prof_name[i] : "";
}

float prism_profile_ms(int i) {
  if (i < 0 || i >= g_prof_n) return -1.f;
  if (hipEventSynchronize(g_prof_ev[i][1]) != hipSuccess) return -1.f;
  float ms = -1.f;
  if (hipEventElapsedTime(&ms, g_prof_ev[i][0], g_prof_ev[i][1]) != hipSuccess)
    return -1.f;
  return ms;
}

int prism_shape_table(int32_t* out_thw) {
  if (!out_thw) return kNumShapes;
  for (int s = 0; s < kNumShapes; ++s) {
    Shape sh = shape_of(s);
    out_thw[3 * s + 0] = sh.t;
    out_thw[3 * s + 1] = sh.h;
    out_thw[3 * s + 2] = sh.w;
  }
  return kNumShapes;
}

size_t prism_zone_shapes_workspace_bytes(int B, int T, int H, int W, int C,
                                         int zone_t, int zone_h, int zone_w) {
  ZoneGeom g;
  if (B < 1 || C < 1 || make_geom(T, H, W, zone_t, zone_h, zone_w, &g) != PRISM_OK)
    return 0;
  return zone_shapes_ws_bytes(B, g, C);
}

}  // extern "C"

namespace prism {
// Every argument check of stage 1 except the workspace's (shared by
// prism_zone_shapes and prism_zone_shapes_noalloc).
static prism_status check_zone_shapes(const void* feat, const void* a2v_res,
                                      int dtype, int B, int T, int H, int W,
                                      int C, int zone_t, int zone_h,
                                      int zone_w, double lambda_a2v,
                                      int fixed_shape, int32_t* zone_shape,
                                      int32_t* perm, int32_t* inv_perm,
                                      double* zone_stats, ZoneGeom* gout) {
  ZoneGeom& g = *gout;
  prism_status st = make_geom(T, H, W, zone_t, zone_h, zone_w, &g);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(B >= 1, PRISM_ERR_INVALID_ARG, "B=%d must be >= 1", B);
  PRISM_CHECK(fixed_shape >= -1 && fixed_shape < kNumShapes,
              PRISM_ERR_INVALID_ARG, "fixed_shape=%d outside [-1, 12]",
              fixed_shape);
  PRISM_CHECK(zone_shape && perm, PRISM_ERR_INVALID_ARG,
              "zone_shape and perm must not be NULL");
  PRISM_CHECK_ALIGNED(feat, 16);
  PRISM_CHECK_ALIGNED(a2v_res, 16);
  PRISM_CHECK_ALIGNED(zone_stats, 8);
  PRISM_CHECK_ALIGNED(zone_shape, 4);
  PRISM_CHECK_ALIGNED(perm, 4);
  PRISM_CHECK_ALIGNED(inv_perm, 4);
  st = check_zone_kinds(g, fixed_shape);
  if (st != PRISM_OK) return st;
  if (fixed_shape < 0) {
    PRISM_CHECK(feat != nullptr, PRISM_ERR_INVALID_ARG,
                "feat must not be NULL when shapes are chosen per zone");
    PRISM_CHECK(C >= 1, PRISM_ERR_INVALID_ARG, "C=%d must be >= 1", C);
    PRISM_CHECK(dtype_ok(dtype), PRISM_ERR_INVALID_ARG, "bad dtype %d", dtype);
    PRISM_CHECK(C % 8 == 0, PRISM_ERR_UNSUPPORTED,
                "C=%d must be a multiple of 8", C);
    PRISM_CHECK(isfinite(lambda_a2v) && lambda_a2v >= 0.0,
                PRISM_ERR_INVALID_ARG, "lambda_a2v must be finite and >= 0");
    PRISM_CHECK((long long)B * T * H * W * C < (1LL << 40),
                PRISM_ERR_UNSUPPORTED, "feature tensor too large");
  }
  return PRISM_OK;
}

// Scratch of prism_zone_shapes_noalloc: a file-scope device array, one copy
// per GPU, held until the process ends.  Host code never passes its name to
// a kernel (on the host it is only a stand-in symbol); the device address of
// each GPU's copy comes from hipGetSymbolAddress, taken once per device with
// that device current.
constexpr size_t kZoneScratchBytes = (size_t)PRISM_ZONE_SHAPES_SCRATCH_BYTES;
static __device__ __align__(256) unsigned char zone_scratch[kZoneScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};
}  // namespace

// Device address of the current GPU's copy of zone_scratch.
static prism_status zone_scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices)
    return fail(PRISM_ERR_HIP, "hipGetDevice failed or device id %d above %d",
                dev, kMaxDevices - 1);
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(zone_scratch));
    if (e != hipSuccess || p == nullptr)
      return fail(PRISM_ERR_HIP, "hipGetSymbolAddress(zone scratch): %s",
                  hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PRISM_OK;
}
}  // namespace prism

extern "C" {

prism_status prism_zone_shapes(const void* feat, const void* a2v_res,
                               int dtype, int B, int T, int H, int W, int C,
                               int zone_t, int zone_h, int zone_w,
                               double lambda_a2v, int fixed_shape,
                               int32_t* zone_shape, int32_t* perm,
                               int32_t* inv_perm, double* zone_stats,
                               void* workspace, size_t workspace_bytes,
                               void* stream) {
  clear_error();
  ZoneGeom g;
  prism_status st = check_zone_shapes(feat, a2v_res, dtype, B, T, H, W, C,
                                      zone_t, zone_h, zone_w, lambda_a2v,
                                      fixed_shape, zone_shape, perm, inv_perm,
                                      zone_stats, &g);
  if (st != PRISM_OK) return st;
  PRISM_CHECK_ALIGNED(workspace, 16);
  if (fixed_shape < 0) {
    size_t need = zone_shapes_ws_bytes(B, g, C);
    PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
                PRISM_ERR_WORKSPACE,
                "workspace of %zu bytes needed, %zu given", need,
                workspace ? workspace_bytes : (size_t)0);
  }
  return launch_zone_shapes(feat, a2v_res, dtype, B, g, C, lambda_a2v,
                            fixed_shape, zone_shape, perm, inv_perm,
                            zone_stats, workspace, (hipStream_t)stream);
}

prism_status prism_zone_shapes_noalloc(const void* feat, const void* a2v_res,
                                       int dtype, int B, int T, int H, int W,
                                       int C, int zone_t, int zone_h,
                                       int zone_w, double lambda_a2v,
                                       int fixed_shape, int32_t* zone_shape,
                                       int32_t* perm, int32_t* inv_perm,
                                       double* zone_stats, void* stream) {
  clear_error();
  ZoneGeom g;
  prism_status st = check_zone_shapes(feat, a2v_res, dtype, B, T, H, W, C,
                                      zone_t, zone_h, zone_w, lambda_a2v,
                                      fixed_shape, zone_shape, perm, inv_perm,
                                      zone_stats, &g);
  if (st != PRISM_OK) return st;
  void* scratch = nullptr;
  if (fixed_shape < 0) {
    const size_t need = zone_shapes_ws_bytes(B, g, C);
    PRISM_CHECK(need <= kZoneScratchBytes, PRISM_ERR_WORKSPACE,
                "the call needs %zu bytes of scratch; the allocation-free "
                "entry point holds %zu (use prism_zone_shapes with a "
                "workspace, or fewer batch elements per call)",
                need, kZoneScratchBytes);
    // every scratch word the kernels read is written earlier in the same
    // call, so nothing needs clearing
    if ((st = zone_scratch_ptr(&scratch)) != PRISM_OK) return st;
  }
  return launch_zone_shapes(feat, a2v_res, dtype, B, g, C, lambda_a2v,
                            fixed_shape, zone_shape, perm, inv_perm,
                            zone_stats, scratch, (hipStream_t)stream);
}

prism_status prism_pool_blocks(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               double* proxy, void* stream) {
  clear_error();
  prism_status st = check_heads(B, Hh, N, d);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(dtype_ok(dtype), PRISM_ERR_INVALID_ARG, "bad dtype %d", dtype);
  PRISM_CHECK(q && k && perm && q_mean && k_mean && proxy,
              PRISM_ERR_INVALID_ARG, "null pointer argument");
  PRISM_CHECK_ALIGNED(q, 16);
  PRISM_CHECK_ALIGNED(k, 16);
  PRISM_CHECK_ALIGNED(q_mean, 16);
  PRISM_CHECK_ALIGNED(k_mean, 16);
  PRISM_CHECK_ALIGNED(proxy, 16);
  PRISM_CHECK_ALIGNED(perm, 4);
  const int Nb = N / PRISM_BLOCK_TOKENS;
  PRISM_CHECK(Nb <= 8192, PRISM_ERR_UNSUPPORTED, "Nb=%d above 8192", Nb);
  return launch_pool_proxy(q, k, dtype, perm, B, Hh, N, d, q_mean, k_mean,
                           proxy, (hipStream_t)stream);
}

prism_status prism_select_blocks(const double* proxy, int B, int Hh, int Nb,
                                 int top_k, double cdf_threshold,
                                 int32_t* counts, int32_t* kv_idx,
                                 int capacity, void* stream) {
  clear_error();
  PRISM_CHECK(B >= 1 && Hh >= 1 && Nb >= 1, PRISM_ERR_INVALID_ARG,
              "sizes must be >= 1 (B=%d Hh=%d Nb=%d)", B, Hh, Nb);
  PRISM_CHECK(proxy && counts && kv_idx, PRISM_ERR_INVALID_ARG,
              "null pointer argument");
  PRISM_CHECK_ALIGNED(proxy, 8);
  PRISM_CHECK_ALIGNED(counts, 4);
  PRISM_CHECK_ALIGNED(kv_idx, 4);
  PRISM_CHECK(top_k >= 0, PRISM_ERR_INVALID_ARG, "top_k=%d must be >= 0",
              top_k);
  PRISM_CHECK(cdf_threshold >= 0.0 && cdf_threshold <= 1.0,
              PRISM_ERR_INVALID_ARG, "cdf_threshold=%g outside [0, 1]",
              cdf_threshold);
  PRISM_CHECK(capacity >= Nb, PRISM_ERR_SHAPE, "capacity=%d < Nb=%d",
              capacity, Nb);
  PRISM_CHECK(Nb <= 8192, PRISM_ERR_UNSUPPORTED, "Nb=%d above 8192", Nb);
  return launch_select(proxy, B, Hh, Nb, top_k, cdf_threshold, counts, kv_idx,
                       capacity, (hipStream_t)stream);
}

size_t prism_route_blocks_workspace_bytes(int B, int Hh, int N, int d) {
  if (check_heads(B, Hh, N, d) != PRISM_OK) return 0;
  return route_fused_ws_bytes(B, Hh, N / PRISM_BLOCK_TOKENS, d);
}

prism_status prism_route_blocks(const void* q, const void* k, int dtype,
                                const int32_t* perm, int B, int Hh, int N,
                                int d, int top_k, double cdf_threshold,
                                double* q_mean, double* k_mean,
                                int32_t* counts, int32_t* kv_idx, int capacity,
                                void* workspace, size_t workspace_bytes,
                                void* stream) {
  clear_error();
  prism_status st = check_heads(B, Hh, N, d);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(dtype_ok(dtype), PRISM_ERR_INVALID_ARG, "bad dtype %d", dtype);
  PRISM_CHECK(q && k && perm && q_mean && k_mean && counts && kv_idx,
              PRISM_ERR_INVALID_ARG, "null pointer argument");
  PRISM_CHECK_ALIGNED(q, 16);
  PRISM_CHECK_ALIGNED(k, 16);
  PRISM_CHECK_ALIGNED(q_mean, 16);
  PRISM_CHECK_ALIGNED(k_mean, 16);
  PRISM_CHECK_ALIGNED(perm, 4);
  PRISM_CHECK_ALIGNED(counts, 4);
  PRISM_CHECK_ALIGNED(kv_idx, 4);
  const int Nb = N / PRISM_BLOCK_TOKENS;
  PRISM_CHECK(Nb <= 8192, PRISM_ERR_UNSUPPORTED, "Nb=%d above 8192", Nb);
  PRISM_CHECK(top_k >= 0, PRISM_ERR_INVALID_ARG, "top_k=%d must be >= 0",
              top_k);
  PRISM_CHECK(cdf_threshold >= 0.0 && cdf_threshold <= 1.0,
              PRISM_ERR_INVALID_ARG, "cdf_threshold=%g outside [0, 1]",
              cdf_threshold);
  PRISM_CHECK(capacity >= Nb, PRISM_ERR_SHAPE, "capacity=%d < Nb=%d",
              capacity, Nb);
  PRISM_CHECK_ALIGNED(workspace, 16);
  const size_t need = route_fused_ws_bytes(B, Hh, Nb, d);
  PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
              PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  hipStream_t s = (hipStream_t)stream;
  if ((st = launch_pool_means(q, k, dtype, perm, B, Hh, N, d, q_mean, k_mean,
                              s)) != PRISM_OK)
    return st;
  return launch_route_fused(q_mean, k_mean, B, Hh, Nb, d, top_k, cdf_threshold,
                            counts, kv_idx, capacity, workspace, s);
}

size_t prism_sparse_attn_fwd_workspace_bytes(int B, int Hh, int N, int d) {
  if (check_heads(B, Hh, N, d) != PRISM_OK) return 0;
  return attn_fwd_ws_bytes(B, Hh, N, d);
}

static prism_status check_attn_common(const void* q, const void* k,
                                      const void* v, int dtype,
                                      const int32_t* perm,
                                      const int32_t* counts,
                                      const int32_t* kv_idx, int capacity,
                                      int B, int Hh, int N, int d,
                                      float softmax_scale) {
  prism_status st = check_heads(B, Hh, N, d);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(dtype_ok(dtype), PRISM_ERR_INVALID_ARG, "bad dtype %d", dtype);
  PRISM_CHECK(q && k && v && perm && counts && kv_idx, PRISM_ERR_INVALID_ARG,
              "null pointer argument");
  PRISM_CHECK_ALIGNED(q, 16);
  PRISM_CHECK_ALIGNED(k, 16);
  PRISM_CHECK_ALIGNED(v, 16);
  PRISM_CHECK_ALIGNED(perm, 4);
  PRISM_CHECK_ALIGNED(counts, 4);
  PRISM_CHECK_ALIGNED(kv_idx, 4);
  PRISM_CHECK(capacity >= N / PRISM_BLOCK_TOKENS, PRISM_ERR_SHAPE,
              "capacity=%d < Nb=%d", capacity, N / PRISM_BLOCK_TOKENS);
  PRISM_CHECK(N / PRISM_BLOCK_TOKENS <= 8192, PRISM_ERR_UNSUPPORTED,
              "Nb=%d above 8192", N / PRISM_BLOCK_TOKENS);
  PRISM_CHECK(isfinite(softmax_scale), PRISM_ERR_INVALID_ARG,
              "softmax_scale must be finite");
  return PRISM_OK;
}

prism_status prism_sparse_attn_fwd(const void* q, const void* k,
                                   const void* v, int dtype,
                                   const int32_t* perm, const int32_t* counts,
                                   const int32_t* kv_idx, int capacity, int B,
                                   int Hh, int N, int d, float softmax_scale,
                                   void* o, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream) {
  clear_error();
  prism_status st = check_attn_common(q, k, v, dtype, perm, counts, kv_idx,
                                      capacity, B, Hh, N, d, softmax_scale);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(o && lse, PRISM_ERR_INVALID_ARG, "null output pointer");
  PRISM_CHECK_ALIGNED(o, 16);
  PRISM_CHECK_ALIGNED(lse, 4);
  if (dtype == PRISM_BF16) {
    PRISM_CHECK_ALIGNED(workspace, 16);
    const size_t need = attn_fwd_ws_bytes(B, Hh, N, d);
    PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
                PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                need, workspace ? workspace_bytes : (size_t)0);
  }
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  return launch_attn_fwd(q, k, v, dtype, perm, counts, kv_idx, capacity, B,
                         Hh, N, d, scale, nullptr, nullptr, o, lse, workspace,
                         (hipStream_t)stream);
}

size_t prism_dropped_terms_workspace_bytes(int B, int Hh, int N, int d) {
  if (check_heads(B, Hh, N, d) != PRISM_OK) return 0;
  return dropped_terms_ws_bytes(B, Hh, N, d);
}

prism_status prism_dropped_terms(const double* proxy, const double* q_mean,
                                 const double* k_mean, const void* v,
                                 int dtype, const int32_t* perm,
                                 const int32_t* counts, const int32_t* kv_idx,
                                 int capacity, int B, int Hh, int N, int d,
                                 float* drop_lse, float* drop_v,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream) {
  clear_error();
  prism_status st = check_heads(B, Hh, N, d);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(dtype_ok(dtype), PRISM_ERR_INVALID_ARG, "bad dtype %d", dtype);
  PRISM_CHECK(proxy && q_mean && k_mean && v && perm && counts && kv_idx &&
                  drop_lse && drop_v,
              PRISM_ERR_INVALID_ARG, "null pointer argument");
  PRISM_CHECK_ALIGNED(proxy, 8);
  PRISM_CHECK_ALIGNED(q_mean, 8);
  PRISM_CHECK_ALIGNED(k_mean, 8);
  PRISM_CHECK_ALIGNED(v, 16);
  PRISM_CHECK_ALIGNED(perm, 4);
  PRISM_CHECK_ALIGNED(counts, 4);
  PRISM_CHECK_ALIGNED(kv_idx, 4);
  PRISM_CHECK_ALIGNED(drop_lse, 4);
  PRISM_CHECK_ALIGNED(drop_v, 16);
  PRISM_CHECK_ALIGNED(workspace, 16);
  const int Nb = N / PRISM_BLOCK_TOKENS;
  PRISM_CHECK(capacity >= Nb, PRISM_ERR_SHAPE, "capacity=%d < Nb=%d", capacity,
              Nb);
  PRISM_CHECK(Nb <= 8192, PRISM_ERR_UNSUPPORTED, "Nb=%d above 8192", Nb);
  const size_t need = dropped_terms_ws_bytes(B, Hh, N, d);
  PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
              PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  return launch_dropped_terms(proxy, q_mean, k_mean, v, dtype, perm, counts,
                              kv_idx, capacity, B, Hh, N, d, drop_lse, drop_v,
                              workspace, (hipStream_t)stream);
}

prism_status prism_sparse_attn_fwd_corrected(
    const void* q, const void* k, const void* v, int dtype,
    const int32_t* perm, const int32_t* counts, const int32_t* kv_idx,
    int capacity, int B, int Hh, int N, int d, float softmax_scale,
    const float* drop_lse, const float* drop_v, void* o, float* lse,
    void* workspace, size_t workspace_bytes, void* stream) {
  clear_error();
  prism_status st = check_attn_common(q, k, v, dtype, perm, counts, kv_idx,
                                      capacity, B, Hh, N, d, softmax_scale);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(o && lse && drop_lse && drop_v, PRISM_ERR_INVALID_ARG,
              "null pointer argument");
  PRISM_CHECK_ALIGNED(o, 16);
  PRISM_CHECK_ALIGNED(lse, 4);
  PRISM_CHECK_ALIGNED(drop_lse, 4);
  PRISM_CHECK_ALIGNED(drop_v, 16);
  if (dtype == PRISM_BF16) {
    PRISM_CHECK_ALIGNED(workspace, 16);
    const size_t need = attn_fwd_ws_bytes(B, Hh, N, d);
    PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
                PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
                need, workspace ? workspace_bytes : (size_t)0);
  }
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  return launch_attn_fwd(q, k, v, dtype, perm, counts, kv_idx, capacity, B,
                         Hh, N, d, scale, drop_lse, drop_v, o, lse, workspace,
                         (hipStream_t)stream);
}

static prism_status check_bridge(int B, int N, int Na, int Cv, int Ca,
                                 int heads) {
  PRISM_CHECK(B >= 1 && N >= 1 && Na >= 1 && Cv >= 1 && Ca >= 1 && heads >= 1,
              PRISM_ERR_INVALID_ARG,
              "sizes must be >= 1 (B=%d N=%d Na=%d Cv=%d Ca=%d heads=%d)", B,
              N, Na, Cv, Ca, heads);
  PRISM_CHECK(heads % 2 == 0, PRISM_ERR_UNSUPPORTED,
              "heads=%d must be even (projection tiles of 256 columns)", heads);
  PRISM_CHECK(Cv % 256 == 0 && Ca % 64 == 0, PRISM_ERR_UNSUPPORTED,
              "Cv=%d must be a multiple of 256 and Ca=%d of 64", Cv, Ca);
  const long long D = 128LL * heads;
  PRISM_CHECK((long long)B * N * (D > Cv ? D : Cv) * 2 < (1LL << 40) &&
                  256LL * (D > Cv ? D : Cv) * 2 < (1LL << 31) &&
                  (long long)B * Na * (Ca > D ? Ca : D) < (1LL << 40) &&
                  (long long)B * N < (1LL << 31),
              PRISM_ERR_UNSUPPORTED, "tensors too large");
  return PRISM_OK;
}

size_t prism_a2v_bridge_workspace_bytes(int B, int N, int Na, int Cv, int Ca,
                                        int heads) {
  if (check_bridge(B, N, Na, Cv, Ca, heads) != PRISM_OK) return 0;
  return a2v_bridge_ws_bytes(B, N, Na, heads);
}

prism_status prism_a2v_bridge(const void* x_v, const void* x_a,
                              const void* w_q, const void* w_k,
                              const void* w_v, const void* w_o,
                              const float* pos_v, const float* pos_a,
                              int dtype, int B, int N, int Na, int Cv, int Ca,
                              int heads, float rope_base, void* dh,
                              void* workspace, size_t workspace_bytes,
                              void* stream) {
  clear_error();
  prism_status st = check_bridge(B, N, Na, Cv, Ca, heads);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(dtype == PRISM_BF16, PRISM_ERR_UNSUPPORTED,
              "the bridge is built for bf16 only (dtype %d)", dtype);
  PRISM_CHECK(x_v && x_a && w_q && w_k && w_v && w_o && dh,
              PRISM_ERR_INVALID_ARG, "null pointer argument");
  PRISM_CHECK((pos_v == nullptr) == (pos_a == nullptr), PRISM_ERR_INVALID_ARG,
              "give both rotary position arrays or neither");
  PRISM_CHECK(isfinite(rope_base) && rope_base > 1.f, PRISM_ERR_INVALID_ARG,
              "rope_base must be finite and > 1");
  PRISM_CHECK_ALIGNED(x_v, 16);
  PRISM_CHECK_ALIGNED(x_a, 16);
  PRISM_CHECK_ALIGNED(w_q, 16);
  PRISM_CHECK_ALIGNED(w_k, 16);
  PRISM_CHECK_ALIGNED(w_v, 16);
  PRISM_CHECK_ALIGNED(w_o, 16);
  PRISM_CHECK_ALIGNED(dh, 16);
  PRISM_CHECK_ALIGNED(pos_v, 4);
  PRISM_CHECK_ALIGNED(pos_a, 4);
  PRISM_CHECK_ALIGNED(workspace, 16);
  const size_t need = a2v_bridge_ws_bytes(B, N, Na, heads);
  PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
              PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  return launch_a2v_bridge(x_v, x_a, w_q, w_k, w_v, w_o, pos_v, pos_a, B, N,
                           Na, Cv, Ca, heads, rope_base, dh, workspace,
                           (hipStream_t)stream);
}

size_t prism_sparse_attn_bwd_workspace_bytes(int B, int Hh, int N, int d) {
  if (check_heads(B, Hh, N, d) != PRISM_OK) return 0;
  return attn_bwd_ws_bytes(B, Hh, N, d);
}

prism_status prism_sparse_attn_bwd(const void* q, const void* k,
                                   const void* v, const void* o,
                                   const void* d_o, const float* lse,
                                   int dtype, const int32_t* perm,
                                   const int32_t* counts,
                                   const int32_t* kv_idx, int capacity, int B,
                                   int Hh, int N, int d, float softmax_scale,
                                   float* dq, float* dk, float* dv,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream) {
  clear_error();
  prism_status st = check_attn_common(q, k, v, dtype, perm, counts, kv_idx,
                                      capacity, B, Hh, N, d, softmax_scale);
  if (st != PRISM_OK) return st;
  PRISM_CHECK(o && d_o && lse && dq && dk && dv, PRISM_ERR_INVALID_ARG,
              "null pointer argument");
  PRISM_CHECK_ALIGNED(o, 16);
  PRISM_CHECK_ALIGNED(d_o, 16);
  PRISM_CHECK_ALIGNED(lse, 4);
  PRISM_CHECK_ALIGNED(dq, 16);
  PRISM_CHECK_ALIGNED(dk, 16);
  PRISM_CHECK_ALIGNED(dv, 16);
  PRISM_CHECK_ALIGNED(workspace, 16);
  size_t need = attn_bwd_ws_bytes(B, Hh, N, d);
  PRISM_CHECK(workspace != nullptr && workspace_bytes >= need,
              PRISM_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given",
              need, workspace ? workspace_bytes : (size_t)0);
  float scale = softmax_scale > 0.f ? softmax_scale : 1.0f / sqrtf((float)d);
  return launch_attn_bwd(q, k, v, o, d_o, lse, dtype, perm, counts, kv_idx,
                         capacity, B, Hh, N, d, scale, dq, dk, dv, workspace,
                         (hipStream_t)stream);
}

}  // extern "C"
