/*
 * prism.h -- C ABI of the MI355X (gfx950) dynamic block-shape, block-sparse
 * video self-attention library (libprism.so).
 *
 * The method (Prism): the T x H x W video token grid is split into
 * spatiotemporal macro-zones; every zone picks one of 13 block shapes of 64
 * tokens from its directional feature variance plus the audio-to-video
 * residual norm; tokens are grouped into those blocks; queries and keys are
 * mean-pooled per block into a block proxy score; every query block keeps
 * its top-k KV blocks plus more in descending score order until the
 * cumulative proxy mass reaches cdf_threshold; attention then runs over the
 * kept blocks only.  Sources: "Tencent-Hunyuan/Prism" README, section
 * "Overview"; the Prism architecture walk-through (wmrh.cn), sections
 * "一个巧妙的联动：桥接残差反哺稀疏注意力" and
 * "三者如何协同：一步去噪里发生了什么"; the "Prism: Dynamic Sparse
 * Attention for Native 2K Joint Video-Audio Generation Model Training"
 * abstract page (block proxy scores, cumulative-mass selection, online
 * softmax over selected blocks).  A forward-only variant keeps the
 * unselected blocks in the softmax as pooled stand-ins built from the proxy
 * scores (prism_dropped_terms, prism_sparse_attn_fwd_corrected; the Sol-Attn
 * abstract listed on that page).
 *
 * Conventions shared by every call
 *  - Tensor pointers are DEVICE pointers owned by the caller.  The library
 *    never allocates, frees or keeps them; scratch memory comes in through
 *    `workspace` (size from the matching *_workspace_bytes query).
 *  - Every argument is checked on the host before any HIP call.  On a
 *    failed check nothing is written or enqueued and a non-zero status is
 *    returned; prism_last_error() gives a message (thread-local).
 *  - Work is only enqueued on `stream` (a hipStream_t; NULL = the null
 *    stream); results are valid once the caller synchronises that stream.
 *    The library never synchronises.
 *  - Token layout is raster order t*H*W + h*W + w.  Per-head tensors are
 *    [B, Hh, N, d] contiguous; block-ordered data is reached through `perm`
 *    (the caller never permutes tensors).
 *  - Float tensors (bf16 / fp32 / fp64) and workspaces must be 16-byte
 *    aligned (they are read and written with 16-byte vector accesses);
 *    int32 arrays, lse and zone_stats need their natural alignment.  A
 *    misaligned pointer is rejected with PRISM_ERR_INVALID_ARG.
 *  - Blocks always hold 64 tokens, so Nb = N / 64.
 *  - Calls that share a workspace or outputs must not overlap in time.
 */
#ifndef PRISM_H
#define PRISM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  PRISM_OK = 0,
  PRISM_ERR_INVALID_ARG = 1, /* null / misaligned pointer, size < 1, bad dtype, ... */
  PRISM_ERR_SHAPE = 2,       /* inconsistent sizes, zone without a legal shape */
  PRISM_ERR_UNSUPPORTED = 3, /* head_dim / dtype combination not built        */
  PRISM_ERR_WORKSPACE = 4,   /* workspace missing or too small                */
  PRISM_ERR_HIP = 5          /* a HIP launch or API call failed               */
} prism_status;

typedef enum { PRISM_FP32 = 0, PRISM_BF16 = 1 } prism_dtype;

#define PRISM_BLOCK_TOKENS 64
#define PRISM_NUM_SHAPES 13

/* Message of the last failed call on this thread ("" if none). */
const char* prism_last_error(void);

/* ABI version (major * 100 + minor). */
int prism_version(void);

/* Optional per-kernel timing, off by default.  While enabled, every kernel
 * the library launches is bracketed by two hipEvents recorded on its
 * stream (up to 4096 launches after the last enable / reset; later launches
 * are not recorded).  Events are created on the device current at the first
 * enable; use one device.  prism_profile_ms(i) waits for launch i to finish
 * and returns its duration in ms (-1 on error).  Not for concurrent use from
 * several host threads. */
int prism_profile_enable(int on);
void prism_profile_reset(void);
int prism_profile_count(void);
const char* prism_profile_name(int i);
float prism_profile_ms(int i);

/* The 13 candidate block shapes as (t, h, w) triples, written to
 * out_thw[3*id + {0,1,2}] (host memory, 39 ints).  Returns 13.  The pages
 * name (4,4,4), (8,2,4) and (2,4,8); the table holds every power-of-two
 * 64-token box whose longest side is at most 8x its shortest. */
int prism_shape_table(int32_t* out_thw);

/* ---------------------------------------------------------------------
 * Stage 1 -- zone shapes and token permutation.
 * README "Overview" and walk-through "三者如何协同": for each macro-zone the
 * directional variance v_a of the video features (per channel, along lines
 * parallel to axis a in {T, H, W}, averaged over lines and channels) and
 * the directional variance u_a of the per-token a2v residual RMS norm
 * ||dh||_2 / sqrt(C) combine as w_a = v_a + lambda_a2v * u_a; the zone takes
 * the legal shape (each extent divides the zone extent) minimising
 * sum_a w_a (e_a^2 - 1) / (L_a^2 - 1), lowest id on ties.
 *
 * feat, a2v_res : [B, N, C] raster tokens, dtype; a2v_res may be NULL (no
 *                 audio term).  Both may be NULL when fixed_shape >= 0.
 * zone_t/h/w    : macro-zone extents (8, 8, 8 in the pages' setting); zones
 *                 tile the grid from the origin, the last zone along an
 *                 axis keeps the remainder.  nZ = ceil(T/zt)*ceil(H/zh)*
 *                 ceil(W/zw).
 * fixed_shape   : -1 = choose per zone; 0..12 = force that shape everywhere.
 * zone_shape    : out [B, nZ] int32 shape ids (zones in raster order).
 * perm          : out [B, N] int32; perm[b][64*i + r] = raster token index of
 *                 the r-th token of block i.  Blocks are numbered zone-major,
 *                 the block lattice of a zone in raster order, tokens inside a
 *                 block in raster order.
 * inv_perm      : out [B, N] int32 (slot of each raster token) or NULL.
 * zone_stats    : out [B, nZ, 6] fp64 (v_T, v_H, v_W, u_T, u_H, u_W) or NULL.
 * Errors: SHAPE if N % 64 != 0, a zone has no legal shape, or fixed_shape
 * does not fit every zone; WORKSPACE if workspace_bytes is below
 * prism_zone_shapes_workspace_bytes(). */
size_t prism_zone_shapes_workspace_bytes(int B, int T, int H, int W, int C,
                                         int zone_t, int zone_h, int zone_w);
prism_status prism_zone_shapes(const void* feat, const void* a2v_res,
                               int dtype, int B, int T, int H, int W, int C,
                               int zone_t, int zone_h, int zone_w,
                               double lambda_a2v, int fixed_shape,
                               int32_t* zone_shape, int32_t* perm,
                               int32_t* inv_perm, double* zone_stats,
                               void* workspace, size_t workspace_bytes,
                               void* stream);

/* Allocation-free variant of prism_zone_shapes, for callers that cannot
 * allocate device memory or pass a workspace (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  Same arguments
 * and results as prism_zone_shapes without the workspace: the scratch (per
 * zone and channel slice partial sums, per-token residual norms) lives in a
 * device array of PRISM_ZONE_SHAPES_SCRATCH_BYTES inside the library, one
 * copy per GPU, held until the process ends.  Calls needing more scratch
 * than that -- prism_zone_shapes_workspace_bytes() above the limit; the 2K
 * grid with C = 3072 needs about 5.6 MB per batch element -- are rejected
 * with PRISM_ERR_WORKSPACE before any HIP call.  The array is shared by
 * every call on a GPU: calls that overlap in time on one GPU (different
 * streams or host threads) race and must be serialised by the caller.  The
 * call allocates nothing (no hipMalloc, no hipFree); its first use on a
 * device looks up that device's copy of the array. */
#define PRISM_ZONE_SHAPES_SCRATCH_BYTES (32u << 20)
prism_status prism_zone_shapes_noalloc(const void* feat, const void* a2v_res,
                                       int dtype, int B, int T, int H, int W,
                                       int C, int zone_t, int zone_h,
                                       int zone_w, double lambda_a2v,
                                       int fixed_shape, int32_t* zone_shape,
                                       int32_t* perm, int32_t* inv_perm,
                                       double* zone_stats, void* stream);

/* ---------------------------------------------------------------------
 * Stage 2 -- block mean-pooling and block proxy scores.
 * README "Overview" (block-level features) and the abstract page (block
 * proxy scores): qbar_i = mean of the 64 query rows of block i (kbar
 * likewise), accumulated in fp64; proxy[i][j] = softmax over j of
 * <qbar_i, kbar_j> / sqrt(d), over all Nb blocks of the same (b, h), fp64.
 *
 * q, k   : [B, Hh, N, d] dtype.  perm: [B, N] from stage 1.
 * q_mean, k_mean : out [B, Hh, Nb, d] fp64.
 * proxy  : out [B, Hh, Nb, Nb] fp64, rows sum to 1.
 * d must be 64 or 128. */
prism_status prism_pool_blocks(const void* q, const void* k, int dtype,
                               const int32_t* perm, int B, int Hh, int N,
                               int d, double* q_mean, double* k_mean,
                               double* proxy, void* stream);

/* ---------------------------------------------------------------------
 * Stage 3 -- hybrid top-k + top-p block selection.
 * Walk-through "三者如何协同": keep the top_k highest-scoring KV blocks, then
 * keep adding blocks in descending proxy order until the cumulative proxy
 * mass reaches cdf_threshold (default 0.20).  Order: descending score,
 * equal scores by lower block index.  The mass is the running fp64 sum in
 * that order; "reaches" means >=.  At least one block is kept; top_k is
 * clipped to Nb.  Count c = min(Nb, max(top_k, m*)), m* the first prefix
 * length whose mass reaches the threshold.
 *
 * proxy    : [B, Hh, Nb, Nb] fp64 (non-negative rows).
 * counts   : out [B, Hh, Nb] int32.
 * kv_idx   : out [B, Hh, Nb, capacity] int32, the first counts[...] entries
 *            of each row hold the kept block ids in ascending order; the
 *            rest of the row is not written.  capacity >= Nb.
 * Nb must be at most 8192.
 * Errors: INVALID_ARG if top_k < 0 or cdf_threshold is not in [0, 1]. */
prism_status prism_select_blocks(const double* proxy, int B, int Hh, int Nb,
                                 int top_k, double cdf_threshold,
                                 int32_t* counts, int32_t* kv_idx,
                                 int capacity, void* stream);

/* ---------------------------------------------------------------------
 * Stages 2-3 fused -- routing without the proxy matrix.
 * The Sol-Attn abstract on the Prism paper page counts computing and
 * materialising proxy scores as an overhead and thresholds blocks without
 * materialising the proxy map; the walk-through ("三者如何协同") runs top-k
 * then the CDF rule in one gating kernel.  This call pools q and k as
 * prism_pool_blocks does, then computes each query block's proxy row
 * (softmax over j of <qbar_i, kbar_j> / sqrt(d), fp64) on chip and selects
 * from it as prism_select_blocks does -- no [B, Hh, Nb, Nb] buffer exists.
 * Counts and lists equal those of prism_pool_blocks + prism_select_blocks
 * except where a decision lies within fp64 rounding of a tie (the logits
 * are accumulated in another order).
 *
 * q, k, dtype, perm, B, Hh, N, d : as prism_pool_blocks.
 * top_k, cdf_threshold : as prism_select_blocks.
 * q_mean, k_mean : out [B, Hh, Nb, d] fp64 (as prism_pool_blocks).
 * counts, kv_idx, capacity : out, as prism_select_blocks.
 * workspace : at least prism_route_blocks_workspace_bytes() (the pooled
 *             keys re-laid out for coalesced column reads: B*Hh*Nb*d fp64).
 * Nb must be at most 8192; d 64 or 128. */
size_t prism_route_blocks_workspace_bytes(int B, int Hh, int N, int d);
prism_status prism_route_blocks(const void* q, const void* k, int dtype,
                                const int32_t* perm, int B, int Hh, int N,
                                int d, int top_k, double cdf_threshold,
                                double* q_mean, double* k_mean,
                                int32_t* counts, int32_t* kv_idx, int capacity,
                                void* workspace, size_t workspace_bytes,
                                void* stream);

/* ---------------------------------------------------------------------
 * Stage 4 -- block-sparse attention, forward.
 * Abstract page (sparse computation over the selected KV blocks with online
 * softmax) and README "Overview": for each query block i and each of its 64
 * query rows, exact softmax attention over the 64 * counts[i] keys of the
 * listed blocks; no causal mask, no dropout.
 *
 * q, k, v : [B, Hh, N, d] dtype (bf16: MFMA path with fp32 accumulation;
 *           fp32: reference-precision path).
 * perm, counts, kv_idx, capacity : from stages 1 and 3.  Every count should
 *           be in [1, Nb], every listed id in [0, Nb) and the ids of one row
 *           distinct, in any order (caller's contract; stage 3 output
 *           satisfies it).  The lists live in device memory, so the host
 *           cannot check them; the kernels clamp each count to [0, Nb] and
 *           skip ids outside [0, Nb), so a list that breaks the contract
 *           never makes them read or write out of bounds.  A query block
 *           with no valid id gets o = 0 and lse = -inf (no key to attend
 *           to).  Duplicate ids count once in the bf16 path and once per
 *           copy in the fp32 path.  The bf16 path processes query blocks in pairs
 *           over the union of their lists: neighbours (within 16 places in
 *           the permuted order) whose lists overlap most, matched on the
 *           device from the lists in every call; results do not depend on
 *           the pairing.
 * softmax_scale : <= 0 means 1/sqrt(d).
 * Nb = N / 64 must be at most 8192 (UNSUPPORTED otherwise), as in stage 2.
 * o   : out [B, Hh, N, d] dtype, raster order.
 * lse : out [B, Hh, N] fp32, natural-log logsumexp of the scaled scores.
 * workspace: bf16 -- at least prism_sparse_attn_fwd_workspace_bytes()
 *           (list bitmaps and the pairing; about 2 * B * Hh * Nb^2 / 8
 *           bytes); WORKSPACE if missing or smaller.  fp32 -- unused, may
 *           be NULL. */
size_t prism_sparse_attn_fwd_workspace_bytes(int B, int Hh, int N, int d);
prism_status prism_sparse_attn_fwd(const void* q, const void* k,
                                   const void* v, int dtype,
                                   const int32_t* perm, const int32_t* counts,
                                   const int32_t* kv_idx, int capacity, int B,
                                   int Hh, int N, int d, float softmax_scale,
                                   void* o, float* lse, void* workspace,
                                   size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Stage 4 -- block-sparse attention, backward (training).
 * README "Overview": the method trains with the sparse attention, so the
 * gradient runs over the same kept blocks.  The selection is constant (no
 * gradient through routing).  With P = exp(s - lse) and D_r = <dO_r, O_r>:
 * dV = P^T dO, dS = P * (dO V^T - D), dQ = dS K * scale, dK = dS^T Q * scale.
 *
 * q, k, v, o, d_o : [B, Hh, N, d] dtype; lse [B, Hh, N] fp32 from the
 *                   forward.
 * dq, dk, dv      : out [B, Hh, N, d] fp32, raster order (fully written).
 *                   Lists are read as in the forward (counts clamped, ids
 *                   outside [0, Nb) skipped); a query block with no valid
 *                   id gets dq = 0 and adds nothing to dk, dv.
 * workspace       : at least prism_sparse_attn_bwd_workspace_bytes() (D
 *                   rows, list bitmaps, and the pairings of KV blocks and
 *                   of query blocks, as in the forward). */
size_t prism_sparse_attn_bwd_workspace_bytes(int B, int Hh, int N, int d);
prism_status prism_sparse_attn_bwd(const void* q, const void* k,
                                   const void* v, const void* o,
                                   const void* d_o, const float* lse,
                                   int dtype, const int32_t* perm,
                                   const int32_t* counts,
                                   const int32_t* kv_idx, int capacity, int B,
                                   int Hh, int N, int d, float softmax_scale,
                                   float* dq, float* dk, float* dv,
                                   void* workspace, size_t workspace_bytes,
                                   void* stream);

/* ---------------------------------------------------------------------
 * Stage 4 variant (forward only) -- a pooled stand-in for the KV blocks a
 * query block did not keep.
 * The Sol-Attn abstract (listed on the Prism paper page) keeps unselected
 * blocks in the online softmax approximately, by reusing their proxy
 * scores, instead of dropping them.  Reading: an unselected block j counts,
 * for every query row of block i, as its 64 keys all scoring the stage-2
 * logit z_ij = <qbar_i, kbar_j> / sqrt(d) and all carrying the block's mean
 * value vbar_j; the kept blocks stay exact; one softmax over both.
 *
 * prism_dropped_terms, per query block i, from the stage-2 probabilities
 * p_ij (reused, not recomputed) and the stage-3 lists:
 *   s_i        = sum of p_ij over the blocks i did not keep (fp64);
 *   drop_lse_i = ln 64 + L_i + ln s_i, L_i = ln sum_j exp(z_ij) taken as
 *                z_ij* - ln p_ij* at the row's largest p (fp64); -inf when
 *                s_i = 0 (every block kept);
 *   drop_v_i   = sum over the same blocks of p_ij vbar_j, divided by s_i
 *                (fp32 products and sums; 0 when s_i = 0).
 * proxy, q_mean, k_mean : stage-2 outputs, fp64 (proxy [B,Hh,Nb,Nb]).
 * v, dtype, perm : values [B, Hh, N, d] and the stage-1 permutation.
 * counts, kv_idx, capacity : stage-3 lists (same contract as the forward).
 * drop_lse : out [B, Hh, Nb] fp32.   drop_v : out [B, Hh, Nb, d] fp32.
 * workspace: at least prism_dropped_terms_workspace_bytes() (block means of
 *            v, fp32, and the two list bitmaps).
 *
 * prism_sparse_attn_fwd_corrected: prism_sparse_attn_fwd (same arguments,
 * same workspace) whose softmax also holds the stand-in.  Per row r of
 * block i, with o, lse the exact sparse results:
 *   lse'_r = ln(exp(lse_r) + exp(drop_lse_i)),
 *   o'_r   = exp(lse_r - lse'_r) o_r + exp(drop_lse_i - lse'_r) drop_v_i,
 * folded into the kernel's final normalisation (no extra pass over o).  A
 * row whose drop_lse is -inf gets exactly the prism_sparse_attn_fwd result.
 * There is no gradient of the stand-in: prism_sparse_attn_bwd differentiates
 * the exact sparse attention and takes that call's o and lse. */
size_t prism_dropped_terms_workspace_bytes(int B, int Hh, int N, int d);
prism_status prism_dropped_terms(const double* proxy, const double* q_mean,
                                 const double* k_mean, const void* v,
                                 int dtype, const int32_t* perm,
                                 const int32_t* counts, const int32_t* kv_idx,
                                 int capacity, int B, int Hh, int N, int d,
                                 float* drop_lse, float* drop_v,
                                 void* workspace, size_t workspace_bytes,
                                 void* stream);
prism_status prism_sparse_attn_fwd_corrected(
    const void* q, const void* k, const void* v, int dtype,
    const int32_t* perm, const int32_t* counts, const int32_t* kv_idx,
    int capacity, int B, int Hh, int N, int d, float softmax_scale,
    const float* drop_lse, const float* drop_v, void* o, float* lse,
    void* workspace, size_t workspace_bytes, void* stream);

/* ---------------------------------------------------------------------
 * Producer of stage 1's audio input -- the unscaled a2v bridge residual.
 * Walk-through sections "a2v / v2a 条件桥" and "一个巧妙的联动：桥接残差反哺稀疏
 * 注意力": a conditional cross-attention block whose queries are the video
 * tokens' hidden states (3072 wide in the pages' model) and whose keys and
 * values come from the audio tokens' hidden states (1536 wide); its output,
 * before the a2v_scale factor, is the residual whose per-token norm stage 1
 * reads.  The pages give no formula; this call computes multi-head scaled
 * dot-product cross-attention with linear projections (no bias, no
 * normalisation) and heads of 128 (D = 128 * heads):
 *   q = x_v Wq^T, k = x_a Wk^T, v = x_a Wv^T          (each [.., D])
 *   optional rotary alignment (both directions of the bridge support one):
 *     q and k of every head rotated pairwise, (2i, 2i+1) by angle
 *     pos * rope_base^(-2i / 128), pos the token's time position
 *   o_h = softmax(q_h k_h^T / sqrt(128)) v_h,  dh = concat_h(o_h) Wo^T.
 *
 * x_v   : [B, N, Cv] bf16 video hidden states (raster tokens).
 * x_a   : [B, Na, Ca] bf16 audio hidden states.
 * w_q   : [D, Cv], w_k, w_v : [D, Ca], w_o : [Cv, D]; bf16, [out, in].
 * pos_v : [B, N] fp32 and pos_a : [B, Na] fp32 time positions on one axis
 *         (e.g. audio steps), or both NULL (no rotation).
 * dtype : PRISM_BF16 (the only one built; UNSUPPORTED otherwise).
 * heads : even; Cv a multiple of 256, Ca of 64.
 * dh    : out [B, N, Cv] bf16 -- the unscaled residual (pass it to
 *         prism_zone_shapes as a2v_res).
 * workspace : at least prism_a2v_bridge_workspace_bytes() (the projected
 *         q -- overwritten by the attention output -- k and v, bf16).
 * Accumulation is fp32 on the bf16 matrix unit; q, k, v, the attention
 * output and dh are rounded to bf16. */
size_t prism_a2v_bridge_workspace_bytes(int B, int N, int Na, int Cv, int Ca,
                                        int heads);
prism_status prism_a2v_bridge(const void* x_v, const void* x_a,
                              const void* w_q, const void* w_k,
                              const void* w_v, const void* w_o,
                              const float* pos_v, const float* pos_a,
                              int dtype, int B, int N, int Na, int Cv, int Ca,
                              int heads, float rope_base, void* dh,
                              void* workspace, size_t workspace_bytes,
                              void* stream);

#ifdef __cplusplus
}
#endif

#endif /* PRISM_H */
