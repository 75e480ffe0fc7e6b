"""Plain fp64 CPU oracle for dynamic block-shape, block-sparse video attention.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module; the library's compute
path never does.  It shares no code with the HIP kernels.

Sources (web pages describing Prism):
  * "Tencent-Hunyuan/Prism" README, section "Overview": macro-zones; per-zone
    video feature variance along the channel and audio-to-video feature
    norms; a tailored block shape per zone with finer partitioning along axes
    of rapid variation and strong audio-visual coupling; block-level
    features; hybrid block selection for per-query sparsity.
  * The Prism architecture walk-through (wmrh.cn), sections
    "一个巧妙的联动：桥接残差反哺稀疏注意力" (the per-token L2 norm of the
    unscaled a2v bridge residual is the audio-influence signal) and
    "三者如何协同：一步去噪里发生了什么" (13 candidate shapes such as
    (4,4,4), (8,2,4), (2,4,8); choice by content variance plus audio
    coupling; top-k first, then continue along the CDF up to cdf_threshold,
    default 0.20).
  * "Prism: Dynamic Sparse Attention for Native 2K Joint Video-Audio
    Generation Model Training" abstract page: block proxy scores, keeping
    blocks until a cumulative proxy mass is reached, online softmax over the
    selected key/value blocks only.

Where the pages leave a step open this file takes the plainest reading and
names it "reading Rn"; the readings are listed with their reasons in the
design notes.  Every float is fp64.  Inputs are the exact buffers the GPU
receives (fp32 or bf16), widened to fp64 by the caller.

Parity pins: every function here is checked in tests/test_oracle_*.py
against closed forms, brute force, invariants and library special cases.
The shape rule's exact constants (reading R2-R7) go beyond what the pages
fix; only its qualitative behaviour on the pages' three named shapes is
pinned to them.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence, Tuple

import numpy as np

BLOCK = 64  # tokens per block; all three example shapes hold 64 tokens

# Reading R1/R2: 13 candidate (t, h, w) extents.  The pages name three of
# them -- (4,4,4) isotropic, (8,2,4) fine along H (mouths / faces), (2,4,8)
# fine along T (fast motion).  The table is every power-of-two 64-token box
# whose longest side is at most 8 times its shortest.
SHAPES: Tuple[Tuple[int, int, int], ...] = (
    (4, 4, 4), (2, 4, 8), (2, 8, 4), (4, 2, 8), (4, 8, 2), (8, 2, 4),
    (8, 4, 2), (1, 8, 8), (8, 1, 8), (8, 8, 1), (2, 2, 16), (2, 16, 2),
    (16, 2, 2),
)

REL_MARGIN_FLAG = 1e-9  # decisions closer than this are reported (R16)


# ---------------------------------------------------------------------------
# Stage 1: macro-zones, zone statistics, shape choice, token permutation
# ---------------------------------------------------------------------------
def zone_tiling(T: int, H: int, W: int, zone=(8, 8, 8)):
    """Macro-zones tiled from the origin, remainders kept (reading R3).

    Returns a list of ((t0, h0, w0), (Lt, Lh, Lw)) in raster zone order
    (w fastest).  README "Overview": the token grid is organised into
    spatiotemporal macro-zones.
    """
    zones = []
    for t0 in range(0, T, zone[0]):
        for h0 in range(0, H, zone[1]):
            for w0 in range(0, W, zone[2]):
                zones.append(((t0, h0, w0),
                              (min(zone[0], T - t0), min(zone[1], H - h0),
                               min(zone[2], W - w0))))
    return zones


def directional_variance(x: np.ndarray) -> np.ndarray:
    """Mean population variance along each grid axis (reading R4).

    ``x`` is a zone's values, shape (Lt, Lh, Lw) or (Lt, Lh, Lw, C).  For axis
    a, every line of the zone parallel to a (and every channel) gets its
    population variance; the result is the mean over lines and channels.
    README "Overview": variance of the video features along the channel,
    capturing how the content varies directionally.
    """
    x = np.asarray(x, dtype=np.float64)
    return np.array([np.var(x, axis=a).mean() for a in range(3)])


def token_rms_norm(a2v: np.ndarray) -> np.ndarray:
    """Per-token L2 norm of the a2v residual divided by sqrt(C) (reading R5).

    Walk-through, bridge-residual section: the per-token L2 norm of the
    *unscaled* a2v residual measures how strongly audio drives a region.
    ``a2v`` is (..., C); the result drops the last axis.
    """
    a2v = np.asarray(a2v, dtype=np.float64)
    return np.sqrt(np.sum(a2v * a2v, axis=-1)) / math.sqrt(a2v.shape[-1])


def zone_statistics(feat_zone: np.ndarray,
                    a2v_zone: Optional[np.ndarray]) -> np.ndarray:
    """[v_T, v_H, v_W, u_T, u_H, u_W] for one zone (readings R4, R5).

    v: directional variance of the video features; u: directional variance
    of the a2v RMS norm (zero when no residual is given).
    """
    v = directional_variance(feat_zone)
    if a2v_zone is None:
        u = np.zeros(3)
    else:
        u = directional_variance(token_rms_norm(a2v_zone))
    return np.concatenate([v, u])


def shape_is_legal(shape, extents) -> bool:
    """A shape fits a zone iff each of its extents divides the zone's."""
    return all(L % e == 0 for e, L in zip(shape, extents))


def shape_cost(w: Sequence[float], extents, shape) -> float:
    """Predicted within-block variance of a shape (reading R7).

    For a field that changes linearly along axis a, a line of L points has
    variance g^2 (L^2 - 1) / 12 and a block side of e points g^2 (e^2 - 1)/12,
    so w_a (e_a^2 - 1) / (L_a^2 - 1) is the within-block share of the measured
    directional variance w_a.  The three terms are added smallest first, so
    two shapes whose costs are equal as real numbers (the same terms in
    another axis order) also compare equal in floating point and the tie
    falls to the lower table id.
    """
    terms = []
    for a in range(3):
        L = extents[a]
        f = (shape[a] * shape[a] - 1) / (L * L - 1) if L > 1 else 0.0
        terms.append(w[a] * f)
    terms.sort()
    return (terms[0] + terms[1]) + terms[2]


def choose_shape(stats: np.ndarray, extents, lam: float = 1.0,
                 fixed_shape: int = -1):
    """Shape id for one zone: argmin of the cost, lowest id on ties.

    Walk-through, "三者如何协同": each macro-zone picks one of the 13 shapes
    by content variance plus audio coupling strength (reading R6: the two
    signals add, w_a = v_a + lam * u_a).  README "Overview": finer partitions
    go along axes of rapid visual change and strong audio-visual coupling --
    the minimum-cost shape is shortest where w_a is largest.

    Returns (shape_id, relative margin to the runner-up).
    """
    if fixed_shape >= 0:
        return fixed_shape, math.inf
    w = [stats[a] + lam * stats[3 + a] for a in range(3)]
    costs = []
    for sid, s in enumerate(SHAPES):
        if shape_is_legal(s, extents):
            costs.append((shape_cost(w, extents, s), sid))
    if not costs:
        raise ValueError(f"no legal shape for zone extents {extents}")
    best_J, best = costs[0]
    for J, sid in costs[1:]:
        if J < best_J:
            best_J, best = J, sid
    others = [J for J, sid in costs if sid != best]
    if not others:
        return best, math.inf
    second = min(others)
    scale = max(abs(best_J), abs(second))
    margin = (second - best_J) / scale if scale > 0 else 0.0
    return best, margin


def block_permutation(T: int, H: int, W: int, zones, shape_ids) -> np.ndarray:
    """perm[slot] = raster token index (reading R8).

    Blocks are numbered zone-major (zones in raster order); inside a zone the
    lattice of blocks is in raster order, and inside a block the tokens are in
    raster order.  Slot = 64 * block + position in block.
    """
    perm = np.empty(T * H * W, dtype=np.int64)
    slot = 0
    for ((t0, h0, w0), (Lt, Lh, Lw)), sid in zip(zones, shape_ids):
        et, eh, ew = SHAPES[sid]
        for bt in range(Lt // et):
            for bh in range(Lh // eh):
                for bw in range(Lw // ew):
                    dt, dh, dw = np.meshgrid(np.arange(et), np.arange(eh),
                                             np.arange(ew), indexing="ij")
                    t = t0 + bt * et + dt.ravel()
                    h = h0 + bh * eh + dh.ravel()
                    w = w0 + bw * ew + dw.ravel()
                    n = t.size
                    perm[slot:slot + n] = (t * H + h) * W + w
                    slot += n
    assert slot == T * H * W
    return perm


def zone_shapes(feat: Optional[np.ndarray], a2v: Optional[np.ndarray],
                T: int, H: int, W: int, zone=(8, 8, 8), lam: float = 1.0,
                fixed_shape: int = -1):
    """Stage 1 for one batch element.

    ``feat`` and ``a2v`` are [N, C] (raster tokens; fp64 or widenable), or
    None when ``fixed_shape`` >= 0 (then no statistics are needed) -- a2v may
    be None on its own (no audio term).
    Returns dict(zone_shape [nZ], perm [N], stats [nZ, 6], margin [nZ]).
    """
    N = T * H * W
    if N % BLOCK:
        raise ValueError("token count must be a multiple of 64")
    zones = zone_tiling(T, H, W, zone)
    nZ = len(zones)
    ids = np.empty(nZ, dtype=np.int64)
    stats = np.zeros((nZ, 6))
    margin = np.full(nZ, math.inf)
    if feat is not None:
        F = np.asarray(feat).reshape(T, H, W, -1)
    if a2v is not None:
        A = np.asarray(a2v).reshape(T, H, W, -1)
    for z, ((t0, h0, w0), (Lt, Lh, Lw)) in enumerate(zones):
        ext = (Lt, Lh, Lw)
        if fixed_shape >= 0:
            if not shape_is_legal(SHAPES[fixed_shape], ext):
                raise ValueError(f"shape {fixed_shape} does not fit {ext}")
            ids[z] = fixed_shape
            continue
        sl = (slice(t0, t0 + Lt), slice(h0, h0 + Lh), slice(w0, w0 + Lw))
        fz = np.asarray(F[sl], dtype=np.float64)
        az = None if a2v is None else np.asarray(A[sl], dtype=np.float64)
        stats[z] = zone_statistics(fz, az)
        ids[z], margin[z] = choose_shape(stats[z], ext, lam)
    perm = block_permutation(T, H, W, zones, ids)
    return dict(zone_shape=ids, perm=perm, stats=stats, margin=margin,
                zones=zones)


# ---------------------------------------------------------------------------
# Stage 2: block mean-pooling and the block proxy score
# ---------------------------------------------------------------------------
def pool_blocks(x: np.ndarray, perm: np.ndarray) -> np.ndarray:
    """Mean of the 64 tokens of each block (reading R9).  x: [N, d]."""
    x = np.asarray(x, dtype=np.float64)
    nb = x.shape[0] // BLOCK
    return x[np.asarray(perm)].reshape(nb, BLOCK, -1).mean(axis=1)


def proxy_scores(q_mean: np.ndarray, k_mean: np.ndarray) -> np.ndarray:
    """Row softmax over KV blocks of the pooled-score matrix (reading R10).

    z_ij = <qbar_i, kbar_j> / sqrt(d); p_i = softmax_j(z_i) over all blocks
    of the same head.  The abstract page calls these block proxy scores;
    README "Overview": block-level features stand for the block.
    """
    d = q_mean.shape[1]
    z = (q_mean @ k_mean.T) / math.sqrt(d)
    z = z - z.max(axis=1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=1, keepdims=True)


# ---------------------------------------------------------------------------
# Stage 3: hybrid top-k + top-p selection
# ---------------------------------------------------------------------------
def select_row(p: np.ndarray, top_k: int, cdf_threshold: float):
    """Selected KV blocks of one query block, ascending (readings R11-R13).

    Walk-through, "三者如何协同": take the k highest-scoring blocks, then keep
    adding blocks in descending score order while the cumulative proxy mass
    is below cdf_threshold.  Order: descending p, equal p by lower index.
    The mass is summed in that order, one block at a time.  At least one
    block is kept; k beyond the row length is clipped.
    """
    p = np.asarray(p, dtype=np.float64)
    nb = p.size
    order = np.lexsort((np.arange(nb), -p))
    c = min(max(top_k, 0), nb)
    mass = 0.0
    for r in range(c):
        mass += p[order[r]]
    while c < nb and (c < 1 or mass < cdf_threshold):
        mass += p[order[c]]
        c += 1
    return np.sort(order[:c])


def select_blocks(P: np.ndarray, top_k: int, cdf_threshold: float):
    """``select_row`` over every row of P, vectorised across rows.

    Returns (counts [nb], lists: list of ascending int arrays, diagnostics).
    The cumulative mass is a sequential running sum along each sorted row
    (numpy's add.accumulate), the same additions in the same order as
    ``select_row``.
    """
    P = np.asarray(P, dtype=np.float64)
    nq, nb = P.shape
    order = np.argsort(-P, axis=1, kind="stable")      # ties: lower index
    ps = np.take_along_axis(P, order, axis=1)
    S = np.cumsum(ps, axis=1)
    reached = S >= cdf_threshold
    m_star = np.where(reached.any(axis=1), reached.argmax(axis=1) + 1, nb)
    counts = np.minimum(nb, np.maximum(max(top_k, 0), m_star))
    lists = [np.sort(order[i, :counts[i]]) for i in range(nq)]
    diag = selection_margins(ps, S, m_star, counts, top_k, cdf_threshold)
    return counts.astype(np.int64), lists, diag


def selection_margins(ps, S, m_star, counts, top_k, tau):
    """Relative gaps of every decision the selection takes (R16).

    set_gap: (p_(c) - p_(c+1)) / p_(c), whether the last kept block beats
    the first dropped one; cdf_gap: distance of the cumulative mass from the
    threshold at the decisive prefix lengths, relative to the threshold.
    """
    nq, nb = ps.shape
    idx = np.arange(nq)
    c = counts
    pc = ps[idx, c - 1]
    pn = np.where(c < nb, ps[idx, np.minimum(c, nb - 1)], -np.inf)
    set_gap = np.where(c < nb, (pc - pn) / np.maximum(pc, 1e-300), np.inf)
    tau_s = max(abs(tau), 1e-300)
    cdf_gap = np.full(nq, np.inf)
    k = max(top_k, 0)
    for i in range(nq):
        ms = m_star[i]
        gaps = []
        if ms > k:              # the threshold set the count
            gaps.append(S[i, ms - 1] - tau)
            if ms >= 2:
                gaps.append(tau - S[i, ms - 2])
        elif 1 <= k <= nb:     # top-k set it: the mass at k must reach tau
            gaps.append(S[i, k - 1] - tau if S[i, k - 1] >= tau else np.inf)
        if gaps:
            cdf_gap[i] = min(abs(g) for g in gaps) / tau_s
    return dict(set_gap=set_gap, cdf_gap=cdf_gap, m_star=m_star)


# ---------------------------------------------------------------------------
# Stage 4: block-sparse attention, forward and backward
# ---------------------------------------------------------------------------
def _block_rows(perm, i):
    return np.asarray(perm[BLOCK * i:BLOCK * (i + 1)])


def _kv_rows(perm, sel):
    return np.concatenate([_block_rows(perm, j) for j in sel])


def sparse_attn_fwd(q, k, v, perm, lists, scale: Optional[float] = None,
                    query_blocks: Optional[Sequence[int]] = None):
    """Exact softmax attention of each query block over its selected blocks.

    Reading R14: bidirectional, no dropout, every row of a query block uses
    the block's list, natural-log LSE.  q, k, v: [N, d]; outputs in raster
    token order.  Only ``query_blocks`` are computed if given (the rest of
    ``o``/``lse`` stay NaN).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nb = N // BLOCK
    o = np.full((N, v.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    blocks = range(nb) if query_blocks is None else query_blocks
    for i in blocks:
        rows = _block_rows(perm, i)
        cols = _kv_rows(perm, lists[i])
        s = (q[rows] @ k[cols].T) * scale
        m = s.max(axis=1, keepdims=True)
        l = np.log(np.exp(s - m).sum(axis=1, keepdims=True)) + m
        P = np.exp(s - l)
        o[rows] = P @ v[cols]
        lse[rows] = l[:, 0]
    return o, lse


def sparse_attn_bwd(q, k, v, do, perm, lists, scale: Optional[float] = None,
                    query_blocks: Optional[Sequence[int]] = None):
    """Gradients of the block-sparse attention; the selection is constant.

    Reading R15: top-k / CDF routing is discrete, so no gradient flows into
    it.  D_r = <dO_r, o_r>; P = exp(s - LSE); dV = P^T dO; dP = dO V^T;
    dS = P * (dP - D); dQ = dS K * scale; dK = dS^T Q * scale.
    Returns dq, dk, dv [N, d] (fp64).  With ``query_blocks`` only those query
    blocks contribute (their dQ rows and their share of dK / dV).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    do = np.asarray(do, dtype=np.float64)
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nb = N // BLOCK
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    blocks = range(nb) if query_blocks is None else query_blocks
    for i in blocks:
        rows = _block_rows(perm, i)
        cols = _kv_rows(perm, lists[i])
        s = (q[rows] @ k[cols].T) * scale
        m = s.max(axis=1, keepdims=True)
        l = np.log(np.exp(s - m).sum(axis=1, keepdims=True)) + m
        P = np.exp(s - l)
        o_i = P @ v[cols]
        dO = do[rows]
        D = np.sum(dO * o_i, axis=1, keepdims=True)
        dv[cols] += P.T @ dO
        dP = dO @ v[cols].T
        dS = P * (dP - D)
        dq[rows] = (dS @ k[cols]) * scale
        dk[cols] += (dS.T @ q[rows]) * scale
    return dq, dk, dv


# ---------------------------------------------------------------------------
# Stage 4 variant: pooled stand-in for the unselected blocks (reading R21)
# ---------------------------------------------------------------------------
def dropped_block_terms(q_mean, k_mean, v_mean, lists):
    """Weight and mean value of the blocks each query block left out (R21).

    Sol-Attn abstract (listed on the Prism paper page): instead of
    discarding unselected blocks, their proxy scores are reused to
    approximate what they contribute, inside the same online softmax.  Reading: an unselected KV block j counts, for every
    query row of block i, as its 64 keys all scoring the pooled logit
    z_ij = <qbar_i, kbar_j> / sqrt(d) (stage 2's logit) and all carrying the
    block's mean value vbar_j.

    Returns (drop_lse [nb], drop_v [nb, dv]): drop_lse_i is the natural log
    of sum over unselected j of 64 exp(z_ij) (-inf when block i selected
    every block) and drop_v_i the mean of vbar_j under those weights (zero
    then).
    """
    q_mean = np.asarray(q_mean, dtype=np.float64)
    k_mean = np.asarray(k_mean, dtype=np.float64)
    v_mean = np.asarray(v_mean, dtype=np.float64)
    d = q_mean.shape[1]
    z = (q_mean @ k_mean.T) / math.sqrt(d)
    nq, nb = z.shape
    drop_lse = np.full(nq, -np.inf)
    drop_v = np.zeros((nq, v_mean.shape[1]))
    for i in range(nq):
        out = np.ones(nb, dtype=bool)
        out[np.asarray(lists[i], dtype=np.int64)] = False
        if not out.any():
            continue
        zi = z[i, out] + math.log(BLOCK)        # 64 keys per block
        m = zi.max()
        w = np.exp(zi - m)
        drop_lse[i] = m + math.log(w.sum())
        drop_v[i] = (w / w.sum()) @ v_mean[out]
    return drop_lse, drop_v


def sparse_attn_fwd_corrected(q, k, v, perm, lists,
                              scale: Optional[float] = None,
                              query_blocks: Optional[Sequence[int]] = None):
    """Block-sparse attention plus the pooled stand-in of unselected blocks.

    Reading R21 written out: query row r of block i attends to the selected
    blocks' keys with their exact scores q_r . k_c * scale, and to 64 copies
    of (logit z_ij, value vbar_j) for every block j it did not select, where
    z_ij = <qbar_i, kbar_j> / sqrt(d) and the bars are block means (stage 2).
    One softmax over both sets.  Same layout and ``query_blocks`` behaviour
    as ``sparse_attn_fwd``; with every block selected the two are equal.
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    N, d = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    nb = N // BLOCK
    qm, km, vm = (pool_blocks(x, perm) for x in (q, k, v))
    z = (qm @ km.T) / math.sqrt(d)
    o = np.full((N, v.shape[1]), np.nan)
    lse = np.full(N, np.nan)
    blocks = range(nb) if query_blocks is None else query_blocks
    for i in blocks:
        rows = _block_rows(perm, i)
        sel = np.asarray(lists[i], dtype=np.int64)
        out = np.setdiff1d(np.arange(nb), sel)
        cols = _kv_rows(perm, sel)
        s = (q[rows] @ k[cols].T) * scale
        zd = np.repeat(z[i, out], BLOCK)                # 64 keys per block
        logits = np.concatenate([s, np.broadcast_to(zd, (BLOCK, zd.size))],
                                axis=1)
        vals = np.concatenate([v[cols], np.repeat(vm[out], BLOCK, axis=0)])
        m = logits.max(axis=1, keepdims=True)
        l = np.log(np.exp(logits - m).sum(axis=1, keepdims=True)) + m
        o[rows] = np.exp(logits - l) @ vals
        lse[rows] = l[:, 0]
    return o, lse


# ---------------------------------------------------------------------------
# Whole path for one (batch, head)
# ---------------------------------------------------------------------------
def route_head(q, k, perm, top_k, cdf_threshold):
    """Stages 2-3 for one head: pooled means, proxy, selection."""
    qm = pool_blocks(q, perm)
    km = pool_blocks(k, perm)
    P = proxy_scores(qm, km)
    counts, lists, diag = select_blocks(P, top_k, cdf_threshold)
    return dict(q_mean=qm, k_mean=km, proxy=P, counts=counts, lists=lists,
                diag=diag)


def lists_to_padded(counts, lists, capacity: int) -> np.ndarray:
    """Pack ascending lists into a [nb, capacity] int32 array (-1 padded)."""
    out = np.full((len(lists), capacity), -1, dtype=np.int32)
    for i, sel in enumerate(lists):
        out[i, :len(sel)] = sel
    return out


def padded_to_lists(counts, kv_idx) -> List[np.ndarray]:
    return [np.asarray(kv_idx[i, :counts[i]]) for i in range(len(counts))]
