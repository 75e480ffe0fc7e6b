"""Plain fp64 CPU oracle of the audio-to-video (a2v) bridge residual.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import this module; the library's compute
path never does.  It shares no code with the HIP kernels.

Source: the Prism architecture walk-through (wmrh.cn), sections
"a2v / v2a 条件桥" and "一个巧妙的联动：桥接残差反哺稀疏注意力".  Each
interaction layer holds a conditional cross-attention block in the
audio-to-video direction: the queries are the video tokens' 3072-wide hidden
states, the keys and values come from the audio tokens' 1536-wide hidden
states, and the output is added to the video tower as a residual (scaled by
a2v_scale).  The *unscaled* residual is handed to the video block, whose
sparse attention reads its per-token L2 norm (stage 1 of the sparse path).
Both bridge directions support a cross-modal rotary alignment that puts
video frames and audio steps on one time axis.

Readings (the pages give no formula; the plainest one is taken):
  R22  the block is multi-head scaled dot-product cross-attention with
       linear query / key / value / output projections and no bias or
       normalisation: q = x_v Wq^T, k = x_a Wk^T, v = x_a Wv^T (each 3072
       wide, heads of head_dim columns), o_h = softmax(q_h k_h^T /
       sqrt(head_dim)) v_h, dh = concat_h(o_h) Wo^T.  Weights are stored as
       [out, in] like a linear layer's.
  R23  the rotary alignment is optional: given a time position per video
       token and per audio token (on the audio-step axis), q and k of every
       head are rotated pairwise, (2i, 2i+1) by angle pos * base^(-2i /
       head_dim) with base 10000, before the scores; positions absent means
       no rotation.
Every float is fp64; inputs are the exact buffers the GPU receives, widened.

Parity pins (tests/test_oracle_bridge.py): torch's multi-head attention
(fp64, CPU) as a library special case; closed forms with one audio token,
uniform scores and a hand-computed two-token softmax; rotary pins (zero
positions, a common shift of all positions, a hand-computed rotation).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def rotate_pairs(x: np.ndarray, pos: np.ndarray, base: float = 10000.0):
    """Rotary rotation of the last axis (head_dim, even) in pairs
    (2i, 2i+1) by angle pos * base^(-2i / head_dim)  (reading R23).

    x: [n, heads, head_dim]; pos: [n]."""
    x = np.asarray(x, dtype=np.float64)
    n, hh, dh = x.shape
    i = np.arange(dh // 2, dtype=np.float64)
    inv = base ** (-2.0 * i / dh)                       # [dh/2]
    ang = np.asarray(pos, dtype=np.float64)[:, None] * inv[None, :]
    c, s = np.cos(ang)[:, None, :], np.sin(ang)[:, None, :]
    xe, xo = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2] = xe * c - xo * s
    out[..., 1::2] = xe * s + xo * c
    return out


def a2v_residual(x_v, x_a, w_q, w_k, w_v, w_o, heads: int,
                 pos_v: Optional[np.ndarray] = None,
                 pos_a: Optional[np.ndarray] = None,
                 rope_base: float = 10000.0,
                 rows: Optional[np.ndarray] = None):
    """Unscaled a2v bridge residual for one batch element (reading R22).

    x_v: [N, Cv] video hidden states; x_a: [Na, Ca] audio hidden states;
    w_q [D, Cv], w_k [D, Ca], w_v [D, Ca], w_o [Cv, D] as [out, in];
    D = heads * head_dim.  pos_v [N] / pos_a [Na]: optional rotary time
    positions (reading R23, both or neither).  ``rows`` restricts the
    computation to those video tokens (the output then has len(rows) rows).
    Returns dh [N or len(rows), Cv].
    """
    x_v = np.asarray(x_v, dtype=np.float64)
    x_a = np.asarray(x_a, dtype=np.float64)
    w_q, w_k, w_v, w_o = (np.asarray(w, dtype=np.float64)
                          for w in (w_q, w_k, w_v, w_o))
    if rows is not None:
        x_v = x_v[rows]
        if pos_v is not None:
            pos_v = np.asarray(pos_v)[rows]
    D = w_q.shape[0]
    dh = D // heads
    n, na = x_v.shape[0], x_a.shape[0]
    q = (x_v @ w_q.T).reshape(n, heads, dh)
    k = (x_a @ w_k.T).reshape(na, heads, dh)
    v = (x_a @ w_v.T).reshape(na, heads, dh)
    if (pos_v is None) != (pos_a is None):
        raise ValueError("give both rotary position arrays or neither")
    if pos_v is not None:
        q = rotate_pairs(q, pos_v, rope_base)
        k = rotate_pairs(k, pos_a, rope_base)
    s = np.einsum("nhd,mhd->hnm", q, k) / math.sqrt(dh)
    s = s - s.max(axis=2, keepdims=True)
    p = np.exp(s)
    p /= p.sum(axis=2, keepdims=True)
    o = np.einsum("hnm,mhd->nhd", p, v).reshape(n, D)
    return o @ w_o.T
