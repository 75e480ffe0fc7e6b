"""Seeded synthetic workloads for block-sparse video self-attention.

The pages that describe the method measure on trained video/audio latents
that are not available here, so every input is synthetic.  The shapes follow
WAN-style video latents (tokens on a T x H x W grid, 20 latent frames,
16x spatial compression of 720p / 1080p / 2K frames).

Recipe (one numpy ``PCG64`` stream per tensor, so every tensor is
reproducible on its own):

* config ``i`` owns ``SeedSequence(1000 + i)``; its 8 children feed, in
  order, Q, K, V, video features, a2v residual, upstream gradient dO, the
  Q/K bump parameters, and one spare.  Children are split further per head
  (Q, K, V, dO), per zone (features) or per frame (a2v) so that the host can
  generate in parallel threads; the split is part of the recipe.
* Q/K (smooth configs): per head, ``n_bumps`` Gaussian bumps shared by Q and
  K; bump centre uniform in the grid, isotropic width sigma ~ U[3, 8] tokens,
  bump vector ~ N(0, I_d).  Q = F + 0.5 * noise, K = F + 0.5 * noise'.
  V ~ N(0, 1).
* video features (C = 3072): 0.25 * (16 smooth bumps, sigma ~ U[8, 16],
  vectors N(0, I_C)) plus a per-zone roughness term that is anisotropic along
  a random axis order (smooth, mid, rough): isotropic with probability 1/4
  (i.i.d. N(0, I_C) per token), single-axis with probability 1/4 (amplitudes
  0 / 0 / 1) and graded with probability 1/2 (amplitudes 0 / 0.5 / 1).  The
  roughness along an axis is one N(0, I_C) vector per slice, constant over the
  other two axes of the zone.
* a2v residual: rho_p * eta_p with eta_p ~ N(0, I_C) and
  rho_p = 0.05 + 1.5 * sum of two Gaussian blobs (width U[4, 10] tokens,
  centres uniform): two high-norm "sound source" regions.
* dO ~ N(0, 1).

Every tensor is generated in float32 and rounded once (round-to-nearest-even)
to the configuration's storage type; that one buffer feeds both the GPU path
and the oracle.  bf16 tensors are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field
from typing import Optional

import numpy as np

# --------------------------------------------------------------------------
# workload table
# --------------------------------------------------------------------------
CONFIGS = {
    0: dict(name="tiny_fp32_4x8x8", B=1, Hh=2, d=64, T=4, H=8, W=8,
            dtype="fp32", qk="iid", n_bumps=0, dynamic=False,
            fixed_shape=0, top_k=1, cdf_threshold=0.20, backward=False,
            seed=1000),
    1: dict(name="720p_20x44x80_fwd", B=1, Hh=24, d=128, T=20, H=44, W=80,
            dtype="bf16", qk="bumps", n_bumps=8, dynamic=False,
            fixed_shape=0, top_k=4, cdf_threshold=0.20, backward=False,
            seed=1001),
    2: dict(name="1080p_20x68x120_dyn_fwd", B=1, Hh=24, d=128, T=20, H=68,
            W=120, C=3072, dtype="bf16", qk="bumps", n_bumps=8, dynamic=True,
            fixed_shape=-1, top_k=4, cdf_threshold=0.20, backward=False,
            seed=1002),
    3: dict(name="2k_20x90x160_dyn_fwd", B=1, Hh=24, d=128, T=20, H=90,
            W=160, C=3072, dtype="bf16", qk="bumps", n_bumps=16,
            dynamic=True, fixed_shape=-1, top_k=8, cdf_threshold=0.20,
            backward=False, seed=1003),
    # the training step at the 1080p grid reuses config 2's inputs (same
    # seed) and adds an upstream gradient
    4: dict(name="1080p_20x68x120_dyn_train", B=1, Hh=24, d=128, T=20, H=68,
            W=120, C=3072, dtype="bf16", qk="bumps", n_bumps=8, dynamic=True,
            fixed_shape=-1, top_k=4, cdf_threshold=0.20, backward=True,
            seed=1002),
    # forward + backward on the 2K grid (config 3's inputs plus dO)
    5: dict(name="2k_20x90x160_dyn_train", B=1, Hh=24, d=128, T=20, H=90,
            W=160, C=3072, dtype="bf16", qk="bumps", n_bumps=16,
            dynamic=True, fixed_shape=-1, top_k=8, cdf_threshold=0.20,
            backward=True, seed=1003),
}

ZONE = (8, 8, 8)          # macro-zone extent used by the generator
_CHILD = dict(q=0, k=1, v=2, feat=3, a2v=4, do=5, bumps=6, spare=7)


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


# --------------------------------------------------------------------------
# storage formats
# --------------------------------------------------------------------------
def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); return uint16 bits."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + (np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1)))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """Expand uint16 bfloat16 bit patterns to float32 (exact)."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32)
            << np.uint32(16)).view(np.float32)


def _store(x32: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "fp32":
        return np.ascontiguousarray(x32, dtype=np.float32)
    if dtype == "bf16":
        return f32_to_bf16_bits(x32)
    raise ValueError(dtype)


def _alloc(shape, dtype: str) -> np.ndarray:
    return np.empty(shape, dtype=np.float32 if dtype == "fp32" else np.uint16)


def _rng(ss: np.random.SeedSequence) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(ss))


def iid_normal(shape, seed, dtype: str = "fp32", scale: float = 1.0):
    """i.i.d. N(0, scale^2) tensor from one PCG64 stream, stored as dtype."""
    g = _rng(np.random.SeedSequence(seed))
    x = g.standard_normal(size=shape, dtype=np.float32)
    if scale != 1.0:
        x *= np.float32(scale)
    return _store(x, dtype)


# --------------------------------------------------------------------------
# field helpers
# --------------------------------------------------------------------------
def _gauss_1d(n: int, centre: float, sigma: float) -> np.ndarray:
    x = np.arange(n, dtype=np.float64)
    return np.exp(-((x - centre) ** 2) / (2.0 * sigma * sigma))


def _bump_weights(T, H, W, centres, sigmas) -> np.ndarray:
    """[T*H*W, n] matrix of separable isotropic Gaussian bump weights."""
    n = len(sigmas)
    G = np.empty((T * H * W, n), dtype=np.float32)
    for b in range(n):
        ct, ch, cw = centres[b]
        s = sigmas[b]
        g = (_gauss_1d(T, ct, s)[:, None, None]
             * _gauss_1d(H, ch, s)[None, :, None]
             * _gauss_1d(W, cw, s)[None, None, :])
        G[:, b] = g.reshape(-1)
    return G


def _zones(T, H, W):
    """Zone origins/extents on the generator's 8x8x8 tiling (raster order)."""
    out = []
    for t0 in range(0, T, ZONE[0]):
        for h0 in range(0, H, ZONE[1]):
            for w0 in range(0, W, ZONE[2]):
                out.append(((t0, h0, w0), (min(ZONE[0], T - t0),
                                           min(ZONE[1], H - h0),
                                           min(ZONE[2], W - w0))))
    return out


# --------------------------------------------------------------------------
# per-tensor generators
# --------------------------------------------------------------------------
def _gen_feat(cfg, ss, pool):
    """Video features [B, N, C]: smooth field plus anisotropic per-zone part."""
    B, T, H, W, C = cfg["B"], cfg["T"], cfg["H"], cfg["W"], cfg["C"]
    N = T * H * W
    dtype = cfg["dtype"]
    zones = _zones(T, H, W)
    out = _alloc((B, N, C), dtype)
    per_b = ss.spawn(B)
    for b in range(B):
        kids = per_b[b].spawn(1 + len(zones))
        g = _rng(kids[0])
        nb = 16
        centres = g.uniform(0.0, 1.0, size=(nb, 3)) * np.array([T, H, W])
        sigmas = g.uniform(8.0, 16.0, size=nb)
        U = g.standard_normal(size=(nb, C), dtype=np.float32)
        U *= np.float32(0.25)
        G = _bump_weights(T, H, W, centres, sigmas).reshape(T, H, W, nb)
        view = out[b].reshape(T, H, W, C)

        def one(zi):
            (t0, h0, w0), (lt, lh, lw) = zones[zi]
            zg = _rng(kids[1 + zi])
            order = zg.permutation(3)          # axis roles: smooth, mid, rough
            kind = zg.uniform()
            if kind < 0.25:                    # isotropic roughness
                R = zg.standard_normal(size=(lt, lh, lw, C), dtype=np.float32)
            else:
                amps = (0.0, 0.0, 1.0) if kind < 0.5 else (0.0, 0.5, 1.0)
                ext = (lt, lh, lw)
                R = np.zeros((lt, lh, lw, C), dtype=np.float32)
                for role, axis in enumerate(order):
                    a = amps[role]
                    if a == 0.0:
                        continue
                    sl = zg.standard_normal(size=(ext[axis], C),
                                            dtype=np.float32)
                    shp = [1, 1, 1, C]
                    shp[axis] = ext[axis]
                    R += np.float32(a) * sl.reshape(shp)
            Gz = G[t0:t0 + lt, h0:h0 + lh, w0:w0 + lw].reshape(-1, nb)
            R += (Gz @ U).reshape(lt, lh, lw, C)
            view[t0:t0 + lt, h0:h0 + lh, w0:w0 + lw] = _store(R, dtype)

        list(pool.map(one, range(len(zones))))
    return out


def _gen_a2v(cfg, ss, pool):
    """a2v residual [B, N, C]: Gaussian-blob norm profile times white noise."""
    B, T, H, W, C = cfg["B"], cfg["T"], cfg["H"], cfg["W"], cfg["C"]
    N = T * H * W
    dtype = cfg["dtype"]
    out = _alloc((B, N, C), dtype)
    per_b = ss.spawn(B)
    for b in range(B):
        kids = per_b[b].spawn(1 + T)
        g = _rng(kids[0])
        centres = g.uniform(0.0, 1.0, size=(2, 3)) * np.array([T, H, W])
        widths = g.uniform(4.0, 10.0, size=2)
        rho = 0.05 + 1.5 * _bump_weights(T, H, W, centres, widths).sum(1)
        rho = rho.astype(np.float32).reshape(T, H * W)
        view = out[b].reshape(T, H * W, C)

        def one(t):
            eta = _rng(kids[1 + t]).standard_normal(size=(H * W, C),
                                                    dtype=np.float32)
            eta *= rho[t][:, None]
            view[t] = _store(eta, dtype)

        list(pool.map(one, range(T)))
    return out


# --------------------------------------------------------------------------
# public entry points
# --------------------------------------------------------------------------
@dataclass
class ConfigInputs:
    cfg: dict
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    feat: Optional[np.ndarray] = None
    a2v: Optional[np.ndarray] = None
    do: Optional[np.ndarray] = None
    extra: dict = field(default_factory=dict)


def make_inputs(cfg_id, with_stage1: bool = True, with_grad: bool = None,
                heads: Optional[int] = None) -> ConfigInputs:
    """Build the seeded inputs of a workload.

    ``cfg_id`` is a key of ``CONFIGS`` or a dict with the same fields.
    ``heads`` (optional) keeps only the first ``heads`` heads (same values as
    the full tensor's first heads, since each head has its own stream).
    """
    cfg = dict(CONFIGS[cfg_id]) if not isinstance(cfg_id, dict) else dict(cfg_id)
    if heads is not None:
        cfg["Hh_full"] = cfg["Hh"]
        cfg["Hh"] = heads
    ss = np.random.SeedSequence(cfg["seed"]).spawn(8)
    B, Hh, d = cfg["B"], cfg["Hh"], cfg["d"]
    N = cfg["T"] * cfg["H"] * cfg["W"]
    full_heads = cfg.get("Hh_full", Hh)

    with ThreadPoolExecutor(_workers()) as pool:
        if cfg["qk"] == "iid":
            q = _gen_heads_iid_sub(ss[_CHILD["q"]], B, Hh, full_heads, N, d,
                                   cfg["dtype"], pool)
            k = _gen_heads_iid_sub(ss[_CHILD["k"]], B, Hh, full_heads, N, d,
                                   cfg["dtype"], pool)
        else:
            q, k = _gen_qk_bumps_sub(cfg, ss[_CHILD["q"]], ss[_CHILD["k"]],
                                     ss[_CHILD["bumps"]], full_heads, pool)
        v = _gen_heads_iid_sub(ss[_CHILD["v"]], B, Hh, full_heads, N, d,
                               cfg["dtype"], pool)
        feat = a2v = do = None
        if cfg.get("dynamic") and with_stage1:
            feat = _gen_feat(cfg, ss[_CHILD["feat"]], pool)
            a2v = _gen_a2v(cfg, ss[_CHILD["a2v"]], pool)
        if with_grad is None:
            with_grad = cfg.get("backward", False)
        if with_grad:
            do = _gen_heads_iid_sub(ss[_CHILD["do"]], B, Hh, full_heads, N, d,
                                    cfg["dtype"], pool)
    return ConfigInputs(cfg=cfg, q=q, k=k, v=v, feat=feat, a2v=a2v, do=do)


def make_upstream_grad(cfg_id, heads: Optional[int] = None) -> np.ndarray:
    """dO ~ N(0, 1) for a workload (same stream as ``make_inputs``)."""
    cfg = dict(CONFIGS[cfg_id]) if not isinstance(cfg_id, dict) else dict(cfg_id)
    full = cfg["Hh"]
    Hh = heads if heads is not None else full
    ss = np.random.SeedSequence(cfg["seed"]).spawn(8)
    N = cfg["T"] * cfg["H"] * cfg["W"]
    with ThreadPoolExecutor(_workers()) as pool:
        return _gen_heads_iid_sub(ss[_CHILD["do"]], cfg["B"], Hh, full, N,
                                  cfg["d"], cfg["dtype"], pool)


def _gen_heads_iid_sub(ss, B, Hh, full_heads, N, d, dtype, pool):
    out = _alloc((B, Hh, N, d), dtype)
    kids = ss.spawn(B * full_heads)

    def one(i):
        b, h = divmod(i, Hh)
        x = _rng(kids[b * full_heads + h]).standard_normal(size=(N, d),
                                                           dtype=np.float32)
        out[b, h] = _store(x, dtype)

    list(pool.map(one, range(B * Hh)))
    return out


def _gen_qk_bumps_sub(cfg, ss_q, ss_k, ss_bumps, full_heads, pool):
    B, Hh, d = cfg["B"], cfg["Hh"], cfg["d"]
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    N = T * H * W
    nb = cfg["n_bumps"]
    dtype = cfg["dtype"]
    q = _alloc((B, Hh, N, d), dtype)
    k = _alloc((B, Hh, N, d), dtype)
    kq = ss_q.spawn(B * full_heads)
    kk = ss_k.spawn(B * full_heads)
    kb = ss_bumps.spawn(B * full_heads)

    def one(i):
        b, h = divmod(i, Hh)
        j = b * full_heads + h
        g = _rng(kb[j])
        centres = g.uniform(0.0, 1.0, size=(nb, 3)) * np.array([T, H, W])
        sigmas = g.uniform(3.0, 8.0, size=nb)
        U = g.standard_normal(size=(nb, d), dtype=np.float32)
        F = _bump_weights(T, H, W, centres, sigmas) @ U
        nq = _rng(kq[j]).standard_normal(size=(N, d), dtype=np.float32)
        nq *= np.float32(0.5)
        nq += F
        q[b, h] = _store(nq, dtype)
        nk = _rng(kk[j]).standard_normal(size=(N, d), dtype=np.float32)
        nk *= np.float32(0.5)
        nk += F
        k[b, h] = _store(nk, dtype)

    list(pool.map(one, range(B * Hh)))
    return q, k


# --------------------------------------------------------------------------
# a2v bridge inputs (the producer of the audio residual)
# --------------------------------------------------------------------------
AUDIO_STEPS_PER_S = 44100.0 / 2048.0   # audio tokens per second (~21.5)
VIDEO_FPS = 16.0                       # frames per second of the decoded video
VAE_T_STRIDE = 4                       # video frames per latent frame


def audio_tokens_for(T: int) -> int:
    """Audio tokens covering the clip of T latent frames: (T-1)*4+1 video
    frames at VIDEO_FPS, AUDIO_STEPS_PER_S audio tokens per second."""
    seconds = (VAE_T_STRIDE * (T - 1) + 1) / VIDEO_FPS
    return int(np.ceil(seconds * AUDIO_STEPS_PER_S))


@dataclass
class BridgeInputs:
    x_a: np.ndarray        # [B, Na, Ca] audio hidden states (bf16 bits)
    w_q: np.ndarray        # [D, Cv]  weights as [out, in] (bf16 bits)
    w_k: np.ndarray        # [D, Ca]
    w_v: np.ndarray        # [D, Ca]
    w_o: np.ndarray        # [Cv, D]
    pos_v: np.ndarray      # [B, N] fp32 time positions in audio steps
    pos_a: np.ndarray      # [B, Na] fp32
    heads: int


def make_bridge_inputs(T: int, H: int, W: int, B: int = 1, Cv: int = 3072,
                       Ca: int = 1536, heads: int = 24, Na: Optional[int] = None,
                       seed: int = 2000) -> BridgeInputs:
    """Random-weight inputs of the a2v bridge for a T x H x W video grid.

    Audio hidden states ~ N(0, 1); each weight ~ N(0, 1 / fan_in) (so
    projections keep unit scale); all stored as bf16.  Time positions on
    the audio-step axis: a video token of latent frame t sits at the time of
    video frame 4t, i.e. 4 t / VIDEO_FPS seconds; audio token j at j.  The
    pages fix the audio rate (44100 / 2048) and the 4x temporal stride, not
    the video frame rate (16 fps here).  Seed children, in order: audio
    states, Wq, Wk, Wv, Wo.
    """
    if Na is None:
        Na = audio_tokens_for(T)
    D = 128 * heads
    kids = np.random.SeedSequence(seed).spawn(5)

    def normal(i, shape, std):
        x = _rng(kids[i]).standard_normal(size=shape, dtype=np.float32)
        x *= np.float32(std)
        return f32_to_bf16_bits(x)

    x_a = normal(0, (B, Na, Ca), 1.0)
    w_q = normal(1, (D, Cv), 1.0 / np.sqrt(Cv))
    w_k = normal(2, (D, Ca), 1.0 / np.sqrt(Ca))
    w_v = normal(3, (D, Ca), 1.0 / np.sqrt(Ca))
    w_o = normal(4, (Cv, D), 1.0 / np.sqrt(D))
    t = np.repeat(np.arange(T, dtype=np.float64), H * W)
    pv = (VAE_T_STRIDE * t / VIDEO_FPS * AUDIO_STEPS_PER_S).astype(np.float32)
    pos_v = np.tile(pv, (B, 1))
    pos_a = np.tile(np.arange(Na, dtype=np.float32), (B, 1))
    return BridgeInputs(x_a=x_a, w_q=w_q, w_k=w_k, w_v=w_v, w_o=w_o,
                        pos_v=pos_v, pos_a=pos_a, heads=heads)
