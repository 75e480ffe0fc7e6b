"""Pins for the oracle's stage 1: zone statistics, shape choice, permutation.

Checks against closed forms (linear ramps, alternating fields), the
hand-derived fixtures in tests/golden/, symmetry, and brute-force geometry.
"""
import math
import os

import numpy as np
import pytest

from oracle import prism_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _ramp(ext, axis, slope=1.0, C=1):
    idx = np.indices(ext, dtype=np.float64)[axis] * slope
    return np.repeat(idx[..., None], C, axis=-1)


@pytest.mark.parametrize("ext", [(8, 8, 8), (4, 8, 8), (8, 2, 8), (4, 2, 8)])
@pytest.mark.parametrize("axis", [0, 1, 2])
def test_directional_variance_linear_ramp(ext, axis):
    # a line of L equally spaced values with step g has population variance
    # g^2 (L^2 - 1) / 12; the other two axes see constant lines
    g = 0.75
    v = po.directional_variance(_ramp(ext, axis, g, C=3))
    L = ext[axis]
    expect = np.zeros(3)
    expect[axis] = g * g * (L * L - 1) / 12.0
    np.testing.assert_allclose(v, expect, rtol=1e-13, atol=1e-14)


def test_directional_variance_alternating_and_channel_mean():
    ext = (8, 8, 8)
    w = np.indices(ext)[2]
    alt = np.where(w % 2 == 0, 1.0, -1.0)          # +-1 along W: variance 1
    ramp_t = np.indices(ext)[0].astype(float)       # variance 5.25 along T
    x = np.stack([alt, ramp_t], axis=-1)            # two channels
    v = po.directional_variance(x)
    # channel mean: W sees (1 + 0)/2, T sees (0 + 5.25)/2, H sees 0
    np.testing.assert_allclose(v, [5.25 / 2, 0.0, 0.5], atol=1e-14)


def test_token_rms_norm_closed_form():
    C = 3072
    rng = np.random.default_rng(0)
    signs = rng.choice([-1.0, 1.0], size=(5, C))
    s = np.array([0.5, 1.0, 2.0, 3.0, 0.0])
    np.testing.assert_allclose(po.token_rms_norm(signs * s[:, None]), s,
                               rtol=1e-14)


def test_audio_term_along_h_only():
    # residual norm profile varies along H only -> u = (0, var_H, 0)
    ext = (8, 8, 8)
    C = 16
    h = np.indices(ext)[1].astype(float)
    rng = np.random.default_rng(1)
    signs = rng.choice([-1.0, 1.0], size=ext + (C,))
    a2v = signs * (0.1 + 0.2 * h)[..., None]
    feat = np.zeros(ext + (C,))
    st = po.zone_statistics(feat, a2v)
    np.testing.assert_allclose(st[:3], 0.0, atol=1e-30)
    np.testing.assert_allclose(st[3:], [0.0, 0.04 * 63 / 12, 0.0],
                               rtol=1e-12, atol=1e-15)
    # with only the audio term, the finest H partition (8,1,8) wins
    sid, margin = po.choose_shape(st, ext)
    assert po.SHAPES[sid] == (8, 1, 8) and margin > 0
    # the audio term is what decides: with lambda = 0 every cost is 0 -> id 0
    assert po.choose_shape(st, ext, lam=0.0)[0] == 0


def _read_shape_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "shape_choice.txt")):
        if line.startswith("#") or not line.strip():
            continue
        ext, w, sid = line.split("|")
        rows.append((tuple(int(x) for x in ext.split()),
                     [float(x) for x in w.split()], int(sid)))
    return rows


@pytest.mark.parametrize("ext,w,sid", _read_shape_golden())
def test_shape_choice_golden(ext, w, sid):
    got, _ = po.choose_shape(np.array(w + [0.0, 0.0, 0.0]), ext)
    assert got == sid, (ext, w, got, po.SHAPES[got])


def test_named_shapes_from_their_triggers():
    # The three shapes the pages name, reached from the triggers they name:
    # fast motion (variation along T) -> (2,4,8); mouth/face detail (variation
    # along H) -> (8,2,4); no directional preference -> (4,4,4).
    ext = (8, 8, 8)
    cases = {(2, 4, 8): (10.0, 2.0, 1.0), (8, 2, 4): (1.0, 10.0, 2.0),
             (4, 4, 4): (1.0, 1.0, 1.0)}
    for shape, w in cases.items():
        sid, _ = po.choose_shape(np.array(list(w) + [0, 0, 0]), ext)
        assert po.SHAPES[sid] == shape


def test_shape_choice_axis_symmetry():
    # permuting the axes of a cubic zone's statistics permutes the chosen
    # shape (when the choice is not a tie)
    rng = np.random.default_rng(5)
    ext = (8, 8, 8)
    for _ in range(200):
        w = rng.exponential(size=3)
        sid, margin = po.choose_shape(np.concatenate([w, np.zeros(3)]), ext)
        if margin < 1e-9:
            continue
        for perm in [(1, 0, 2), (2, 1, 0), (0, 2, 1), (1, 2, 0)]:
            wp = w[list(perm)]
            sp, _ = po.choose_shape(np.concatenate([wp, np.zeros(3)]), ext)
            want = tuple(po.SHAPES[sid][a] for a in perm)
            assert po.SHAPES[sp] == want


def test_shape_table_properties():
    assert len(po.SHAPES) == 13
    assert len(set(po.SHAPES)) == 13
    for s in po.SHAPES:
        assert s[0] * s[1] * s[2] == 64
        assert max(s) <= 8 * min(s)
        assert all(e & (e - 1) == 0 for e in s)
    # the three shapes named on the pages are present
    for named in [(4, 4, 4), (8, 2, 4), (2, 4, 8)]:
        assert named in po.SHAPES
    legal_8 = [i for i, s in enumerate(po.SHAPES) if po.shape_is_legal(s, (8, 8, 8))]
    assert legal_8 == list(range(10))


def test_ramp_zone_end_to_end():
    # feature field that changes only along T -> finest T partition (1,8,8)
    T, H, W, C = 8, 8, 16, 4
    feat = _ramp((T, H, W), 0, 1.0, C).reshape(-1, C)
    out = po.zone_shapes(feat, None, T, H, W)
    assert [po.SHAPES[s] for s in out["zone_shape"]] == [(1, 8, 8)] * 2
    # same along W -> (8,8,1)
    feat = _ramp((T, H, W), 2, 1.0, C).reshape(-1, C)
    out = po.zone_shapes(feat, None, T, H, W)
    assert [po.SHAPES[s] for s in out["zone_shape"]] == [(8, 8, 1)] * 2


def test_zone_tiling_counts_and_remainders():
    z = po.zone_tiling(20, 90, 160)
    assert len(z) == 3 * 12 * 20
    kinds = {}
    for _, e in z:
        kinds[e] = kinds.get(e, 0) + 1
    assert kinds == {(8, 8, 8): 440, (4, 8, 8): 220, (8, 2, 8): 40,
                     (4, 2, 8): 20}
    assert sum(e[0] * e[1] * e[2] for _, e in z) == 20 * 90 * 160


def _read_perm_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "perm_small_grid.txt")):
        if line.startswith("#") or not line.strip():
            continue
        head, pairs = line.split("|")
        sid = int(head.split()[0])
        kv = [tuple(int(x) for x in p.split(":")) for p in pairs.split()]
        rows.append((sid, kv))
    return rows


@pytest.mark.parametrize("sid,pairs", _read_perm_golden())
def test_permutation_golden(sid, pairs):
    out = po.zone_shapes(None, None, 4, 8, 8, fixed_shape=sid)
    perm = out["perm"]
    for slot, tok in pairs:
        assert perm[slot] == tok, (slot, perm[slot], tok)


def _check_blocks_are_boxes(T, H, W, zones, ids, perm):
    # every block is an axis-aligned box of its zone's shape inside the zone;
    # blocks are numbered zone-major; the permutation is a bijection
    assert np.array_equal(np.sort(perm), np.arange(T * H * W))
    t, h, w = perm // (H * W), (perm // W) % H, perm % W
    slot = 0
    for ((t0, h0, w0), (Lt, Lh, Lw)), sid in zip(zones, ids):
        et, eh, ew = po.SHAPES[sid]
        nblk = (Lt * Lh * Lw) // 64
        for b in range(nblk):
            s = slice(slot, slot + 64)
            for coord, o, L, e in ((t, t0, Lt, et), (h, h0, Lh, eh),
                                   (w, w0, Lw, ew)):
                c = coord[s]
                assert c.min() >= o and c.max() < o + L
                assert c.max() - c.min() + 1 == e
                assert (c.min() - o) % e == 0
            # raster order inside the block
            assert np.all(np.diff(perm[s]) > 0)
            slot += 64


def test_permutation_structure_dynamic_shapes():
    T, H, W = 20, 18, 24
    zones = po.zone_tiling(T, H, W)
    rng = np.random.default_rng(3)
    ids = []
    for _, e in zones:
        legal = [i for i, s in enumerate(po.SHAPES) if po.shape_is_legal(s, e)]
        ids.append(int(rng.choice(legal)))
    perm = po.block_permutation(T, H, W, zones, ids)
    _check_blocks_are_boxes(T, H, W, zones, ids, perm)


def test_fixed_shape_rejects_illegal_zone():
    with pytest.raises(ValueError):
        po.zone_shapes(None, None, 4, 8, 8, fixed_shape=5)  # (8,2,4) vs T=4


def test_synthetic_dynamic_config_uses_many_shapes_and_audio_matters():
    # a cut-down grid of the dynamic workloads: the generator's anisotropic
    # zones must spread over several shapes, and the audio term must change
    # some choices
    from synth import CONFIGS, make_inputs, bf16_bits_to_f32
    cfg = dict(CONFIGS[2])
    cfg.update(T=16, H=32, W=40, Hh=1)
    x = make_inputs(cfg)
    feat = bf16_bits_to_f32(x.feat[0]).astype(np.float64)
    a2v = bf16_bits_to_f32(x.a2v[0]).astype(np.float64)
    out = po.zone_shapes(feat, a2v, cfg["T"], cfg["H"], cfg["W"])
    assert len(set(out["zone_shape"].tolist())) >= 5
    out0 = po.zone_shapes(feat, a2v, cfg["T"], cfg["H"], cfg["W"], lam=0.0)
    assert np.any(out0["zone_shape"] != out["zone_shape"])
    _check_blocks_are_boxes(cfg["T"], cfg["H"], cfg["W"], out["zones"],
                            out["zone_shape"], out["perm"])
