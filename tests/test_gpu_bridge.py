"""GPU parity of the a2v bridge residual (prism_a2v_bridge) against the fp64
oracle (oracle/bridge_oracle.py), and of stage 1 fed with it.

* small widths with ragged sizes (token tiles of 256, a partial 64-key tile),
  with and without the rotary alignment, every row;
* the pages' widths (video 3072, audio 1536, 24 heads of 128) on a small
  grid, every row;
* the 2K grid, sampled rows;
* stage 1 on the bridge's own residual: zone shapes and permutation equal
  the oracle's (oracle residual, oracle stage 1) wherever the decision's
  margin exceeds the difference of the two zone statistics.
"""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_shape_amd as P
from oracle import bridge_oracle as bo
from oracle import prism_oracle as po
from synth import CONFIGS, make_bridge_inputs, make_inputs
from tests.gpu_util import assert_close, err_stats, to_dev, widen

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _gpu_bridge(x_v, br, rotary=True):
    args = [to_dev(a) for a in (x_v, br.x_a, br.w_q, br.w_k, br.w_v, br.w_o)]
    pv = to_dev(br.pos_v) if rotary else None
    pa = to_dev(br.pos_a) if rotary else None
    dh = P.a2v_bridge(*args, heads=br.heads, pos_v=pv, pos_a=pa)
    torch.cuda.synchronize()
    return dh


def _oracle(x_v, br, b, rotary=True, rows=None):
    return bo.a2v_residual(widen(x_v[b]), widen(br.x_a[b]), widen(br.w_q),
                           widen(br.w_k), widen(br.w_v), widen(br.w_o),
                           br.heads,
                           pos_v=br.pos_v[b] if rotary else None,
                           pos_a=br.pos_a[b] if rotary else None, rows=rows)


def _feat(cfg):
    return make_inputs(cfg).feat


@pytest.mark.parametrize("rotary", [True, False])
def test_bridge_small_ragged(rotary):
    cfg = dict(CONFIGS[2])
    cfg.update(T=20, H=18, W=24, C=512, B=2, Hh=1, name="bridge_small")
    x_v = _feat(cfg)                          # [2, 8640, 512]: 33.75 tiles
    br = make_bridge_inputs(20, 18, 24, B=2, Cv=512, Ca=256, heads=4, Na=70,
                            seed=2100)
    _print("bridge small", x_v.shape, br.x_a.shape, "rotary", rotary)
    dh = _gpu_bridge(x_v, br, rotary).float().cpu().numpy()
    for b in range(2):
        ref = _oracle(x_v, br, b, rotary)
        r = assert_close(dh[b], ref, True, f"dh[{b}]")
        _print(f"  batch {b}: rel L2 {r[0]:.2e}, max-abs {r[1]:.2e}, "
               f"|ref| max {np.abs(ref).max():.2f}")


def test_bridge_model_widths():
    cfg = dict(CONFIGS[2])
    cfg.update(T=4, H=16, W=16, C=3072, B=1, Hh=1, name="bridge_wide")
    x_v = _feat(cfg)
    br = make_bridge_inputs(4, 16, 16, Cv=3072, Ca=1536, heads=24, seed=2200)
    _print("bridge widths", x_v.shape, br.x_a.shape)
    dh = _gpu_bridge(x_v, br).float().cpu().numpy()
    ref = _oracle(x_v, br, 0)
    r = assert_close(dh[0], ref, True, "dh")
    _print(f"  rel L2 {r[0]:.2e}, max-abs {r[1]:.2e}")


def test_bridge_2k_sampled_rows():
    x = make_inputs(3, with_grad=False)
    cfg = x.cfg
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    br = make_bridge_inputs(T, H, W, Cv=cfg["C"], Ca=1536, heads=24, seed=2300)
    _print("bridge 2K", x.feat.shape, br.x_a.shape)
    dh = _gpu_bridge(x.feat, br)
    rng = np.random.default_rng(5)
    rows = np.sort(rng.choice(T * H * W, size=384, replace=False))
    got = dh[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    ref = _oracle(x.feat, br, 0, rows=rows)
    r = assert_close(got, ref, True, "dh rows")
    _print(f"  rel L2 {r[0]:.2e}, max-abs {r[1]:.2e}")


def test_zone_shapes_on_the_bridge_residual():
    """Stage 1 reading the bridge's residual: the GPU path (bridge, then
    zone shapes) against the oracle path (oracle residual, oracle stage 1).
    The two residuals differ by bf16 rounding, so a zone's decision is
    demanded equal where its relative margin exceeds 20x the relative
    difference of its statistics w_a = v_a + u_a."""
    cfg = dict(CONFIGS[2])
    cfg.update(T=20, H=18, W=24, C=3072, B=1, Hh=1, name="bridge_stage1")
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    feat = make_inputs(cfg).feat
    br = make_bridge_inputs(T, H, W, Cv=3072, Ca=1536, heads=24, seed=2400)
    _print("stage 1 on the bridge residual", feat.shape)
    dh = _gpu_bridge(feat, br)
    ref_dh = _oracle(feat, br, 0)
    base = po.zone_shapes(widen(feat[0]), ref_dh, T, H, W)
    v_sum, u_sum = base["stats"][:, :3].sum(), base["stats"][:, 3:].sum()
    # lambda 1 (the pages' setting, where this random-weight residual is a
    # small share of w) and a power of two that makes the audio term about
    # half of w, so the residual's norm field decides shapes
    for lam in (1.0, float(2.0 ** np.round(np.log2(v_sum / u_sum)))):
        zs, perm, _, stats = P.zone_shapes(to_dev(feat), dh, T, H, W, lam=lam)
        torch.cuda.synchronize()
        ref = po.zone_shapes(widen(feat[0]), ref_dh, T, H, W, lam=lam)
        gs = stats[0].cpu().numpy()
        w_g = gs[:, :3] + lam * gs[:, 3:]
        w_r = ref["stats"][:, :3] + lam * ref["stats"][:, 3:]
        delta = np.max(np.abs(w_g - w_r) / np.maximum(np.abs(w_r), 1e-300),
                       axis=1)
        ok = ref["margin"] > 20.0 * delta + po.REL_MARGIN_FLAG
        share = lam * u_sum / w_r.sum()
        _print(f"  lambda {lam:g}: audio share of w {share:.3f}, zones "
               f"{len(ok)}, compared {int(ok.sum())}, max stat diff "
               f"{delta.max():.1e}, shapes {np.bincount(ref['zone_shape'], minlength=13).tolist()}")
        assert ok.mean() >= 0.9
        assert np.array_equal(zs[0].cpu().numpy()[ok], ref["zone_shape"][ok])
        if ok.all():
            assert np.array_equal(perm[0].cpu().numpy(), ref["perm"])
        assert len(set(ref["zone_shape"].tolist())) >= 3
