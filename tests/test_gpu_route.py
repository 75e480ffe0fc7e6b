"""GPU parity of the fused routing call (prism_route_blocks: pooling, proxy
scores and selection without the [B, Hh, Nb, Nb] proxy matrix) against the
oracle and against the unfused calls, at sizes the oracle finishes in
seconds: 1 to 5 blocks (one workgroup row group, ragged), 135 blocks
(several row groups, ragged tail), 1100 and 4500 blocks (two and five
column chunks of 1024); peaked, flat and smooth-field scores; top-k and
threshold corner cases.  Full-size workloads are checked in
test_gpu_fullsize.py."""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_shape_amd as P
from oracle import prism_oracle as po
from synth import iid_normal
from tests.gpu_util import to_dev, widen

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _case(T, H, W, d, seed, scale, dtype="bf16", B=1, Hh=2):
    N = T * H * W
    q = iid_normal((B, Hh, N, d), seed=seed, dtype=dtype, scale=scale)
    k = iid_normal((B, Hh, N, d), seed=seed + 1, dtype=dtype, scale=scale)
    zones = po.zone_tiling(T, H, W)
    sid = [i for i in range(13)
           if all(po.shape_is_legal(po.SHAPES[i], e) for _, e in zones)][0]
    perm = po.block_permutation(T, H, W, zones, [sid] * len(zones))
    return q, k, np.stack([perm] * B)


def _compare(q, k, perm, top_k, tau, fused, unfused):
    counts, kv = (t.cpu().numpy() for t in fused[2:])
    ucounts, ukv = (t.cpu().numpy() for t in unfused)
    B, Hh, nb = counts.shape
    undecided = 0
    for b in range(B):
        for h in range(Hh):
            route = po.route_head(widen(q[b, h]), widen(k[b, h]), perm[b], top_k,
                                  tau)
            dg = route["diag"]
            ok = (dg["set_gap"] > 1e-12) & (dg["cdf_gap"] > 1e-12)
            undecided += int((~ok).sum())
            for i in range(nb):
                c = counts[b, h, i]
                assert 1 <= c <= nb
                if ok[i]:
                    assert c == route["counts"][i], (b, h, i, c, route["counts"][i])
                    assert np.array_equal(kv[b, h, i, :c], route["lists"][i]), (b, h, i)
                    # the unfused path decides the same
                    assert ucounts[b, h, i] == c
                    assert np.array_equal(ukv[b, h, i, :c], kv[b, h, i, :c])
                else:
                    sel = kv[b, h, i, :c]
                    assert np.all(np.diff(sel) > 0)
                    assert abs(int(c) - int(route["counts"][i])) <= 1
    return undecided


@pytest.mark.parametrize("grid,d,scale", [((4, 4, 4), 128, 1.0),
                                          ((4, 4, 20), 64, 2.0),
                                          ((20, 18, 24), 128, 1.0),
                                          ((20, 18, 24), 64, 0.05),
                                          ((20, 44, 80), 128, 0.5),
                                          ((20, 90, 160), 128, 0.3)])
def test_route_fused_matches_oracle(grid, d, scale):
    T, H, W = grid
    Hh = 1 if T * H * W > 100000 else 2
    q, k, perm = _case(T, H, W, d, seed=31 + d, scale=scale, Hh=Hh)
    nb = T * H * W // 64
    cases = [(4, 0.2), (8, 0.2), (0, 0.5), (1, 0.0), (nb + 3, 0.2), (2, 1.0)]
    if nb > 1000:
        cases = cases[:3]
    dq, dk, dperm = to_dev(q), to_dev(k), to_dev(perm)
    for top_k, tau in cases:
        _print("fused routing", grid, d, scale, top_k, tau)
        fused = P.route_blocks(dq, dk, dperm, top_k, tau)
        qm, km, proxy = P.pool_blocks(dq, dk, dperm)
        unfused = P.select_blocks(proxy, top_k, tau)
        torch.cuda.synchronize()
        assert torch.equal(fused[0], qm) and torch.equal(fused[1], km)
        und = _compare(q, k, perm, top_k, tau, fused, unfused)
        _print(f"  rows within rounding of a tie: {und}")


def test_route_fused_capacity_and_fp32():
    T, H, W = 4, 8, 24
    q, k, perm = _case(T, H, W, 64, seed=77, scale=1.5, dtype="fp32", B=2)
    nb = T * H * W // 64
    fused = P.route_blocks(to_dev(q), to_dev(k), to_dev(perm), 2, 0.3,
                           capacity=nb + 9)
    qm, km, proxy = P.pool_blocks(to_dev(q), to_dev(k), to_dev(perm))
    unfused = P.select_blocks(proxy, 2, 0.3)
    torch.cuda.synchronize()
    _compare(q, k, perm, 2, 0.3, fused, unfused)
