"""GPU parity of every stage against the fp64 oracle, at sizes the oracle
finishes in seconds (several tiles, ragged tails, remainder zones).

Integer outputs (zone shapes, perm, counts, index lists) must match bit for
bit; float outputs within the stated tolerances.  All calls go through the
C ABI (the ctypes binding).
"""
import math

import numpy as np
import pytest
import torch

import dynamic_block_sparse_shape_amd as P
from oracle import prism_oracle as po
from synth import CONFIGS, iid_normal, make_inputs
from tests.gpu_util import assert_close, err_stats, to_dev, to_host, widen

pytestmark = pytest.mark.gpu

SMALL_DYN = dict(CONFIGS[2])
SMALL_DYN.update(T=20, H=18, W=24, C=512, Hh=2, name="small_dyn")


def _print(*a):
    print(*a, flush=True)


# ------------------------------------------------------------------ stage 1
@pytest.mark.parametrize("grid,sid", [((4, 8, 8), 0), ((4, 8, 8), 1),
                                      ((20, 44, 80), 0), ((20, 18, 24), 3),
                                      ((8, 16, 24), 7)])
def test_stage1_fixed_shape(grid, sid):
    T, H, W = grid
    _print("stage1 fixed", grid, sid)
    zs, perm, inv, _ = P.zone_shapes(None, None, T, H, W, fixed_shape=sid, B=2)
    torch.cuda.synchronize()
    ref = po.zone_shapes(None, None, T, H, W, fixed_shape=sid)
    for b in range(2):
        assert np.array_equal(perm[b].cpu().numpy(), ref["perm"])
        assert np.all(zs[b].cpu().numpy() == sid)
        inv_ref = np.empty_like(ref["perm"])
        inv_ref[ref["perm"]] = np.arange(T * H * W)
        assert np.array_equal(inv[b].cpu().numpy(), inv_ref)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_stage1_dynamic(dtype):
    cfg = dict(SMALL_DYN)
    cfg["dtype"] = dtype
    x = make_inputs(cfg)
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    _print("stage1 dynamic", dtype, (T, H, W), cfg["C"])
    zs, perm, inv, stats = P.zone_shapes(to_dev(x.feat), to_dev(x.a2v), T, H, W)
    torch.cuda.synchronize()
    ref = po.zone_shapes(widen(x.feat[0]), widen(x.a2v[0]), T, H, W)
    # every decision is clear of rounding
    assert ref["margin"].min() > po.REL_MARGIN_FLAG
    assert np.array_equal(zs[0].cpu().numpy(), ref["zone_shape"])
    assert np.array_equal(perm[0].cpu().numpy(), ref["perm"])
    inv_ref = np.empty_like(ref["perm"])
    inv_ref[ref["perm"]] = np.arange(T * H * W)
    assert np.array_equal(inv[0].cpu().numpy(), inv_ref)
    np.testing.assert_allclose(stats[0].cpu().numpy(), ref["stats"], rtol=1e-11,
                               atol=1e-14)
    assert len(set(ref["zone_shape"].tolist())) >= 4


@pytest.mark.parametrize("grid", [(16, 12, 30), (16, 11, 32)])
def test_stage1_dynamic_odd_remainders(grid):
    """bf16 zone statistics on zones whose remainder extent is 6 (W = 30)
    or 3 (H = 11): line lengths whose reciprocal is not a power of two."""
    cfg = dict(SMALL_DYN)
    T, H, W = grid
    cfg.update(T=T, H=H, W=W, C=256, name="odd_remainders")
    x = make_inputs(cfg)
    _print("stage1 odd remainders", grid)
    zs, perm, _, stats = P.zone_shapes(to_dev(x.feat), to_dev(x.a2v), T, H, W)
    torch.cuda.synchronize()
    ref = po.zone_shapes(widen(x.feat[0]), widen(x.a2v[0]), T, H, W)
    assert sorted(set(e for _, ext in ref["zones"] for e in ext)) != [8]
    np.testing.assert_allclose(stats[0].cpu().numpy(), ref["stats"], rtol=1e-11,
                               atol=1e-14)
    ok = ref["margin"] > po.REL_MARGIN_FLAG
    assert ok.all(), ref["margin"].min()
    assert np.array_equal(zs[0].cpu().numpy(), ref["zone_shape"])
    assert np.array_equal(perm[0].cpu().numpy(), ref["perm"])


def test_stage1_without_audio_and_lambda():
    cfg = dict(SMALL_DYN)
    x = make_inputs(cfg)
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    feat = to_dev(x.feat)
    zs0, perm0, _, st0 = P.zone_shapes(feat, None, T, H, W)
    zs2, perm2, _, _ = P.zone_shapes(feat, to_dev(x.a2v), T, H, W, lam=4.0)
    torch.cuda.synchronize()
    r0 = po.zone_shapes(widen(x.feat[0]), None, T, H, W)
    r2 = po.zone_shapes(widen(x.feat[0]), widen(x.a2v[0]), T, H, W, lam=4.0)
    for got, ref in ((zs0, r0), (zs2, r2)):
        ok = ref["margin"] > po.REL_MARGIN_FLAG
        assert np.array_equal(got[0].cpu().numpy()[ok], ref["zone_shape"][ok])
    assert np.all(st0[0, :, 3:].cpu().numpy() == 0.0)


# ------------------------------------------------------------------ stage 2
def _two_perms(T, H, W, seed=5):
    """Batch 0: one shape everywhere; batch 1: a random legal shape per zone
    (remainder zones included)."""
    zones = po.zone_tiling(T, H, W)
    fixed = [i for i in range(13)
             if all(po.shape_is_legal(po.SHAPES[i], e) for _, e in zones)][0]
    rng = np.random.default_rng(seed)
    ids = [int(rng.choice([i for i in range(13)
                           if po.shape_is_legal(po.SHAPES[i], e)]))
           for _, e in zones]
    return np.stack([po.block_permutation(T, H, W, zones, [fixed] * len(zones)),
                     po.block_permutation(T, H, W, zones, ids)])


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64),
                                     ("fp32", 64), ("fp32", 128)])
def test_stage2_pool_and_proxy(dtype, d):
    T, H, W = 20, 18, 24              # Nb = 135: two full tiles + ragged 7
    N = T * H * W
    B, Hh = 2, 2
    q = iid_normal((B, Hh, N, d), seed=11, dtype=dtype, scale=2.0)
    k = iid_normal((B, Hh, N, d), seed=12, dtype=dtype, scale=2.0)
    perm = _two_perms(T, H, W)
    _print("stage2", dtype, d)
    qm, km, proxy = P.pool_blocks(to_dev(q), to_dev(k), to_dev(perm))
    torch.cuda.synchronize()
    qm, km, proxy = qm.cpu().numpy(), km.cpu().numpy(), proxy.cpu().numpy()
    for b in range(B):
        for h in range(Hh):
            rq = po.pool_blocks(widen(q[b, h]), perm[b])
            rk = po.pool_blocks(widen(k[b, h]), perm[b])
            if dtype == "bf16":       # a sum of 64 bf16 values is exact in fp64
                assert np.array_equal(qm[b, h], rq) and np.array_equal(km[b, h], rk)
            else:
                np.testing.assert_allclose(qm[b, h], rq, rtol=1e-15, atol=1e-16)
            rp = po.proxy_scores(rq, rk)
            np.testing.assert_allclose(proxy[b, h], rp, rtol=1e-12, atol=1e-300)
            np.testing.assert_allclose(proxy[b, h].sum(1), 1.0, rtol=1e-13)


# ------------------------------------------------------------------ stage 3
def _special_rows(nb, rng):
    rows = []
    z = rng.normal(scale=3.0, size=nb)
    p = np.exp(z - z.max())
    rows.append(p / p.sum())                          # peaked
    rows.append(np.full(nb, 1.0 / nb))                # exactly flat (ties)
    w = rng.integers(0, 4, size=nb).astype(float)     # many exact ties
    w[0] += 1
    rows.append(w / w.sum())
    z = rng.normal(scale=0.05, size=nb)               # nearly flat
    p = np.exp(z)
    rows.append(p / p.sum())
    r = np.zeros(nb)
    r[nb // 2] = 1.0                                  # one-hot
    rows.append(r)
    return rows


@pytest.mark.parametrize("nb", [5, 135, 1100, 4500])
def test_stage3_select_matches_oracle_exactly(nb):
    rng = np.random.default_rng(nb)
    rows = _special_rows(nb, rng)
    while len(rows) < 24:
        z = rng.normal(scale=rng.uniform(0.1, 6.0), size=nb)
        p = np.exp(z - z.max())
        rows.append(p / p.sum())
    U = np.stack(rows)                                # 24 distinct rows
    idx = np.arange(nb) % len(U)
    Pm = np.stack([U[idx], U[(idx + 7) % len(U)]])[None]   # [1, 2, nb, nb]
    cases = [(4, 0.2), (8, 0.2), (0, 0.2), (1, 0.0), (0, 0.9), (nb, 0.2),
             (nb + 5, 0.5), (3, 1.0)]
    dP = to_dev(Pm)
    for k, tau in cases:
        _print("stage3", nb, k, tau)
        counts, kv = P.select_blocks(dP, k, tau)
        torch.cuda.synchronize()
        counts, kv = counts.cpu().numpy(), kv.cpu().numpy()
        rc, rl, _ = po.select_blocks(U, k, tau)
        for h, shift in ((0, 0), (1, 7)):
            for i in range(nb):
                u = (i % len(U) + shift) % len(U)
                assert counts[0, h, i] == rc[u], (k, tau, h, i)
                assert np.array_equal(kv[0, h, i, :rc[u]], rl[u]), (k, tau, h, i)


def test_stage3_golden_dyadic_row():
    p = np.array([1, 3, 5, 3, 0, 2, 2, 0], dtype=float) / 16.0
    Pm = np.tile(p, (8, 1))[None, None]
    dP = to_dev(Pm)
    for k, tau, want in [(1, 0.5, [1, 2]), (4, 0.2, [1, 2, 3, 5]),
                         (0, 0.0, [2]), (1, 1.0, [0, 1, 2, 3, 5, 6]),
                         (7, 0.2, [0, 1, 2, 3, 4, 5, 6])]:
        counts, kv = P.select_blocks(dP, k, tau)
        torch.cuda.synchronize()
        assert counts[0, 0, 0].item() == len(want)
        assert kv[0, 0, 0, :len(want)].cpu().tolist() == want


def test_stage3_capacity_larger_than_nb():
    rng = np.random.default_rng(0)
    nb = 70
    z = rng.normal(size=(1, 1, nb, nb))
    Pm = np.exp(z - z.max(-1, keepdims=True))
    Pm /= Pm.sum(-1, keepdims=True)
    counts, kv = P.select_blocks(to_dev(Pm), 2, 0.3, capacity=nb + 13)
    torch.cuda.synchronize()
    rc, rl, _ = po.select_blocks(Pm[0, 0], 2, 0.3)
    assert np.array_equal(counts[0, 0].cpu().numpy(), rc)
    kv = kv.cpu().numpy()
    for i in range(nb):
        assert np.array_equal(kv[0, 0, i, :rc[i]], rl[i])


# ------------------------------------------------------------------ stage 4
def _random_lists(nb, rng, maxc=None):
    counts = np.empty(nb, dtype=np.int64)
    lists = []
    for i in range(nb):
        c = int(rng.integers(1, min(maxc or nb, nb) + 1))
        if i == 0:
            c = nb                      # one full row
        if i == 1:
            c = 1
        L = np.sort(rng.choice(nb, size=c, replace=False))
        counts[i] = c
        lists.append(L)
    return counts, lists


def _pack(counts_bh, lists_bh, nb):
    B, Hh = len(counts_bh), len(counts_bh[0])
    counts = np.zeros((B, Hh, nb), dtype=np.int32)
    kv = np.full((B, Hh, nb, nb), -1, dtype=np.int32)
    for b in range(B):
        for h in range(Hh):
            counts[b, h] = counts_bh[b][h]
            for i, L in enumerate(lists_bh[b][h]):
                kv[b, h, i, :len(L)] = L
    return counts, kv


def _attn_case(dtype, d, T=20, H=18, W=24, B=2, Hh=2, seed=0, maxc=12):
    N = T * H * W
    nb = N // 64
    rng = np.random.default_rng(seed)
    q = iid_normal((B, Hh, N, d), seed=seed + 1, dtype=dtype)
    k = iid_normal((B, Hh, N, d), seed=seed + 2, dtype=dtype)
    v = iid_normal((B, Hh, N, d), seed=seed + 3, dtype=dtype)
    do = iid_normal((B, Hh, N, d), seed=seed + 4, dtype=dtype)
    perm = _two_perms(T, H, W)[:B]
    cl = [[_random_lists(nb, rng, maxc) for _ in range(Hh)] for _ in range(B)]
    counts, kv = _pack([[c for c, _ in row] for row in cl],
                       [[l for _, l in row] for row in cl], nb)
    return dict(q=q, k=k, v=v, do=do, perm=perm, counts=counts, kv=kv,
                lists=[[l for _, l in row] for row in cl], B=B, Hh=Hh, N=N)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64),
                                     ("fp32", 64), ("fp32", 128)])
def test_stage4_forward(dtype, d):
    c = _attn_case(dtype, d)
    _print("fwd", dtype, d)
    o, lse = P.sparse_attn_fwd(to_dev(c["q"]), to_dev(c["k"]), to_dev(c["v"]),
                               to_dev(c["perm"]), to_dev(c["counts"]),
                               to_dev(c["kv"]))
    torch.cuda.synchronize()
    o, lse = to_host(o), lse.cpu().numpy()
    bf = dtype == "bf16"
    for b in range(c["B"]):
        for h in range(c["Hh"]):
            ro, rl = po.sparse_attn_fwd(widen(c["q"][b, h]), widen(c["k"][b, h]),
                                        widen(c["v"][b, h]), c["perm"][b],
                                        c["lists"][b][h])
            r1 = assert_close(o[b, h], ro, bf, f"o[{b},{h}]")
            r2 = assert_close(lse[b, h], rl, bf, f"lse[{b},{h}]")
            _print("  o", r1, "lse", r2)


@pytest.mark.parametrize("dtype,d,maxc", [("bf16", 128, 12), ("bf16", 64, 12),
                                          ("fp32", 64, 12), ("fp32", 128, 12),
                                          ("bf16", 128, None), ("bf16", 64, None)])
def test_stage4_backward(dtype, d, maxc):
    """Every row of dQ, dK, dV against the oracle.  maxc=None draws list
    lengths up to Nb, so every KV block is selected by about half of the 135
    query blocks and the dK / dV kernel walks long column unions."""
    c = _attn_case(dtype, d, seed=7, maxc=maxc)
    _print("bwd", dtype, d, maxc)
    args = [to_dev(c[n]) for n in ("q", "k", "v")]
    perm, counts, kv = to_dev(c["perm"]), to_dev(c["counts"]), to_dev(c["kv"])
    o, lse = P.sparse_attn_fwd(*args, perm, counts, kv)
    dq, dk, dv = P.sparse_attn_bwd(*args, o, to_dev(c["do"]), lse, perm,
                                   counts, kv)
    torch.cuda.synchronize()
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    bf = dtype == "bf16"
    for b in range(c["B"]):
        for h in range(c["Hh"]):
            ref = po.sparse_attn_bwd(widen(c["q"][b, h]), widen(c["k"][b, h]),
                                     widen(c["v"][b, h]), widen(c["do"][b, h]),
                                     c["perm"][b], c["lists"][b][h])
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                st = assert_close(g[b, h], r, bf, f"{name}[{b},{h}]")
                _print(" ", name, st)


@pytest.mark.parametrize("grid", [(4, 4, 4), (4, 4, 8), (4, 4, 12)])
@pytest.mark.parametrize("d", [128, 64])
def test_stage4_tiny_block_counts(grid, d):
    """1, 2 and 3 blocks: a pair with no second block, one full pair, and a
    pair plus a single (neighbouring blocks are processed in pairs)."""
    T, H, W = grid
    c = _attn_case("bf16", d, T=T, H=H, W=W, B=2, Hh=2, seed=11)
    _print("tiny", grid, d)
    args = [to_dev(c[n]) for n in ("q", "k", "v")]
    perm, counts, kv = to_dev(c["perm"]), to_dev(c["counts"]), to_dev(c["kv"])
    o, lse = P.sparse_attn_fwd(*args, perm, counts, kv)
    dq, dk, dv = P.sparse_attn_bwd(*args, o, to_dev(c["do"]), lse, perm,
                                   counts, kv)
    torch.cuda.synchronize()
    o, lse = to_host(o), lse.cpu().numpy()
    got = [t.cpu().numpy() for t in (dq, dk, dv)]
    for b in range(c["B"]):
        for h in range(c["Hh"]):
            qq, kk, vv = (widen(c[n][b, h]) for n in ("q", "k", "v"))
            ro, rl = po.sparse_attn_fwd(qq, kk, vv, c["perm"][b], c["lists"][b][h])
            assert_close(o[b, h], ro, True, f"o[{b},{h}]")
            assert_close(lse[b, h], rl, True, f"lse[{b},{h}]")
            ref = po.sparse_attn_bwd(qq, kk, vv, widen(c["do"][b, h]),
                                     c["perm"][b], c["lists"][b][h])
            for name, g, r in zip(("dq", "dk", "dv"), got, ref):
                assert_close(g[b, h], r, True, f"{name}[{b},{h}]")


def test_stage4_max_block_count():
    """Nb = 8192 (the largest supported): one query block selects every KV
    block (a union of 8192 entries), the others a few random ones; sampled
    rows of o, lse, dq and dK / dV of little-used KV blocks against the
    oracle."""
    T, H, W = 32, 128, 128
    N = T * H * W
    nb = N // 64
    assert nb == 8192
    rng = np.random.default_rng(8192)
    d = 128
    q, k, v, do = (iid_normal((1, 1, N, d), seed=s, dtype="bf16")
                   for s in (81, 82, 83, 84))
    perm = _two_perms(T, H, W)[1:2]
    counts = np.zeros((1, 1, nb), dtype=np.int32)
    kv = np.full((1, 1, nb, nb), -1, dtype=np.int32)
    lists = []
    for i in range(nb):
        L = (np.arange(nb) if i == 0 else
             np.sort(rng.choice(nb, size=int(rng.integers(1, 17)), replace=False)))
        counts[0, 0, i] = len(L)
        kv[0, 0, i, :len(L)] = L
        lists.append(L)
    _print("max blocks", nb)
    args = [to_dev(a) for a in (q, k, v)]
    dperm, dcounts, dkv = to_dev(perm), to_dev(counts), to_dev(kv)
    o, lse = P.sparse_attn_fwd(*args, dperm, dcounts, dkv)
    dq, dk, dv = P.sparse_attn_bwd(*args, o, to_dev(do), lse, dperm, dcounts, dkv)
    torch.cuda.synchronize()
    o, lse = to_host(o), lse.cpu().numpy()
    dq, dk, dv = (t.cpu().numpy() for t in (dq, dk, dv))
    pm = perm[0]
    q0, k0, v0, do0 = (widen(a[0, 0]) for a in (q, k, v, do))
    blocks = [0, 1, 4095, 8191]
    ro, rl = po.sparse_attn_fwd(q0, k0, v0, pm, lists, query_blocks=blocks)
    rows = np.concatenate([pm[64 * i:64 * (i + 1)] for i in blocks])
    assert_close(o[0, 0][rows], ro[rows], True, "o")
    assert_close(lse[0, 0][rows], rl[rows], True, "lse")
    rq, _, _ = po.sparse_attn_bwd(q0, k0, v0, do0, pm, lists, query_blocks=blocks)
    assert_close(dq[0, 0][rows], rq[rows], True, "dq")
    users = [[] for _ in range(nb)]
    for i, L in enumerate(lists):
        for j in L:
            users[j].append(i)
    picks = sorted(range(nb), key=lambda j: len(users[j]))[:3]
    qb = sorted(set(i for j in picks for i in users[j]))
    _, rk, rv = po.sparse_attn_bwd(q0, k0, v0, do0, pm, lists, query_blocks=qb)
    cols = np.concatenate([pm[64 * j:64 * (j + 1)] for j in picks])
    assert_close(dk[0, 0][cols], rk[cols], True, "dk")
    assert_close(dv[0, 0][cols], rv[cols], True, "dv")


def test_stage4_list_order_does_not_matter():
    """The ABI takes each row's ids in any order: the bf16 kernels walk the
    ascending union of a pair's lists, so shuffled lists must give
    bit-identical outputs and gradients."""
    c = _attn_case("bf16", 128, seed=5, B=2, Hh=2)
    _print("list order")
    args = [to_dev(c[n]) for n in ("q", "k", "v")]
    perm, counts = to_dev(c["perm"]), to_dev(c["counts"])
    kv = c["kv"]
    rng = np.random.default_rng(77)
    shuffled = kv.copy()
    for b in range(c["B"]):
        for h in range(c["Hh"]):
            for i in range(kv.shape[2]):
                n = int(c["counts"][b, h, i])
                shuffled[b, h, i, :n] = rng.permutation(kv[b, h, i, :n])
    assert not np.array_equal(shuffled, kv)
    do = to_dev(c["do"])
    outs = []
    for lists in (kv, shuffled):
        kvd = to_dev(lists)
        o, lse = P.sparse_attn_fwd(*args, perm, counts, kvd)
        g = P.sparse_attn_bwd(*args, o, do, lse, perm, counts, kvd)
        torch.cuda.synchronize()
        outs.append([o, lse, *g])
    for a, b in zip(*outs):
        assert torch.equal(a, b)


def test_stage4_deterministic_and_poison_safe():
    c = _attn_case("bf16", 128, seed=3, B=1, Hh=2)
    args = [to_dev(c[n]) for n in ("q", "k", "v")]
    perm, counts, kv = to_dev(c["perm"]), to_dev(c["counts"]), to_dev(c["kv"])
    o1, l1 = P.sparse_attn_fwd(*args, perm, counts, kv)
    g1 = P.sparse_attn_bwd(*args, o1, to_dev(c["do"]), l1, perm, counts, kv)
    # poison the outputs' memory, run again: everything must be rewritten
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    wsf = torch.full((P.prism_sparse_attn_fwd_workspace_bytes(1, 2, c["N"], 128),),
                     255, dtype=torch.uint8, device="cuda")
    P.prism_sparse_attn_fwd(args[0].data_ptr(), args[1].data_ptr(),
                            args[2].data_ptr(), P.PRISM_BF16, perm.data_ptr(),
                            counts.data_ptr(), kv.data_ptr(), kv.shape[-1], 1, 2,
                            c["N"], 128, -1.0, o2.data_ptr(), l2.data_ptr(),
                            wsf.data_ptr(), wsf.numel(),
                            torch.cuda.current_stream().cuda_stream)
    g2 = [torch.full_like(t, float("nan")) for t in g1]
    ws = torch.full((P.prism_sparse_attn_bwd_workspace_bytes(1, 2, c["N"], 128),),
                    255, dtype=torch.uint8, device="cuda")
    P.prism_sparse_attn_bwd(args[0].data_ptr(), args[1].data_ptr(),
                            args[2].data_ptr(), o2.data_ptr(),
                            to_dev(c["do"]).data_ptr(), l2.data_ptr(),
                            P.PRISM_BF16, perm.data_ptr(), counts.data_ptr(),
                            kv.data_ptr(), kv.shape[-1], 1, 2, c["N"], 128, -1.0,
                            g2[0].data_ptr(), g2[1].data_ptr(), g2[2].data_ptr(),
                            ws.data_ptr(), ws.numel(),
                            torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


# ---------------------------------------------------------- whole pipeline
def test_pipeline_tiny_fp32_config():
    """The tiny fp32 workload end to end: stages 1-4 on the GPU."""
    x = make_inputs(0)
    cfg = x.cfg
    T, H, W = cfg["T"], cfg["H"], cfg["W"]
    _print("pipeline tiny fp32")
    zs, perm, _, _ = P.zone_shapes(None, None, T, H, W, fixed_shape=0)
    q, k, v = to_dev(x.q), to_dev(x.k), to_dev(x.v)
    qm, km, proxy = P.pool_blocks(q, k, perm)
    counts, kv = P.select_blocks(proxy, cfg["top_k"], cfg["cdf_threshold"])
    o, lse = P.sparse_attn_fwd(q, k, v, perm, counts, kv)
    torch.cuda.synchronize()
    rperm = po.zone_shapes(None, None, T, H, W, fixed_shape=0)["perm"]
    assert np.array_equal(perm[0].cpu().numpy(), rperm)
    for h in range(cfg["Hh"]):
        rq, rk, rv = (widen(a[0, h]) for a in (x.q, x.k, x.v))
        route = po.route_head(rq, rk, rperm, cfg["top_k"], cfg["cdf_threshold"])
        assert np.array_equal(counts[0, h].cpu().numpy(), route["counts"])
        assert np.all(route["counts"] == 1)   # max p >= 1/4 > 0.2
        kvh = kv[0, h].cpu().numpy()
        for i, L in enumerate(route["lists"]):
            assert np.array_equal(kvh[i, :len(L)], L)
        ro, rl = po.sparse_attn_fwd(rq, rk, rv, rperm, route["lists"])
        assert_close(o[0, h].cpu().numpy(), ro, False, "o")
        assert_close(lse[0, h].cpu().numpy(), rl, False, "lse")


def test_stage4_lists_outside_the_contract():
    """Lists the host cannot check (they live in device memory): a count of
    0, a count above Nb, ids outside [0, Nb) and duplicate ids.  The kernels
    clamp counts to [0, Nb], skip invalid ids and (bf16) merge duplicates:
    results equal those of the cleaned lists, a block with no valid id gets
    o = 0, lse = -inf, dq = 0 and adds nothing to dk, dv."""
    T, H, W = 20, 18, 24
    c = _attn_case("bf16", 128, T=T, H=H, W=W, B=1, Hh=2, seed=21, maxc=20)
    nb = c["N"] // 64
    counts, kv = c["counts"].copy(), c["kv"].copy()
    clean = [list(L) for L in c["lists"][0]]
    # head 0: block 3 empty, block 4 with every id invalid, block 5 with a
    # count above Nb over a row padded with invalid ids; head 1: invalid and
    # duplicate ids mixed into valid lists
    counts[0, 0, 3] = 0
    clean[0][3] = []
    counts[0, 0, 4] = 3
    kv[0, 0, 4, :3] = [-1, nb, 1 << 20]
    clean[0][4] = []
    L5 = list(clean[0][5])
    kv[0, 0, 5, :] = -7
    kv[0, 0, 5, :len(L5)] = L5
    counts[0, 0, 5] = nb + 50
    for i in (6, 7, 8):
        L = list(c["lists"][0][1][i])
        row = [L[0], -3, L[0], nb + 1] + L[1:] + [L[-1]]
        kv[0, 1, i, :len(row)] = row
        counts[0, 1, i] = len(row)
    _print("lists outside the contract")
    args = [to_dev(c[n]) for n in ("q", "k", "v")]
    perm, dcounts, dkv = to_dev(c["perm"]), to_dev(counts), to_dev(kv)
    o, lse = P.sparse_attn_fwd(*args, perm, dcounts, dkv)
    dq, dk, dv = P.sparse_attn_bwd(*args, o, to_dev(c["do"]), lse, perm,
                                   dcounts, dkv)
    torch.cuda.synchronize()
    o, lse = to_host(o), lse.cpu().numpy()
    dq, dk, dv = (t.cpu().numpy() for t in (dq, dk, dv))
    pm = c["perm"][0]
    for h in range(2):
        qq, kk, vv, dd = (widen(c[n][0, h]) for n in ("q", "k", "v", "do"))
        lists = [np.array(sorted(set(L)), dtype=np.int64) for L in clean[h]]
        live = [i for i in range(nb) if len(lists[i])]
        dead = [i for i in range(nb) if not len(lists[i])]
        ro, rl = po.sparse_attn_fwd(qq, kk, vv, pm, lists, query_blocks=live)
        rdq, rdk, rdv = po.sparse_attn_bwd(qq, kk, vv, dd, pm, lists,
                                           query_blocks=live)
        rows = np.concatenate([pm[64 * i:64 * (i + 1)] for i in live])
        assert_close(o[0, h][rows], ro[rows], True, f"o head {h}")
        assert_close(lse[0, h][rows], rl[rows], True, f"lse head {h}")
        assert_close(dq[0, h][rows], rdq[rows], True, f"dq head {h}")
        assert_close(dk[0, h], rdk, True, f"dk head {h}")
        assert_close(dv[0, h], rdv, True, f"dv head {h}")
        if dead:
            drows = np.concatenate([pm[64 * i:64 * (i + 1)] for i in dead])
            assert np.all(o[0, h][drows] == 0.0)
            assert np.all(np.isneginf(lse[0, h][drows]))
            assert np.all(dq[0, h][drows] == 0.0)
        _print(f"  head {h}: {len(dead)} blocks without a valid id")
