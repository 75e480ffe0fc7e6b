"""GPU parity of the forward-only variant that keeps a pooled stand-in of
the unselected blocks in the softmax (prism_dropped_terms +
prism_sparse_attn_fwd_corrected), against the fp64 oracle.

Sizes: Nb = 135 (two full 64-row tiles of query blocks plus 7, and 32-column
proxy slices with a ragged last one), batch 2 with two different
permutations, random lists including a row that keeps every block and a row
that keeps one.  All calls go through the C ABI.
"""
import numpy as np
import pytest
import torch

import dynamic_block_sparse_shape_amd as P
from oracle import prism_oracle as po
from tests.gpu_util import assert_close, err_stats, to_dev, to_host, widen
from tests.test_gpu_parity import _attn_case

pytestmark = pytest.mark.gpu


def _print(*a):
    print(*a, flush=True)


def _run(c):
    q, k, v = (to_dev(c[n]) for n in ("q", "k", "v"))
    perm, counts, kv = to_dev(c["perm"]), to_dev(c["counts"]), to_dev(c["kv"])
    qm, km, proxy = P.pool_blocks(q, k, perm)
    dl, dv = P.dropped_terms(proxy, qm, km, v, perm, counts, kv)
    oc, lc = P.sparse_attn_fwd_corrected(q, k, v, perm, counts, kv, dl, dv)
    o, l = P.sparse_attn_fwd(q, k, v, perm, counts, kv)
    torch.cuda.synchronize()
    return dl, dv, oc, lc, o, l


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64),
                                     ("fp32", 64), ("fp32", 128)])
def test_dropped_terms_and_corrected_forward(dtype, d):
    c = _attn_case(dtype, d, seed=21, maxc=12)
    _print("corrected fwd", dtype, d)
    dl, dv, oc, lc, o, l = _run(c)
    dl, dv, lc, l = (t.cpu().numpy() for t in (dl, dv, lc, l))
    oc, o = to_host(oc), to_host(o)
    bf = dtype == "bf16"
    changed = 0.0
    for b in range(c["B"]):
        perm = c["perm"][b]
        for h in range(c["Hh"]):
            qh, kh, vh = (widen(c[n][b, h]) for n in ("q", "k", "v"))
            lists = c["lists"][b][h]
            rdl, rdv = po.dropped_block_terms(po.pool_blocks(qh, perm),
                                              po.pool_blocks(kh, perm),
                                              po.pool_blocks(vh, perm), lists)
            fin = np.isfinite(rdl)
            assert np.array_equal(np.isfinite(dl[b, h]), fin), (b, h)
            assert not fin[0] and fin[1:].all()       # row 0 keeps every block
            np.testing.assert_allclose(dl[b, h][fin], rdl[fin], rtol=1e-6,
                                       atol=1e-6)
            rel, mx = err_stats(dv[b, h], rdv)
            assert rel < 1e-5 and mx < 1e-5, ("drop_v", b, h, rel, mx)
            ro, rl = po.sparse_attn_fwd_corrected(qh, kh, vh, perm, lists)
            r1 = assert_close(oc[b, h], ro, bf, f"o corrected [{b},{h}]")
            r2 = assert_close(lc[b, h], rl, bf, f"lse corrected [{b},{h}]")
            _print("  drop_v", (rel, mx), "o", r1, "lse", r2)
            # the query block that keeps every block: bit-identical to the
            # plain forward
            rows0 = perm[:64]
            assert np.array_equal(oc[b, h][rows0], o[b, h][rows0])
            assert np.array_equal(lc[b, h][rows0], l[b, h][rows0])
            changed = max(changed, float(np.abs(oc[b, h] - o[b, h]).max()))
    assert changed > 1e-2          # the stand-in does change the other rows


@pytest.mark.parametrize("grid", [(4, 4, 8), (4, 4, 12), (4, 8, 16)])
def test_corrected_forward_tiny_block_counts(grid):
    """2, 3 and 8 blocks per head (one 32-column proxy slice, partly empty;
    one 64-row tile, mostly empty): rows that keep one block and rows that
    keep all."""
    T, H, W = grid
    c = _attn_case("bf16", 128, T=T, H=H, W=W, seed=13)
    _print("corrected fwd tiny", grid)
    dl, dv, oc, lc, o, l = _run(c)
    dl, dv, lc = (t.cpu().numpy() for t in (dl, dv, lc))
    oc = to_host(oc)
    for b in range(c["B"]):
        perm = c["perm"][b]
        for h in range(c["Hh"]):
            qh, kh, vh = (widen(c[n][b, h]) for n in ("q", "k", "v"))
            lists = c["lists"][b][h]
            rdl, rdv = po.dropped_block_terms(po.pool_blocks(qh, perm),
                                              po.pool_blocks(kh, perm),
                                              po.pool_blocks(vh, perm), lists)
            fin = np.isfinite(rdl)
            assert np.array_equal(np.isfinite(dl[b, h]), fin)
            np.testing.assert_allclose(dl[b, h][fin], rdl[fin], rtol=1e-6, atol=1e-6)
            rel, mx = err_stats(dv[b, h], rdv)
            assert rel < 1e-5 and mx < 1e-5, ("drop_v", b, h, rel, mx)
            ro, rl = po.sparse_attn_fwd_corrected(qh, kh, vh, perm, lists)
            assert_close(oc[b, h], ro, True, f"o corrected [{b},{h}]")
            assert_close(lc[b, h], rl, True, f"lse corrected [{b},{h}]")


@pytest.mark.parametrize("grid", [(1, 8, 8), (4, 4, 12), (20, 18, 24)])
def test_corrected_forward_with_every_block_kept_is_the_plain_forward(grid):
    T, H, W = grid
    c = _attn_case("bf16", 128, T=T, H=H, W=W, seed=5)
    nb = c["N"] // 64
    c["counts"][:] = nb
    c["kv"][:] = np.arange(nb, dtype=np.int32)
    _print("all kept", grid)
    dl, dv, oc, lc, o, l = _run(c)
    assert torch.isneginf(dl).all() and (dv == 0).all()
    assert torch.equal(oc, o) and torch.equal(lc, l)


def test_corrected_forward_max_block_count():
    """Nb = 8192 (the largest supported): the stand-in terms stream 256
    bitmap words per row; one query block keeps every block, the others a
    few; sampled rows against the oracle."""
    from synth import iid_normal
    from tests.test_gpu_parity import _two_perms
    T, H, W = 32, 128, 128
    N = T * H * W
    nb = N // 64
    assert nb == 8192
    rng = np.random.default_rng(4096)
    d = 128
    q, k, v = (iid_normal((1, 1, N, d), seed=s, dtype="bf16", scale=2.0)
               for s in (91, 92, 93))
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
    _print("corrected fwd, max blocks", nb)
    c = dict(q=q, k=k, v=v, perm=perm, counts=counts, kv=kv)
    dl, dv, oc, lc, o, l = _run(c)
    dl, dv, lc, l = (t.cpu().numpy() for t in (dl, dv, lc, l))
    oc, o = to_host(oc), to_host(o)
    pm = perm[0]
    q0, k0, v0 = (widen(a[0, 0]) for a in (q, k, v))
    blocks = [0, 1, 5000, 8191]
    qm = po.pool_blocks(q0, pm)
    rdl, rdv = po.dropped_block_terms(qm[blocks], po.pool_blocks(k0, pm),
                                      po.pool_blocks(v0, pm),
                                      [lists[i] for i in blocks])
    assert np.isneginf(dl[0, 0, 0]) and np.isneginf(rdl[0])
    np.testing.assert_allclose(dl[0, 0][blocks[1:]], rdl[1:], rtol=1e-6)
    rel, mx = err_stats(dv[0, 0][blocks], rdv)
    assert rel < 1e-5 and mx < 1e-5, (rel, mx)
    ro, rl = po.sparse_attn_fwd_corrected(q0, k0, v0, pm, lists,
                                          query_blocks=blocks)
    rows = np.concatenate([pm[64 * i:64 * (i + 1)] for i in blocks])
    assert_close(oc[0, 0][rows], ro[rows], True, "o corrected")
    assert_close(lc[0, 0][rows], rl[rows], True, "lse corrected")
    rows0 = pm[:64]
    assert np.array_equal(oc[0, 0][rows0], o[0, 0][rows0])
