"""Pins for the oracle's pooled stand-in of unselected blocks (reading R21).

* blocks whose 64 query, key and value rows are each constant: the stand-in
  is exact, so the corrected output equals dense attention (torch
  scaled_dot_product_attention in fp64 on the CPU), while the plain sparse
  output does not;
* every block selected: nothing is left out, corrected == sparse == dense;
* the one-softmax definition equals the log-sum-exp merge of the sparse
  output with ``dropped_block_terms``;
* ``dropped_block_terms`` equals the route through the stage-2 proxy
  probabilities (log-normaliser from scipy's logsumexp), which is how the
  GPU path computes it;
* permuting tokens inside a block leaves the corrected output unchanged.
"""
import math

import numpy as np
import torch
import torch.nn.functional as F
from scipy.special import logsumexp

from oracle import prism_oracle as po


def _perm(T, H, W, sid):
    return po.zone_shapes(None, None, T, H, W, fixed_shape=sid)["perm"]


def _sdpa(q, k, v):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    return F.scaled_dot_product_attention(t(q), t(k), t(v))[0, 0].numpy()


def _random_lists(nb, rng, lo=1, hi=None):
    hi = nb if hi is None else hi
    return [np.sort(rng.choice(nb, size=int(rng.integers(lo, hi + 1)),
                               replace=False)) for _ in range(nb)]


def _blockwise_constant(perm, nb, d, rng, scale=1.0):
    """[N, d] array whose 64 rows of each block (through perm) are equal."""
    x = np.empty((nb * 64, d))
    rows = rng.normal(size=(nb, d)) * scale
    for i in range(nb):
        x[perm[64 * i:64 * (i + 1)]] = rows[i]
    return x


def test_constant_blocks_make_the_stand_in_exact():
    T, H, W, d = 4, 16, 16, 32
    perm = _perm(T, H, W, 1)
    nb = T * H * W // 64
    rng = np.random.default_rng(4)
    q = _blockwise_constant(perm, nb, d, rng, 1.5)
    k = _blockwise_constant(perm, nb, d, rng, 1.5)
    v = _blockwise_constant(perm, nb, d, rng)
    lists = _random_lists(nb, rng, 1, nb // 2)
    dense = _sdpa(q, k, v)
    oc, lc = po.sparse_attn_fwd_corrected(q, k, v, perm, lists)
    np.testing.assert_allclose(oc, dense, rtol=1e-11, atol=1e-12)
    s = (q @ k.T) / math.sqrt(d)
    np.testing.assert_allclose(lc, logsumexp(s, axis=1), rtol=1e-13)
    o_sparse, _ = po.sparse_attn_fwd(q, k, v, perm, lists)
    assert np.abs(o_sparse - dense).max() > 1e-2      # the pin is not vacuous


def test_every_block_selected_leaves_nothing_out():
    T, H, W, d = 8, 8, 8, 64
    perm = _perm(T, H, W, 0)
    nb = T * H * W // 64
    rng = np.random.default_rng(2)
    q, k, v = (rng.normal(size=(nb * 64, d)) for _ in range(3))
    lists = [np.arange(nb)] * nb
    oc, lc = po.sparse_attn_fwd_corrected(q, k, v, perm, lists)
    o, l = po.sparse_attn_fwd(q, k, v, perm, lists)
    np.testing.assert_allclose(oc, o, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(lc, l, rtol=1e-14)
    np.testing.assert_allclose(oc, _sdpa(q, k, v), rtol=1e-11, atol=1e-12)
    dl, dv = po.dropped_block_terms(po.pool_blocks(q, perm),
                                    po.pool_blocks(k, perm),
                                    po.pool_blocks(v, perm), lists)
    assert np.all(np.isneginf(dl)) and np.all(dv == 0)


def test_one_softmax_equals_merge_with_dropped_terms():
    T, H, W, d = 4, 16, 16, 64
    perm = _perm(T, H, W, 3)
    nb = T * H * W // 64
    rng = np.random.default_rng(8)
    q, k, v = (rng.normal(size=(nb * 64, d)) for _ in range(3))
    lists = _random_lists(nb, rng)
    lists[0] = np.arange(nb)                  # one row with nothing left out
    oc, lc = po.sparse_attn_fwd_corrected(q, k, v, perm, lists)
    o, l = po.sparse_attn_fwd(q, k, v, perm, lists)
    dl, dv = po.dropped_block_terms(po.pool_blocks(q, perm),
                                    po.pool_blocks(k, perm),
                                    po.pool_blocks(v, perm), lists)
    blk = np.empty(nb * 64, dtype=np.int64)
    blk[perm] = np.arange(nb * 64) // 64
    L = np.logaddexp(l, dl[blk])
    om = (np.exp(l - L)[:, None] * o +
          np.exp(dl[blk] - L)[:, None] * dv[blk])
    np.testing.assert_allclose(lc, L, rtol=1e-13)
    np.testing.assert_allclose(oc, om, rtol=1e-11, atol=1e-12)


def test_dropped_terms_through_proxy_probabilities():
    T, H, W, d = 4, 16, 32, 128
    perm = _perm(T, H, W, 7)
    nb = T * H * W // 64
    rng = np.random.default_rng(12)
    q, k, v = (rng.normal(size=(nb * 64, d)) * 2.0 for _ in range(3))
    qm, km, vm = (po.pool_blocks(x, perm) for x in (q, k, v))
    P = po.proxy_scores(qm, km)
    lists = _random_lists(nb, rng)
    lse_p = logsumexp((qm @ km.T) / math.sqrt(d), axis=1)
    dl, dv = po.dropped_block_terms(qm, km, vm, lists)
    for i in range(nb):
        out = np.setdiff1d(np.arange(nb), lists[i])
        if out.size == 0:
            assert np.isneginf(dl[i])
            continue
        mass = P[i, out].sum()
        np.testing.assert_allclose(dl[i], math.log(64) + lse_p[i] + math.log(mass),
                                   rtol=1e-13)
        np.testing.assert_allclose(dv[i], (P[i, out] @ vm[out]) / mass,
                                   rtol=1e-11, atol=1e-13)


def test_corrected_in_block_permutation_invariance():
    T, H, W, d = 4, 8, 16, 32
    perm = _perm(T, H, W, 0)
    nb = T * H * W // 64
    rng = np.random.default_rng(5)
    q, k, v = (rng.normal(size=(nb * 64, d)) for _ in range(3))
    lists = _random_lists(nb, rng, 1, 3)
    o1, l1 = po.sparse_attn_fwd_corrected(q, k, v, perm, lists)
    perm2 = perm.copy()
    for i in range(nb):
        perm2[64 * i:64 * (i + 1)] = rng.permutation(perm[64 * i:64 * (i + 1)])
    o2, l2 = po.sparse_attn_fwd_corrected(q, k, v, perm2, lists)
    np.testing.assert_allclose(o1, o2, rtol=1e-11, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)
