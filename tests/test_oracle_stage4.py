"""Pins for the oracle's block-sparse attention, forward and backward.

* every block selected == dense attention (torch scaled_dot_product_attention
  in fp64 on the CPU);
* arbitrary lists == dense attention under the equivalent boolean mask;
* one block selected == dense attention inside each block;
* permuting tokens inside a block leaves the raster-order output unchanged;
* gradients == torch autograd through the masked dense attention (fp64) and
  central finite differences.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import prism_oracle as po


def _setup(T=4, H=8, W=8, d=64, sid=0, seed=0, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    N = T * H * W
    q = rng.normal(size=(N, d)) * scale_qk
    k = rng.normal(size=(N, d)) * scale_qk
    v = rng.normal(size=(N, d))
    perm = po.zone_shapes(None, None, T, H, W, fixed_shape=sid)["perm"]
    return q, k, v, perm


def _mask_from_lists(perm, lists, N):
    nb = N // 64
    blk = np.empty(N, dtype=np.int64)       # block of each raster token
    blk[perm] = np.arange(N) // 64
    sel = np.zeros((nb, nb), bool)
    for i, L in enumerate(lists):
        sel[i, L] = True
    return sel[blk[:, None], blk[None, :]]  # [N, N] allowed(query, key)


def _sdpa(q, k, v, mask=None):
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))[None, None]
    o = F.scaled_dot_product_attention(t(q), t(k), t(v),
                                       attn_mask=None if mask is None
                                       else torch.from_numpy(mask)[None, None])
    return o[0, 0].numpy()


def _lse(q, k, mask=None):
    s = torch.from_numpy(q) @ torch.from_numpy(k).T / math.sqrt(q.shape[1])
    if mask is not None:
        s = s.masked_fill(~torch.from_numpy(mask), -math.inf)
    return torch.logsumexp(s, dim=1).numpy()


def test_all_blocks_equals_dense():
    q, k, v, perm = _setup(T=8, H=8, W=8, d=64, sid=1)
    nb = q.shape[0] // 64
    lists = [np.arange(nb)] * nb
    o, lse = po.sparse_attn_fwd(q, k, v, perm, lists)
    np.testing.assert_allclose(o, _sdpa(q, k, v), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lse, _lse(q, k), rtol=1e-13)


def test_single_block_equals_blockwise_dense():
    q, k, v, perm = _setup(T=4, H=8, W=16, d=32, sid=0)
    nb = q.shape[0] // 64
    lists = [np.array([i]) for i in range(nb)]
    o, _ = po.sparse_attn_fwd(q, k, v, perm, lists)
    for i in range(nb):
        rows = perm[64 * i:64 * (i + 1)]
        np.testing.assert_allclose(o[rows], _sdpa(q[rows], k[rows], v[rows]),
                                   rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("d,sid", [(64, 0), (128, 7)])
def test_random_lists_equal_masked_dense(d, sid):
    q, k, v, perm = _setup(T=4, H=16, W=16, d=d, sid=sid, seed=3)
    N = q.shape[0]
    nb = N // 64
    rng = np.random.default_rng(9)
    lists = [np.sort(rng.choice(nb, size=int(rng.integers(1, nb + 1)),
                                replace=False)) for _ in range(nb)]
    mask = _mask_from_lists(perm, lists, N)
    o, lse = po.sparse_attn_fwd(q, k, v, perm, lists)
    np.testing.assert_allclose(o, _sdpa(q, k, v, mask), rtol=1e-11,
                               atol=1e-12)
    np.testing.assert_allclose(lse, _lse(q, k, mask), rtol=1e-13)


def test_in_block_permutation_invariance():
    q, k, v, perm = _setup(T=4, H=8, W=8, d=64, seed=7)
    nb = q.shape[0] // 64
    lists = [np.array([0, 2]), np.array([1]), np.array([0, 1, 2, 3]),
             np.array([3])]
    o1, l1 = po.sparse_attn_fwd(q, k, v, perm, lists)
    rng = np.random.default_rng(1)
    perm2 = perm.copy()
    for i in range(nb):
        perm2[64 * i:64 * (i + 1)] = rng.permutation(perm[64 * i:64 * (i + 1)])
    o2, l2 = po.sparse_attn_fwd(q, k, v, perm2, lists)
    np.testing.assert_allclose(o1, o2, rtol=1e-12, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=1e-13)


def test_query_block_subset():
    q, k, v, perm = _setup(T=4, H=8, W=8, d=64, seed=2)
    lists = [np.array([0, 1]), np.array([1]), np.array([2, 3]),
             np.array([0, 3])]
    o_all, _ = po.sparse_attn_fwd(q, k, v, perm, lists)
    o_sub, _ = po.sparse_attn_fwd(q, k, v, perm, lists, query_blocks=[2])
    rows = perm[128:192]
    np.testing.assert_array_equal(o_sub[rows], o_all[rows])
    assert np.isnan(o_sub[perm[0]]).all()


def _autograd_grads(q, k, v, do, mask):
    tq, tk, tv = (torch.from_numpy(a).clone().requires_grad_(True)
                  for a in (q, k, v))
    o = F.scaled_dot_product_attention(
        tq[None, None], tk[None, None], tv[None, None],
        attn_mask=torch.from_numpy(mask)[None, None])[0, 0]
    o.backward(torch.from_numpy(do))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


@pytest.mark.parametrize("d", [64, 128])
def test_backward_matches_autograd(d):
    q, k, v, perm = _setup(T=4, H=16, W=16, d=d, sid=3, seed=5)
    N = q.shape[0]
    nb = N // 64
    rng = np.random.default_rng(21)
    do = rng.normal(size=(N, d))
    lists = [np.sort(rng.choice(nb, size=int(rng.integers(1, 6)),
                                replace=False)) for _ in range(nb)]
    dq, dk, dv = po.sparse_attn_bwd(q, k, v, do, perm, lists)
    gq, gk, gv = _autograd_grads(q, k, v, do, _mask_from_lists(perm, lists, N))
    for a, b in ((dq, gq), (dk, gk), (dv, gv)):
        np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-11)


def test_backward_finite_differences():
    # central differences of L = <dO, O> on a few coordinates
    q, k, v, perm = _setup(T=4, H=8, W=8, d=16, seed=8)
    N = q.shape[0]
    rng = np.random.default_rng(6)
    do = rng.normal(size=(N, 16))
    lists = [np.array([0, 2]), np.array([1, 3]), np.array([2]),
             np.array([0, 1, 2, 3])]
    dq, dk, dv = po.sparse_attn_bwd(q, k, v, do, perm, lists)

    def loss(q, k, v):
        o, _ = po.sparse_attn_fwd(q, k, v, perm, lists)
        return float(np.sum(o * do))

    h = 1e-6
    for name, arr, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        for _ in range(6):
            r, c = int(rng.integers(N)), int(rng.integers(16))
            ap, am = arr.copy(), arr.copy()
            ap[r, c] += h
            am[r, c] -= h
            args_p = dict(q=q, k=k, v=v)
            args_m = dict(q=q, k=k, v=v)
            args_p[name], args_m[name] = ap, am
            fd = (loss(**args_p) - loss(**args_m)) / (2 * h)
            assert abs(fd - grad[r, c]) < 1e-6 * max(1.0, abs(fd)), \
                (name, r, c, fd, grad[r, c])


def test_unselected_kv_get_zero_gradient():
    q, k, v, perm = _setup(T=4, H=8, W=8, d=32, seed=4)
    N = q.shape[0]
    do = np.random.default_rng(0).normal(size=(N, 32))
    lists = [np.array([0]), np.array([0, 1]), np.array([1]), np.array([0])]
    _, dk, dv = po.sparse_attn_bwd(q, k, v, do, perm, lists)
    for j in (2, 3):
        rows = perm[64 * j:64 * (j + 1)]
        assert np.all(dk[rows] == 0) and np.all(dv[rows] == 0)
