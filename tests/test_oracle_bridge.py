"""Pins for the oracle's a2v bridge residual (oracle/bridge_oracle.py).

* library special case: torch's multi-head attention (fp64, CPU, separate
  query / key / value projection weights, no bias) equals the oracle without
  rotary alignment;
* closed forms: one audio token (the softmax is 1, every video token gets
  x_a Wv^T Wo^T); zero query weights (uniform scores, the audio mean); a
  two-token softmax worked out by hand, and two heads that attend to
  different audio tokens;
* rotary alignment: zero positions change nothing; shifting every position
  by one constant changes nothing (scores depend on differences only); a
  hand-computed rotation.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import bridge_oracle as bo


def _weights(rng, Cv, Ca, D, scale=0.1):
    return (rng.normal(size=(D, Cv)) * scale, rng.normal(size=(D, Ca)) * scale,
            rng.normal(size=(D, Ca)) * scale, rng.normal(size=(Cv, D)) * scale)


@pytest.mark.parametrize("heads,dh,Ca,N,Na", [(4, 8, 16, 50, 7),
                                             (3, 16, 24, 20, 33),
                                             (1, 4, 12, 9, 1)])
def test_bridge_equals_torch_multi_head_attention(heads, dh, Ca, N, Na):
    rng = np.random.default_rng(heads * 100 + Na)
    D = heads * dh
    Cv = D                             # torch's MHA has embed_dim = D = Cv
    x_v = rng.normal(size=(N, Cv))
    x_a = rng.normal(size=(Na, Ca))
    wq, wk, wv, wo = _weights(rng, Cv, Ca, D, scale=0.3)
    got = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads)
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a))
    out, _ = F.multi_head_attention_forward(
        t(x_v)[:, None, :], t(x_a)[:, None, :], t(x_a)[:, None, :],
        embed_dim_to_check=D, num_heads=heads, in_proj_weight=None,
        in_proj_bias=None, bias_k=None, bias_v=None, add_zero_attn=False,
        dropout_p=0.0, out_proj_weight=t(wo), out_proj_bias=None,
        training=False, need_weights=False, use_separate_proj_weight=True,
        q_proj_weight=t(wq), k_proj_weight=t(wk), v_proj_weight=t(wv))
    np.testing.assert_allclose(got, out[:, 0, :].numpy(), rtol=1e-12, atol=1e-13)


def test_one_audio_token_closed_form():
    rng = np.random.default_rng(1)
    heads, dh, Ca, N = 2, 8, 12, 30
    D = heads * dh
    x_v = rng.normal(size=(N, D))
    x_a = rng.normal(size=(1, Ca))
    wq, wk, wv, wo = _weights(rng, D, Ca, D, scale=1.0)
    got = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads)
    want = (x_a @ wv.T) @ wo.T                     # softmax over one key = 1
    np.testing.assert_allclose(got, np.repeat(want, N, axis=0), rtol=1e-13)


def test_zero_query_weights_give_the_audio_mean():
    rng = np.random.default_rng(2)
    heads, dh, Ca, N, Na = 3, 4, 10, 17, 9
    D = heads * dh
    x_v = rng.normal(size=(N, D))
    x_a = rng.normal(size=(Na, Ca))
    _, wk, wv, wo = _weights(rng, D, Ca, D, scale=1.0)
    got = bo.a2v_residual(x_v, x_a, np.zeros((D, D)), wk, wv, wo, heads)
    want = (x_a @ wv.T).mean(axis=0) @ wo.T        # uniform scores
    np.testing.assert_allclose(got, np.repeat(want[None], N, axis=0), rtol=1e-12)


def test_two_token_softmax_by_hand():
    # one head of width 2, identity weights: scores x_v . x_a / sqrt(2);
    # x_v = (sqrt(2) ln 3, 0) scores ln 3 on (1, 0) and 0 on (0, 0), so the
    # weights are 3/4 and 1/4 and the residual (3/4, 0)
    I = np.eye(2)
    x_v = np.array([[math.sqrt(2) * math.log(3.0), 0.0]])
    x_a = np.array([[1.0, 0.0], [0.0, 0.0]])
    got = bo.a2v_residual(x_v, x_a, I, I, I, I, heads=1)
    np.testing.assert_allclose(got, [[0.75, 0.0]], rtol=1e-14, atol=1e-16)
    # two heads of width 1 (scale 1): head 0 sees dimension 0, head 1
    # dimension 1.  Video (ln 3, ln 2) against audio (1, 0) and (0, 1):
    # head 0 weights 3/4, 1/4 -> v dim 0 = 3/4; head 1 weights 1/3, 2/3
    # (scores 0 and ln 2) -> v dim 1 = 2/3
    x_v = np.array([[math.log(3.0), math.log(2.0)]])
    x_a = np.eye(2)
    got = bo.a2v_residual(x_v, x_a, I, I, I, I, heads=2)
    np.testing.assert_allclose(got, [[0.75, 2.0 / 3.0]], rtol=1e-14)


def test_rotary_positions():
    rng = np.random.default_rng(3)
    heads, dh, Ca, N, Na = 2, 8, 6, 12, 5
    D = heads * dh
    x_v = rng.normal(size=(N, D))
    x_a = rng.normal(size=(Na, Ca))
    wq, wk, wv, wo = _weights(rng, D, Ca, D, scale=0.5)
    plain = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads)
    zero = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads,
                           pos_v=np.zeros(N), pos_a=np.zeros(Na))
    np.testing.assert_allclose(zero, plain, rtol=1e-14)
    pv, pa = rng.uniform(0, 100, N), rng.uniform(0, 100, Na)
    a = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads, pos_v=pv, pos_a=pa)
    b = bo.a2v_residual(x_v, x_a, wq, wk, wv, wo, heads, pos_v=pv + 37.5,
                        pos_a=pa + 37.5)
    np.testing.assert_allclose(a, b, rtol=1e-9, atol=1e-12)
    assert np.abs(a - plain).max() > 1e-3           # rotation does something
    # by hand, head_dim 2 (one pair, frequency base^0 = 1), identity
    # weights: the query (1, 0) at position t turns into (cos t, sin t); the
    # keys (1, 0) at position 0 and (0, 1) at position pi/2 into (1, 0) and
    # (-1, 0).  Scores cos t / sqrt 2 and -cos t / sqrt 2, values (1, 0) and
    # (0, 1), so the residual is the pair of softmax weights.
    t = 0.3
    I = np.eye(2)
    got = bo.a2v_residual(np.array([[1.0, 0.0]]), np.eye(2), I, I, I, I,
                          heads=1, pos_v=np.array([t]),
                          pos_a=np.array([0.0, math.pi / 2]))
    s = np.array([math.cos(t), -math.cos(t)]) / math.sqrt(2.0)
    w = np.exp(s) / np.exp(s).sum()
    np.testing.assert_allclose(got, [w], rtol=1e-13)
    # a second pair rotates base^(-2/4) = 1/100 as fast (head_dim 4, base
    # 10000): at position 100 its angle is 1 radian
    x = np.array([[0.0, 0.0, 1.0, 0.0]])
    r = bo.rotate_pairs(x[:, None, :], np.array([100.0]))[:, 0]
    np.testing.assert_allclose(r, [[0.0, 0.0, math.cos(1.0), math.sin(1.0)]],
                               rtol=1e-13, atol=1e-15)


def test_rows_subset():
    rng = np.random.default_rng(4)
    heads, dh, Ca, N, Na = 2, 4, 6, 20, 3
    D = heads * dh
    x_v = rng.normal(size=(N, D))
    x_a = rng.normal(size=(Na, Ca))
    w = _weights(rng, D, Ca, D)
    pv, pa = rng.uniform(0, 9, N), rng.uniform(0, 9, Na)
    full = bo.a2v_residual(x_v, x_a, *w, heads, pos_v=pv, pos_a=pa)
    rows = np.array([3, 0, 19])
    part = bo.a2v_residual(x_v, x_a, *w, heads, pos_v=pv, pos_a=pa, rows=rows)
    np.testing.assert_allclose(part, full[rows], rtol=1e-14)
