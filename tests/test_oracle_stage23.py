"""Pins for the oracle's stages 2 and 3: pooling, proxy score, selection.

Pooling: closed forms (block of constants, token-index field).  Proxy:
hand-derived logits whose softmax is rational, invariances, row sums.
Selection: hand-derived dyadic fixture, brute-force enumeration of all
subsets on small rows (exact rational arithmetic), invariants.
"""
import itertools
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import prism_oracle as po

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------------ pooling
def test_pool_blocks_constant_blocks():
    T, H, W = 4, 8, 8
    perm = po.zone_shapes(None, None, T, H, W, fixed_shape=0)["perm"]
    vals = np.array([3.0, -1.5, 0.25, 7.0])
    x = np.zeros((T * H * W, 5))
    for b in range(4):
        x[perm[64 * b:64 * (b + 1)]] = vals[b]
    np.testing.assert_array_equal(po.pool_blocks(x, perm),
                                  np.repeat(vals[:, None], 5, axis=1))


def test_pool_blocks_token_coordinates_are_box_centres():
    # pooling the coordinate fields gives each block's box centre
    T, H, W = 8, 8, 16
    for sid in (0, 1, 5, 7):
        out = po.zone_shapes(None, None, T, H, W, fixed_shape=sid)
        perm = out["perm"]
        coords = np.stack(np.indices((T, H, W)), axis=-1).reshape(-1, 3)
        means = po.pool_blocks(coords.astype(float), perm)
        et, eh, ew = po.SHAPES[sid]
        # block lattice of zone z: raster order of (bt, bh, bw)
        expect = []
        for (o, e) in out["zones"]:
            for bt in range(e[0] // et):
                for bh in range(e[1] // eh):
                    for bw in range(e[2] // ew):
                        expect.append([o[0] + bt * et + (et - 1) / 2,
                                       o[1] + bh * eh + (eh - 1) / 2,
                                       o[2] + bw * ew + (ew - 1) / 2])
        np.testing.assert_array_equal(means, np.array(expect))


# -------------------------------------------------------------------- proxy
def _read_proxy_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "proxy_log_integers.txt")):
        if line.startswith("#") or not line.strip():
            continue
        d, p = line.split("|")
        rows.append((int(d), [float(x) for x in p.split()]))
    return rows


@pytest.mark.parametrize("d,expect", _read_proxy_golden())
def test_proxy_closed_form(d, expect):
    qm = np.zeros((1, d))
    qm[0, 0] = math.sqrt(d)
    km = np.zeros((4, d))
    km[:, 0] = np.log(np.arange(1, 5))
    p = po.proxy_scores(qm, km)
    np.testing.assert_allclose(p[0], expect, rtol=1e-14)


def test_proxy_invariants():
    rng = np.random.default_rng(0)
    qm = rng.normal(size=(30, 64))
    km = rng.normal(size=(30, 64)) * 2
    p = po.proxy_scores(qm, km)
    np.testing.assert_allclose(p.sum(1), 1.0, rtol=1e-14)
    assert np.all(p > 0)
    # shifting every kbar by the same vector shifts a row's logits by a
    # constant, which the softmax ignores
    shift = rng.normal(size=64)
    np.testing.assert_allclose(po.proxy_scores(qm, km + shift), p, rtol=1e-11)
    # a zero query block scores every KV block equally
    np.testing.assert_allclose(po.proxy_scores(np.zeros((1, 64)), km),
                               np.full((1, 30), 1 / 30), rtol=1e-14)
    # logits are scaled by 1/sqrt(d): doubling d with duplicated features
    # keeps <q,k> doubled and sqrt(d) up by sqrt(2), so logits grow sqrt(2)x
    z = (qm @ km.T) / 8.0
    q2 = np.concatenate([qm, qm], 1)
    k2 = np.concatenate([km, km], 1)
    z2 = np.log(po.proxy_scores(q2, k2))
    z1 = math.sqrt(2.0) * z
    np.testing.assert_allclose(z2 - z2.max(1, keepdims=True),
                               z1 - z1.max(1, keepdims=True), atol=1e-10)


def test_proxy_extreme_logits_no_overflow():
    qm = np.array([[1e4, 0.0]])
    km = np.array([[1.0, 0.0], [0.999, 0.0], [-1.0, 0.0]])
    p = po.proxy_scores(qm, km)
    assert np.all(np.isfinite(p)) and abs(p.sum() - 1) < 1e-15
    assert p[0, 0] > 0.99


# ---------------------------------------------------------------- selection
def _read_sel_golden():
    rows = []
    p16 = None
    for line in open(os.path.join(GOLDEN, "selection_dyadic.txt")):
        if line.startswith("#") or not line.strip():
            continue
        if line.startswith("p16"):
            p16 = [int(x) for x in line.split("=")[1].split()]
            continue
        a, sel = line.split("|")
        k, tau = a.split()
        rows.append((p16, int(k), float(tau), [int(x) for x in sel.split()]))
    return rows


@pytest.mark.parametrize("p16,k,tau,expect", _read_sel_golden())
def test_selection_golden(p16, k, tau, expect):
    p = np.array(p16, dtype=float) / 16.0
    assert list(po.select_row(p, k, tau)) == expect
    counts, lists, _ = po.select_blocks(p[None, :], k, tau)
    assert list(lists[0]) == expect and counts[0] == len(expect)


def _brute_force(p_frac, k, tau):
    """Smallest set holding at least min(k, n) and at least one block whose
    mass reaches tau (or every block); among those, the largest mass; then
    the lexicographically smallest index list (lower indices first on equal
    scores).  Exact rational arithmetic."""
    n = len(p_frac)
    tau_f = Fraction(tau)
    lo = max(1, min(k, n))
    for size in range(lo, n + 1):
        best = None
        for S in itertools.combinations(range(n), size):
            mass = sum((p_frac[j] for j in S), Fraction(0))
            if mass < tau_f and size < n:
                continue
            key = (-mass, S)
            if best is None or key < best:
                best = key
        if best is not None:
            return list(best[1])
    raise AssertionError("unreachable")


def test_selection_brute_force_small_rows():
    rng = np.random.default_rng(11)
    for trial in range(300):
        n = int(rng.integers(1, 9))
        # dyadic scores with deliberate ties: every partial sum is exact
        w = rng.integers(0, 6, size=n)
        if w.sum() == 0:
            w[0] = 1
        total = 1 << int(math.ceil(math.log2(w.sum())))
        w[-1] += total - w.sum()
        p = w / total
        p_frac = [Fraction(int(x), total) for x in w]
        k = int(rng.integers(0, n + 2))
        tau = float(rng.choice([0.0, 0.1, 0.2, 0.25, 0.5, 0.75, 0.9, 1.0]))
        got = list(po.select_row(p, k, tau))
        assert got == _brute_force(p_frac, k, tau), (p, k, tau, got)


def test_selection_vectorised_matches_row_form_and_invariants():
    rng = np.random.default_rng(2)
    nb = 300
    z = rng.normal(scale=3.0, size=(nb, nb))
    P = np.exp(z - z.max(1, keepdims=True))
    P /= P.sum(1, keepdims=True)
    P[5, 10] = P[5, 11]                    # an exact tie
    for k, tau in [(4, 0.2), (8, 0.2), (0, 0.5), (1, 0.9), (600, 0.2)]:
        counts, lists, diag = po.select_blocks(P, k, tau)
        for i in range(nb):
            row = po.select_row(P[i], k, tau)
            assert np.array_equal(row, lists[i])
            sel = lists[i]
            c = len(sel)
            assert c == counts[i]
            # top-k floor, at least one block
            assert c >= max(1, min(k, nb))
            # ascending, unique
            assert np.all(np.diff(sel) > 0)
            mask = np.zeros(nb, bool)
            mask[sel] = True
            # prefix property: every kept score >= every dropped score
            if c < nb:
                assert P[i, mask].min() >= P[i, ~mask].max()
            # the mass reaches the threshold unless everything is kept
            mass = P[i, mask].sum()
            assert mass >= tau - 1e-12 or c == nb
            # minimality: beyond the top-k floor, dropping the smallest kept
            # block takes the mass below the threshold
            if c > max(1, k):
                assert mass - P[i, mask].min() < tau + 1e-12


def test_cumsum_is_sequential():
    # the vectorised selection relies on add.accumulate being a plain running
    # sum; check bitwise against a Python loop
    rng = np.random.default_rng(4)
    x = rng.random((7, 1000)) ** 6
    cs = np.cumsum(x, axis=1)
    for i in range(7):
        acc = 0.0
        for j in range(1000):
            acc += x[i, j]
            assert cs[i, j] == acc


def test_selection_margins_report_ties():
    P = np.array([[0.25, 0.25, 0.25, 0.25]])
    _, _, diag = po.select_blocks(P, 1, 0.2)
    assert diag["set_gap"][0] == 0.0       # kept and dropped blocks tie
    P = np.array([[0.5, 0.3, 0.2]])
    _, lists, diag = po.select_blocks(P, 0, 0.8)
    assert list(lists[0]) == [0, 1]
    assert diag["cdf_gap"][0] < 1e-12      # mass lands exactly on tau


_MARGIN_ROWS = {"A": [1, 3, 5, 3, 0, 2, 2, 0], "B": [6, 1, 4, 2, 3, 0, 0, 0]}


def _frac(text):
    if text == "inf":
        return math.inf
    if "/" in text:
        a, b = text.split("/")
        return float(a) / float(b)
    return float(text)


def _read_margin_golden():
    rows = []
    for line in open(os.path.join(GOLDEN, "selection_margins.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, ktau, count, sg, cg = (f.strip() for f in line.split("|"))
        k, tau = ktau.split()
        rows.append((name, int(k), float(tau), int(count), _frac(sg), _frac(cg)))
    return rows


@pytest.mark.parametrize("name,k,tau,count,set_gap,cdf_gap", _read_margin_golden())
def test_selection_margins_golden(name, k, tau, count, set_gap, cdf_gap):
    """Hand-derived decision margins (tests/golden/selection_margins.txt):
    rows where k decides the count and rows where tau does, with and without
    a mass gap below the crossing."""
    p = np.array(_MARGIN_ROWS[name], dtype=float) / 16.0
    counts, _, diag = po.select_blocks(p[None, :], k, tau)
    assert counts[0] == count
    for got, want in ((diag["set_gap"][0], set_gap), (diag["cdf_gap"][0], cdf_gap)):
        if math.isinf(want):
            assert math.isinf(got)
        else:
            assert got == pytest.approx(want, rel=1e-12, abs=1e-15)
