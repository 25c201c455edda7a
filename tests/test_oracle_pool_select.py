"""Pins of the oracle's pooling (O4) and top-budget selection (O5)."""

import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import OracleError, pool_scores, select_prefix, window_vote


@pytest.mark.parametrize("kernel", [1, 3, 5, 7, 9, 13])
@pytest.mark.parametrize("p", [1, 2, 5, 13, 100])
def test_pool_matches_torch(kernel, p):
    rng = np.random.default_rng(kernel * 1000 + p)
    s = rng.exponential(size=p)
    r = kernel // 2
    st = torch.from_numpy(s)[None, None, :]
    avg = F.avg_pool1d(st, kernel, stride=1, padding=r, count_include_pad=True)
    mx = F.max_pool1d(st, kernel, stride=1, padding=r)
    np.testing.assert_allclose(pool_scores(s, kernel, "avg"), avg[0, 0].numpy(),
                               rtol=1e-15, atol=1e-300)
    np.testing.assert_array_equal(pool_scores(s, kernel, "max"), mx[0, 0].numpy())


@pytest.mark.parametrize("mode", ["avg", "max"])
def test_kernel_one_is_identity(mode):
    s = np.random.default_rng(1).exponential(size=50)
    np.testing.assert_array_equal(pool_scores(s, 1, mode), s)


@pytest.mark.parametrize("kernel", [3, 5, 13])
def test_constant_input_edges(kernel):
    # constant a: interior values a; average pooling at position j < r sees
    # r + 1 + j in-range values out of k; the far edge mirrors it
    a, p, r = 0.75, 40, kernel // 2
    c = pool_scores(np.full(p, a), kernel, "avg")
    for j in range(p):
        inside = min(j, r) + 1 + min(p - 1 - j, r)
        assert abs(c[j] - a * inside / kernel) < 1e-15
    np.testing.assert_array_equal(pool_scores(np.full(p, a), kernel, "max"), a)


def test_avg_pool_mass_identity():
    # each s_u lands in the windows of the positions within r of it that lie
    # in the prefix: sum(c) = sum_u s_u * (#such positions) / k
    rng = np.random.default_rng(3)
    p, kernel = 30, 7
    r = kernel // 2
    s = rng.exponential(size=p)
    weights = np.array([min(u, r) + 1 + min(p - 1 - u, r) for u in range(p)])
    np.testing.assert_allclose(pool_scores(s, kernel, "avg").sum(),
                               (s * weights).sum() / kernel, rtol=1e-14)


def test_max_pool_dominates_and_plateaus():
    s = np.zeros(20); s[9] = 5.0
    c = pool_scores(s, 7, "max")
    assert (c >= s).all()
    np.testing.assert_array_equal(np.flatnonzero(c == 5.0), np.arange(6, 13))


def _brute_select(c, m):
    """Maximum-sum m-subset; among equal sums the lexicographically smallest
    ascending index tuple. Exact rational sums."""
    vals = [Fraction(float(x)) for x in c]
    best, best_key = None, None
    for comb in itertools.combinations(range(len(c)), m):
        tot = sum(vals[j] for j in comb)
        key = (-tot, comb)
        if best_key is None or key < best_key:
            best_key, best = key, comb
    return np.array(best)


@pytest.mark.parametrize("seed", range(40))
def test_select_equals_subset_enumeration(seed):
    rng = np.random.default_rng(seed)
    p = int(rng.integers(2, 11))
    m = int(rng.integers(1, p))
    if seed % 2:
        c = rng.integers(0, 4, size=p).astype(float) / 4  # many ties
    else:
        c = rng.exponential(size=p)
    np.testing.assert_array_equal(select_prefix(c, m), _brute_select(c, m))


def test_select_exchange_property():
    rng = np.random.default_rng(5)
    c = rng.integers(0, 6, size=500).astype(float)
    m = 123
    sel = select_prefix(c, m)
    out = np.setdiff1d(np.arange(c.size), sel)
    assert len(sel) == m and (np.diff(sel) > 0).all()
    assert c[sel].min() >= c[out].max()
    tau = c[sel].min()
    # ties at the threshold: every tied outsider is above every tied member
    assert sel[c[sel] == tau].max() < out[c[out] == tau].min()


@pytest.mark.parametrize("kernel", [1, 5, 7])
def test_zero_queries_select_by_pool_edges(kernel):
    # Q = 0 makes every raw score identical (same row values, same order).
    # Max pooling keeps them identical -> lowest positions 0..m-1.
    # Average pooling lowers the r edge positions at each end -> r..r+m-1.
    w, p, d, m = 4, 60, 8, 20
    k = np.random.default_rng(0).standard_normal((p + w, d))
    s = window_vote(np.zeros((2, w, d)), k, w)
    assert (s == s[0]).all()
    r = kernel // 2
    np.testing.assert_array_equal(select_prefix(pool_scores(s, kernel, "max"), m),
                                  np.arange(m))
    np.testing.assert_array_equal(select_prefix(pool_scores(s, kernel, "avg"), m),
                                  np.arange(r, r + m))


def test_unknown_pool_rejected():
    with pytest.raises(OracleError):
        pool_scores(np.ones(4), 3, "median")
