"""Pins of the oracle's decode (O1) and window vote (O3).

The vote is pinned against things other than its own formula: exact harmonic
sums (all-zero queries), a rank-one closed form evaluated in 50-digit
arithmetic, torch's softmax, the probability-mass identity and the GQA
replication identity.
"""

import itertools
from fractions import Fraction

import mpmath
import numpy as np
import pytest
import torch

from oracle import bf16_bits_to_f64, causal_window_probs, window_vote


def test_bf16_decode_matches_torch_for_every_pattern():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).double().numpy()
    finite = np.isfinite(ref)
    assert finite.sum() == 65536 - 2 * 128  # 2*127 NaN + 2 inf patterns
    np.testing.assert_array_equal(ours[finite], ref[finite])
    np.testing.assert_array_equal(np.isnan(ours), np.isnan(ref))


@pytest.mark.parametrize("g,w,p,d", [(1, 1, 1, 4), (1, 3, 5, 8), (4, 5, 11, 16),
                                     (2, 32, 100, 64), (8, 4, 3, 2)])
def test_zero_queries_give_harmonic_scores(g, w, p, d):
    # Q = 0: every logit is 0, row i is uniform over its P+i+1 visible keys,
    # so every prefix key gets G * sum_i 1/(P+i+1) = G * (H_L - H_P).
    rng = np.random.default_rng(0)
    k = rng.standard_normal((p + w, d))
    s = window_vote(np.zeros((g, w, d)), k, w)
    exact = g * sum(Fraction(1, p + i + 1) for i in range(w))
    np.testing.assert_allclose(s, float(exact), rtol=1e-14)
    assert s.shape == (p,)


def _rank_one_closed_form(alphas, kappa, d, w):
    """s_j for Q rows = alpha_g * e0 (all window rows of head g) and
    K_j = kappa_j * e0: row (g, i) has logits alpha_g*kappa_j/sqrt(d) for
    j <= P+i. Evaluated with 50-digit arithmetic."""
    mpmath.mp.dps = 50
    length = len(kappa)
    p = length - w
    s = [mpmath.mpf(0)] * p
    for a in alphas:
        for i in range(w):
            t = p + i
            ex = [mpmath.e ** (mpmath.mpf(a) * kappa[j] / mpmath.sqrt(d))
                  for j in range(t + 1)]
            z = mpmath.fsum(ex)
            for j in range(p):
                s[j] += ex[j] / z
    return np.array([float(x) for x in s])


@pytest.mark.parametrize("seed", range(6))
def test_rank_one_closed_form(seed):
    rng = np.random.default_rng(seed)
    d = int(rng.choice([4, 16, 64]))
    w = int(rng.integers(1, 6))
    p = int(rng.integers(1, 12))
    g = int(rng.integers(1, 4))
    kappa = rng.integers(-2, 3, size=p + w).astype(float)
    alphas = rng.uniform(-6, 6, size=g)
    q = np.zeros((g, w, d))
    k = np.zeros((p + w, d))
    q[:, :, 0] = alphas[:, None]
    k[:, 0] = kappa
    # spread the same contraction over other coordinates too: rotate e0 by a
    # random orthogonal matrix (dot products are unchanged)
    rot, _ = np.linalg.qr(rng.standard_normal((d, d)))
    s = window_vote(q @ rot, k @ rot, w)
    ref = _rank_one_closed_form(alphas, kappa, d, w)
    np.testing.assert_allclose(s, ref, rtol=1e-12, atol=1e-15)


def test_rank_one_pins_scale_and_mask():
    # A wrong 1/sqrt(D) scale, an off-by-one causal boundary or a softmax over
    # the prefix only would each move this value.
    d, w, p = 16, 2, 3
    kappa = np.array([0, 3, 0, 1, 2], dtype=float)  # keys 0..4
    q = np.zeros((1, w, d)); q[0, :, 0] = 2.0
    k = np.zeros((p + w, d)); k[:, 0] = kappa
    s = window_vote(q, k, w)
    e = np.exp(2.0 * kappa / 4.0)
    row0 = e[:4] / e[:4].sum()  # window row 0 sees keys 0..3
    row1 = e[:5] / e[:5].sum()  # window row 1 sees keys 0..4
    np.testing.assert_allclose(s, row0[:3] + row1[:3], rtol=1e-14)


@pytest.mark.parametrize("w,p,d", [(1, 1, 8), (4, 9, 8), (32, 200, 64)])
def test_rows_match_torch_softmax(w, p, d):
    rng = np.random.default_rng(w * 100 + p)
    q = rng.standard_normal((w, d)) * 2
    k = rng.standard_normal((p + w, d)) * 2
    probs = causal_window_probs(q, k, p)
    qt, kt = torch.from_numpy(q), torch.from_numpy(k)
    logits = (qt @ kt.T) / d ** 0.5
    mask = torch.arange(p + w)[None, :] > (p + torch.arange(w))[:, None]
    ref = torch.softmax(logits.masked_fill(mask, float("-inf")), dim=-1)
    np.testing.assert_allclose(probs, ref.numpy(), rtol=1e-13, atol=1e-300)
    assert (probs[mask.numpy()] == 0).all()


@pytest.mark.parametrize("g,w,p", [(1, 3, 7), (4, 32, 300), (8, 64, 65)])
def test_probability_mass_identity(g, w, p):
    # each causal row sums to 1, so prefix votes + window mass = G * W
    rng = np.random.default_rng(g + w + p)
    d = 32
    q = rng.standard_normal((g, w, d)) * 3
    k = rng.standard_normal((p + w, d)) * 3
    s = window_vote(q, k, w)
    window_mass = sum(causal_window_probs(q[i], k, p)[:, p:].sum() for i in range(g))
    np.testing.assert_allclose(s.sum() + window_mass, g * w, rtol=1e-13)
    for i in range(g):
        np.testing.assert_allclose(causal_window_probs(q[i], k, p).sum(axis=1), 1.0,
                                   rtol=1e-14)
    assert (s >= 0).all()


@pytest.mark.parametrize("g", [2, 4, 8])
def test_gqa_replication_scales_by_group(g):
    rng = np.random.default_rng(g)
    w, p, d = 8, 40, 16
    q1 = rng.standard_normal((1, w, d))
    k = rng.standard_normal((p + w, d))
    s1 = window_vote(q1, k, w)
    sg = window_vote(np.repeat(q1, g, axis=0), k, w)
    np.testing.assert_allclose(sg, g * s1, rtol=1e-13)


def test_group_sum_is_sum_of_single_heads():
    rng = np.random.default_rng(7)
    w, p, d, g = 4, 20, 8, 3
    q = rng.standard_normal((g, w, d))
    k = rng.standard_normal((p + w, d))
    parts = sum(window_vote(q[i:i + 1], k, w) for i in range(g))
    np.testing.assert_allclose(window_vote(q, k, w), parts, rtol=1e-14)


def _mp_vote(q, k, w):
    """Element-by-element 50-digit evaluation on tiny inputs."""
    mpmath.mp.dps = 50
    g, _, d = q.shape
    length = k.shape[0]
    p = length - w
    out = [mpmath.mpf(0)] * p
    for gi, i in itertools.product(range(g), range(w)):
        t = p + i
        z = [mpmath.fsum(mpmath.mpf(float(q[gi, i, e])) * mpmath.mpf(float(k[j, e]))
                         for e in range(d)) / mpmath.sqrt(d) for j in range(t + 1)]
        zmax = max(z)
        ex = [mpmath.e ** (x - zmax) for x in z]
        tot = mpmath.fsum(ex)
        for j in range(p):
            out[j] += ex[j] / tot
    return np.array([float(x) for x in out])


@pytest.mark.parametrize("seed", range(4))
def test_brute_force_tiny(seed):
    rng = np.random.default_rng(100 + seed)
    w = int(rng.integers(1, 5))
    length = int(rng.integers(w + 1, 17))
    g, d = int(rng.integers(1, 3)), 4
    q = rng.standard_normal((g, w, d)) * 2
    k = rng.standard_normal((length, d)) * 2
    np.testing.assert_allclose(window_vote(q, k, w), _mp_vote(q, k, w), rtol=1e-12)
