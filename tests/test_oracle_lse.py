"""Pins of the oracle's window-row normalisers and of the vote taken from
supplied normalisers (O3').

window_lse is pinned by closed forms (zero queries or keys: the log of the
visible-key count; per-head constant keys: a shifted log count that exposes
the head mapping, the scale, the causal bound and the packed offsets) and by
50-digit brute force. window_vote_from_lse is pinned against window_vote (a
different route to the same value), a single-row reduction to
causal_window_probs, and the exact effect of shifting the normalisers.
"""

import math

import mpmath
import numpy as np
import pytest

import oracle
from synth import bf16_round_bits, make_custom


def _bits(x):
    return bf16_round_bits(np.asarray(x, dtype=np.float32))


def _log_counts(lens, window):
    out = np.full((len(lens), window), np.nan)
    for b, length in enumerate(lens):
        p = length - window
        for i in range(window):
            if p + i >= 0:
                out[b, i] = math.log(p + i + 1)
    return out


@pytest.mark.parametrize("zero", ["q", "k"])
def test_zero_operand_gives_log_of_visible_count(zero):
    lens, hq, hkv, d, w = [9, 20, 3], 4, 2, 8, 5
    rng = np.random.default_rng(1)
    q = rng.standard_normal((len(lens), hq, w, d))
    k = rng.standard_normal((sum(lens), hkv, d))
    if zero == "q":
        q[:] = 0
    else:
        k[:] = 0
    lse = oracle.window_lse(_bits(q), _bits(k), lens, w)
    want = np.repeat(_log_counts(lens, w)[:, None, :], hq, axis=1)
    np.testing.assert_array_equal(np.isnan(lse), np.isnan(want))
    np.testing.assert_allclose(lse[~np.isnan(lse)], want[~np.isnan(want)], rtol=1e-15)


def test_constant_keys_shift_the_log_count_per_head_and_prompt():
    # every key of prompt b, KV head h equals u[b, h]; query head q reads KV
    # head q // G, so row i's normaliser is q_i . u[b, q // G] / sqrt(D) plus
    # the log of its P + i + 1 visible keys. Small integers keep every
    # product exact.
    lens, hq, hkv, d, w = [12, 7, 30], 6, 3, 16, 4
    g = hq // hkv
    rng = np.random.default_rng(2)
    q = rng.integers(-3, 4, size=(len(lens), hq, w, d)).astype(np.float64)
    u = rng.integers(-2, 3, size=(len(lens), hkv, d)).astype(np.float64)
    k = np.concatenate([np.repeat(u[b][None], n, axis=0) for b, n in enumerate(lens)])
    lse = oracle.window_lse(_bits(q), _bits(k), lens, w)
    counts = _log_counts(lens, w)
    for b in range(len(lens)):
        for qh in range(hq):
            dots = [sum(int(a) * int(c) for a, c in zip(q[b, qh, i], u[b, qh // g]))
                    for i in range(w)]
            want = np.array(dots) / math.sqrt(d) + counts[b]
            np.testing.assert_allclose(lse[b, qh], want, rtol=1e-14, atol=1e-14)


def test_brute_force_in_50_digits():
    lens, hq, hkv, d, w = [7, 4], 2, 1, 4, 3
    rng = np.random.default_rng(3)
    qb = _bits(rng.standard_normal((len(lens), hq, w, d)) * 2)
    kb = _bits(rng.standard_normal((sum(lens), hkv, d)) * 2)
    lse = oracle.window_lse(qb, kb, lens, w)
    q = oracle.bf16_bits_to_f64(qb)
    k = oracle.bf16_bits_to_f64(kb)
    mpmath.mp.dps = 50
    off = 0
    for b, length in enumerate(lens):
        p = length - w
        for qh in range(hq):
            for i in range(w):
                if p + i < 0:
                    assert math.isnan(lse[b, qh, i])
                    continue
                terms = []
                for j in range(p + i + 1):
                    dot = mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(c))
                                      for a, c in zip(q[b, qh, i], k[off + j, qh // (hq // hkv)]))
                    terms.append(mpmath.e ** (dot / mpmath.sqrt(d)))
                want = float(mpmath.log(mpmath.fsum(terms)))
                assert lse[b, qh, i] == pytest.approx(want, rel=1e-14, abs=1e-14)
        off += length


def _group(x, b, h, g):
    length = int(x.seq_lens[b])
    off = int(x.offsets[b])
    k_head = oracle.bf16_bits_to_f64(x.k[off:off + length, h])
    q_group = oracle.bf16_bits_to_f64(x.q_win[b, h * g:(h + 1) * g])
    return q_group, k_head


def test_vote_from_exact_normalisers_equals_vote():
    x = make_custom([300, 41], 8, 2, 64, 16, seed=4)
    lse = oracle.window_lse(x.q_win, x.k, x.seq_lens, 16)
    for b in range(2):
        for h in range(2):
            qg, kh = _group(x, b, h, 4)
            ref = oracle.window_vote(qg, kh, 16)
            got = oracle.window_vote_from_lse(qg, kh, 16, lse[b, h * 4:(h + 1) * 4])
            np.testing.assert_allclose(got, ref, rtol=1e-12)


def test_single_row_reduces_to_that_rows_probabilities():
    # normalisers of +inf silence a row; with one row left the vote is that
    # row's attention over the prefix keys
    x = make_custom([200], 1, 1, 64, 8, seed=5)
    lse = oracle.window_lse(x.q_win, x.k, x.seq_lens, 8)[0]
    qg, kh = _group(x, 0, 0, 1)
    probs = oracle.causal_window_probs(qg[0], kh, 200 - 8)
    for i in range(8):
        one = np.full_like(lse, np.inf)
        one[0, i] = lse[0, i]
        got = oracle.window_vote_from_lse(qg, kh, 8, one)
        np.testing.assert_allclose(got, probs[i, :192], rtol=1e-12)


def test_shifted_normalisers_scale_the_vote():
    x = make_custom([150], 4, 1, 128, 16, seed=6)
    lse = oracle.window_lse(x.q_win, x.k, x.seq_lens, 16)[0]
    qg, kh = _group(x, 0, 0, 4)
    base = oracle.window_vote_from_lse(qg, kh, 16, lse)
    for delta in (-2.0, 0.75, 5.0):
        got = oracle.window_vote_from_lse(qg, kh, 16, lse + delta)
        np.testing.assert_allclose(got, base * math.exp(-delta), rtol=1e-12)


def test_compress_with_own_normalisers_matches_compress():
    x = make_custom([400, 90, 700], 8, 2, 64, 16, seed=7)
    lens = x.seq_lens.tolist()
    lse = oracle.window_lse(x.q_win, x.k, lens, 16)
    a = oracle.compress(x.q_win, x.k, x.v, lens, 16, 5, "max", 64)
    b = oracle.compress(x.q_win, x.k, x.v, lens, 16, 5, "max", 64, lse=lse)
    np.testing.assert_array_equal(a.out_idx, b.out_idx)
    np.testing.assert_array_equal(a.out_k, b.out_k)
    for pa, pb in zip(a.pooled, b.pooled):
        if pa is not None:
            np.testing.assert_allclose(pb, pa, rtol=1e-12)
