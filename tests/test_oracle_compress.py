"""Whole-path invariants of the oracle (O2, O6 and the composition)."""

import numpy as np
import pytest

import oracle
from oracle import OracleError, compress, pool_scores, select_prefix, validate
from synth import WORKLOADS, make_custom, make_layer


def _run(x, w, kernel, pool, budget, **kw):
    return compress(x.q_win, x.k, x.v, x.seq_lens, w, kernel, pool, budget, **kw)


@pytest.mark.parametrize("lens,w,budget", [([40], 4, 16), ([16], 4, 16), ([17], 4, 16),
                                           ([3], 4, 16), ([5], 4, 16),
                                           ([30, 9, 16, 50], 6, 16)])
@pytest.mark.parametrize("pool", ["avg", "max"])
def test_structure(lens, w, budget, pool):
    x = make_custom(lens, h_q=4, h_kv=2, head_dim=16, window=w, seed=len(lens))
    res = _run(x, w, 5, pool, budget)
    offs = x.offsets
    for b, length in enumerate(lens):
        n = min(length, budget)
        for h in range(2):
            idx = res.out_idx[b, h]
            assert (idx[n:] == -1).all()
            valid = idx[:n]
            assert (np.diff(valid) > 0).all() and valid.min() >= 0  # unique, ascending
            assert valid.max() < length
            if length <= budget:
                np.testing.assert_array_equal(valid, np.arange(length))  # identity
            else:
                np.testing.assert_array_equal(valid[-w:], np.arange(length - w, length))
            np.testing.assert_array_equal(res.out_k[b, h, :n], x.k[offs[b] + valid, h])
            np.testing.assert_array_equal(res.out_v[b, h, :n], x.v[offs[b] + valid, h])
            assert (res.out_k[b, h, n:] == 0).all() and (res.out_v[b, h, n:] == 0).all()


def test_values_never_change_selection():
    x = make_custom([80, 64], h_q=2, h_kv=1, head_dim=8, window=8, seed=3)
    a = _run(x, 8, 5, "avg", 24)
    x.v[:] = np.random.default_rng(1).integers(0, 2**16, size=x.v.shape, dtype=np.uint16)
    b = _run(x, 8, 5, "avg", 24)
    np.testing.assert_array_equal(a.out_idx, b.out_idx)
    np.testing.assert_array_equal(a.out_k, b.out_k)


def test_ragged_batch_equals_single_prompts():
    lens = [50, 12, 90]
    x = make_custom(lens, h_q=4, h_kv=2, head_dim=8, window=5, seed=9)
    whole = _run(x, 5, 3, "max", 20)
    offs = x.offsets
    for b, length in enumerate(lens):
        sl = slice(offs[b], offs[b] + length)
        one = compress(x.q_win[b:b + 1], x.k[sl], x.v[sl], [length], 5, 3, "max", 20)
        np.testing.assert_array_equal(one.out_idx[0], whole.out_idx[b])
        np.testing.assert_array_equal(one.out_k[0], whole.out_k[b])


def test_kernel_one_means_raw_scores_select():
    x = make_custom([70], h_q=2, h_kv=2, head_dim=8, window=6, seed=4)
    res = _run(x, 6, 1, "avg", 20)
    for h in range(2):
        np.testing.assert_array_equal(res.pooled[0][h], res.raw[0][h])
        np.testing.assert_array_equal(res.out_idx[0, h, :14],
                                      select_prefix(res.raw[0][h], 14))


def test_selection_uses_pooled_scores():
    x = make_custom([120], h_q=4, h_kv=1, head_dim=8, window=8, seed=2)
    res = _run(x, 8, 7, "avg", 40)
    c = pool_scores(res.raw[0][0], 7, "avg")
    np.testing.assert_array_equal(res.pooled[0][0], c)
    np.testing.assert_array_equal(res.out_idx[0, 0, :32], select_prefix(c, 32))


def test_planted_heavy_hitters_are_kept():
    # sanity (statistical, not a parity pin): planted positions dominate
    w = WORKLOADS["tiny_mha_1k"]
    x = make_layer(w)
    res = _run(x, w.window, w.kernel, w.pool, w.budget)
    for h in range(w.h_kv):
        kept = set(res.out_idx[0, h].tolist())
        planted = set(x.planted[0][h].tolist())
        assert len(planted & kept) >= 0.9 * len(planted)


@pytest.mark.parametrize("args", [
    dict(h_q=3, h_kv=2), dict(window=0), dict(budget=8), dict(kernel=4),
    dict(kernel=0), dict(pool="median"), dict(seq_lens=[5, 0]),
])
def test_validation(args):
    base = dict(h_q=4, h_kv=2, d=8, seq_lens=[10], window=8, kernel=5,
                pool="avg", budget=16)
    base.update(args)
    with pytest.raises(OracleError):
        validate(**base)


def test_prompt_scores_map_query_groups_to_kv_heads():
    # query head q reads KV head q // G: with rank-one queries and keys each
    # KV head's raw scores follow the closed form of its own group's queries
    from test_oracle_vote import _rank_one_closed_form
    from synth import bf16_round_bits
    hq, hkv, d, length, w = 6, 3, 16, 20, 4
    g = hq // hkv
    rng = np.random.default_rng(11)
    alphas = rng.choice([-2.0, -1.0, -0.5, 0.5, 1.0, 1.5, 2.0], size=hq)
    kappa = rng.integers(-3, 4, size=(hkv, length)).astype(float)
    q = np.zeros((1, hq, w, d), dtype=np.float32)
    q[0, :, :, 0] = alphas[:, None]
    k = np.zeros((length, hkv, d), dtype=np.float32)
    k[:, :, 0] = kappa.T
    raw, _ = oracle.prompt_scores(bf16_round_bits(q), bf16_round_bits(k), 0, length, 0, hq,
                                  hkv, w, 1, "avg")
    for h in range(hkv):
        ref = _rank_one_closed_form(alphas[h * g:(h + 1) * g], kappa[h], d, w)
        np.testing.assert_allclose(raw[h], ref, rtol=1e-12, atol=1e-15)
