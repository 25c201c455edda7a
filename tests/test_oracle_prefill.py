"""Pins of the oracle's prefill attention (causal attention of every prompt
row, with each row's natural-log normaliser).

torch's scaled_dot_product_attention with the causal mask and torch's
logsumexp in float64; closed forms (zero queries: the running mean of V and
log(i + 1); equal keys: the same weights with the logit added to the
normaliser; row 0: v_0); 50-digit brute force on a tiny prompt; the GQA head
mapping and packed prompts; agreement with the window normalisers
(oracle.window_lse, pinned on its own) on each prompt's last rows.
"""

import mpmath
import numpy as np
import pytest
import torch

import oracle
from synth import bf16_round_bits, make_custom


def _bits(x):
    return bf16_round_bits(np.asarray(x, dtype=np.float32))


def _f(bits):
    return oracle.bf16_bits_to_f64(bits)


@pytest.mark.parametrize("length,d", [(1, 16), (7, 16), (40, 64), (129, 128)])
def test_matches_torch_causal_attention(length, d):
    rng = np.random.default_rng(length)
    q = _f(_bits(rng.standard_normal((length, d)) / np.sqrt(d) * 3))
    k = _f(_bits(rng.standard_normal((length, d))))
    v = _f(_bits(rng.standard_normal((length, d))))
    out, lse = oracle.causal_attention(q, k, v)
    tq, tk, tv = (torch.from_numpy(a)[None, None] for a in (q, k, v))
    want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
    np.testing.assert_allclose(out, want[0, 0].numpy(), rtol=1e-12, atol=1e-13)
    logits = (torch.from_numpy(q) @ torch.from_numpy(k).T) / np.sqrt(d)
    mask = torch.ones(length, length, dtype=torch.bool).tril()
    want_lse = torch.logsumexp(logits.masked_fill(~mask, float("-inf")), dim=1)
    np.testing.assert_allclose(lse, want_lse.numpy(), rtol=1e-13, atol=1e-13)


def test_zero_queries_give_running_means():
    rng = np.random.default_rng(3)
    length, d = 50, 32
    k = _f(_bits(rng.standard_normal((length, d))))
    v = _f(_bits(rng.standard_normal((length, d))))
    out, lse = oracle.causal_attention(np.zeros((length, d)), k, v)
    running = np.cumsum(v, axis=0) / np.arange(1, length + 1)[:, None]
    np.testing.assert_allclose(out, running, rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(lse, np.log(np.arange(1, length + 1)), rtol=1e-14)


def test_equal_keys_give_running_means_and_shifted_normalisers():
    rng = np.random.default_rng(4)
    length, d = 33, 16
    krow = _f(_bits(rng.standard_normal(d)))
    k = np.repeat(krow[None], length, axis=0)
    q = _f(_bits(rng.standard_normal((length, d))))
    v = _f(_bits(rng.standard_normal((length, d))))
    out, lse = oracle.causal_attention(q, k, v)
    running = np.cumsum(v, axis=0) / np.arange(1, length + 1)[:, None]
    np.testing.assert_allclose(out, running, rtol=1e-12, atol=1e-13)
    want = np.log(np.arange(1, length + 1)) + (q @ krow) / np.sqrt(d)
    np.testing.assert_allclose(lse, want, rtol=1e-13, atol=1e-13)
    # row 0 sees key 0 only
    np.testing.assert_allclose(out[0], v[0], rtol=0, atol=0)


def test_brute_force_tiny():
    rng = np.random.default_rng(5)
    length, d = 4, 4
    q = _f(_bits(rng.standard_normal((length, d))))
    k = _f(_bits(rng.standard_normal((length, d))))
    v = _f(_bits(rng.standard_normal((length, d))))
    out, lse = oracle.causal_attention(q, k, v)
    mpmath.mp.dps = 50
    for i in range(length):
        logit = [mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b)) for a, b in zip(q[i], k[j]))
                 / mpmath.sqrt(d) for j in range(i + 1)]
        z = mpmath.fsum(mpmath.e ** x for x in logit)
        assert abs(float(mpmath.log(z)) - lse[i]) <= 1e-14 * max(1.0, abs(lse[i]))
        for c in range(d):
            o = mpmath.fsum(mpmath.e ** logit[j] / z * mpmath.mpf(float(v[j, c]))
                            for j in range(i + 1))
            assert abs(float(o) - out[i, c]) <= 1e-14


def test_packed_prompts_and_gqa_mapping():
    # two prompts, 6 query heads over 2 KV heads (G = 3): each query head
    # must use KV head q // 3 and only its own prompt's rows
    lens = [37, 20]
    x = make_custom(lens, 6, 2, 32, 8, seed=6)
    rng = np.random.default_rng(6)
    total = sum(lens)
    q_bits = _bits(rng.standard_normal((total, 6, 32)) / np.sqrt(32) * 2)
    out, lse = oracle.prefill_attention(q_bits, x.k, x.v, lens)
    off = 0
    for length in lens:
        for q in range(6):
            tq = torch.from_numpy(_f(q_bits[off:off + length, q]))[None, None]
            tk = torch.from_numpy(_f(x.k[off:off + length, q // 3]))[None, None]
            tv = torch.from_numpy(_f(x.v[off:off + length, q // 3]))[None, None]
            want = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=True)
            np.testing.assert_allclose(out[off:off + length, q], want[0, 0].numpy(), rtol=1e-12,
                                       atol=1e-13)
        off += length


def test_window_rows_agree_with_the_window_normalisers():
    lens = [90, 40, 10]
    window = 16
    x = make_custom(lens, 8, 2, 64, window, seed=7)
    rng = np.random.default_rng(7)
    total = sum(lens)
    q_bits = _bits(rng.standard_normal((total, 8, 64)) / 8)
    # the window queries of q_bits in the [batch, H_q, W, D] layout
    q_win = np.zeros((len(lens), 8, window, 64), dtype=np.uint16)
    off = 0
    for b, length in enumerate(lens):
        for i in range(window):
            t = length - window + i
            if t >= 0:
                q_win[b, :, i] = q_bits[off + t]
        off += length
    _, lse = oracle.prefill_attention(q_bits, x.k, x.v, lens)
    got = oracle.window_rows(lse, lens, window)
    want = oracle.window_lse(q_win, x.k, lens, window)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    np.testing.assert_allclose(got[~np.isnan(got)], want[~np.isnan(want)], rtol=1e-13, atol=1e-13)
    # the 10-token prompt has no rows before its start inside the window: NaN
    assert np.isnan(got[2, :, :window - 10]).all() and not np.isnan(got[2, :, window - 10:]).any()
