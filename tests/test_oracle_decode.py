"""Pins of the oracle's decode-step attention over a cache.

Closed forms (zero query or equal keys: the mean of V; two rows: the
logistic weight in 50-digit arithmetic; a dominant row), torch's
scaled_dot_product_attention in float64, the GQA head mapping, padding rows
that must not be read, and the compressed layout agreeing with the packed one
when every row is kept.
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


def test_zero_query_or_equal_keys_give_the_mean_of_v():
    rng = np.random.default_rng(0)
    v = _bits(rng.standard_normal((37, 64)))
    k = _bits(rng.standard_normal((37, 64)))
    q0 = np.zeros((3, 64))
    np.testing.assert_allclose(oracle.attend(q0, _f(k), _f(v)), np.repeat(_f(v).mean(0)[None], 3, 0),
                               rtol=1e-14, atol=1e-15)
    keq = np.repeat(_f(k)[:1], 37, axis=0)
    q = _f(_bits(rng.standard_normal((2, 64)) * 3))
    np.testing.assert_allclose(oracle.attend(q, keq, _f(v)), np.repeat(_f(v).mean(0)[None], 2, 0),
                               rtol=1e-14, atol=1e-15)


def test_two_rows_follow_the_logistic_weight():
    rng = np.random.default_rng(1)
    d = 16
    q = _f(_bits(rng.standard_normal((1, d))))
    k = _f(_bits(rng.standard_normal((2, d)) * 2))
    v = _f(_bits(rng.standard_normal((2, d))))
    mpmath.mp.dps = 50
    delta = mpmath.fsum(mpmath.mpf(float(a)) * (mpmath.mpf(float(b)) - mpmath.mpf(float(c)))
                        for a, b, c in zip(q[0], k[0], k[1])) / mpmath.sqrt(d)
    w0 = 1 / (1 + mpmath.e ** (-delta))
    want = [float(w0 * mpmath.mpf(float(a)) + (1 - w0) * mpmath.mpf(float(b)))
            for a, b in zip(v[0], v[1])]
    np.testing.assert_allclose(oracle.attend(q, k, v)[0], want, rtol=1e-13, atol=1e-15)


def test_dominant_row_takes_all_the_weight():
    rng = np.random.default_rng(2)
    d = 128
    k = rng.standard_normal((50, d)) * 0.01
    q = np.zeros((1, d))
    q[0, 7] = 8.0
    k[21, 7] = 100.0  # logit 8 * 100 / sqrt(128) ~ 70.7 above the rest
    v = rng.standard_normal((50, d))
    np.testing.assert_allclose(oracle.attend(q, k, v)[0], v[21], rtol=1e-12)


def test_matches_torch_sdpa_in_float64():
    rng = np.random.default_rng(3)
    q = _f(_bits(rng.standard_normal((4, 128))))
    k = _f(_bits(rng.standard_normal((300, 128))))
    v = _f(_bits(rng.standard_normal((300, 128))))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[:, None], torch.from_numpy(k)[None].expand(4, -1, -1),
        torch.from_numpy(v)[None].expand(4, -1, -1))[:, 0].numpy()
    np.testing.assert_allclose(oracle.attend(q, k, v), ref, rtol=1e-12, atol=1e-14)


def test_gqa_mapping_and_padding_rows():
    # V of KV head h is the constant h + 1 and queries are zero: every query
    # head of group h returns h + 1; rows past the cache length hold garbage
    batch, hq, hkv, d, cap = 2, 8, 4, 64, 20
    lens = [20, 7]
    k = np.zeros((batch, hkv, cap, d), dtype=np.uint16)
    v = np.zeros((batch, hkv, cap, d), dtype=np.float64)
    for h in range(hkv):
        v[:, h] = h + 1
    v[1, :, 7:] = 1000.0
    q = np.zeros((batch, hq, d), dtype=np.uint16)
    out = oracle.decode_compressed(q, k, _bits(v), lens)
    for qh in range(hq):
        np.testing.assert_allclose(out[:, qh], qh // 2 + 1, rtol=1e-15)


def test_compressed_layout_with_every_row_kept_equals_packed():
    x = make_custom([50, 80], 8, 2, 64, 16, seed=4)
    lens = x.seq_lens.tolist()
    ref = oracle.compress(x.q_win, x.k, x.v, lens, 16, 5, "avg", 96)  # L <= B: kept whole
    rng = np.random.default_rng(5)
    qd = _bits(rng.standard_normal((2, 8, 64)))
    a = oracle.decode_compressed(qd, ref.out_k, ref.out_v, [50, 80])
    b = oracle.decode_packed(qd, x.k, x.v, lens)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-15)


def test_empty_cache_is_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.attend(np.zeros((1, 8)), np.zeros((0, 8)), np.zeros((0, 8)))
