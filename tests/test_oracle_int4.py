"""Pins of the oracle's 4-bit storage of the compressed cache.

Exact grids (rows that are integer multiples of a power of two map to those
integers), ties to even, the per-row error bound, the extremes, zero rows,
the nibble layout written out by hand, and the combination with the
selection (same indices, rows quantised one by one).
"""

import numpy as np
import pytest

import oracle
from synth import bf16_round_bits, make_custom


def _bits(x):
    return bf16_round_bits(np.asarray(x, dtype=np.float32))


@pytest.mark.parametrize("e", [-20, -3, 0, 5, 40])
def test_integer_grid_maps_to_its_integers(e):
    # x_d = k_d * 2^e with k in [-7, 7] and some |k| = 7: amax = 7 * 2^e, so
    # inv = 2^-e and scale = 2^e exactly and every product is an integer
    rng = np.random.default_rng(e + 100)
    k = rng.integers(-7, 8, size=(5, 128))
    k[:, 3] = 7
    k[1, 3] = -7
    x = k.astype(np.float64) * 2.0 ** e
    codes, scales = oracle.quantize_rows_int4(_bits(x))
    np.testing.assert_array_equal(codes, k)
    np.testing.assert_array_equal(scales, np.float32(2.0 ** e))


def test_halves_round_to_even():
    # amax 7 gives inv 1: the product is the value itself
    row = np.zeros(64)
    row[:8] = [7, 2.5, 3.5, -2.5, -3.5, 0.5, -0.5, 1.5]
    codes, scales = oracle.quantize_rows_int4(_bits(row[None]))
    np.testing.assert_array_equal(codes[0, :8], [7, 2, 4, -2, -4, 0, 0, 2])
    assert scales[0] == 1.0


def test_error_bound_and_extremes_on_random_rows():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 128)) * np.exp(rng.uniform(-8, 8, size=(300, 1)))
    bits = _bits(x)
    xf = oracle.bf16_bits_to_f64(bits)
    codes, scales = oracle.quantize_rows_int4(bits)
    assert codes.min() >= -7 and codes.max() <= 7
    amax = np.abs(xf).max(axis=1)
    np.testing.assert_allclose(scales, amax / 7, rtol=2 ** -23)
    # the largest magnitude maps to +-7, and every value is within half a step
    arg = np.abs(xf).argmax(axis=1)
    np.testing.assert_array_equal(np.abs(codes[np.arange(300), arg]), 7)
    err = np.abs(xf - codes * scales.astype(np.float64)[:, None])
    assert (err <= scales[:, None] * (0.5 + 1e-5)).all()


def test_zero_rows():
    codes, scales = oracle.quantize_rows_int4(np.zeros((3, 64), dtype=np.uint16))
    assert (codes == 0).all() and (scales == 0).all()


def test_nibble_layout():
    codes = np.array([[1, -1, 7, -7, 0, -8 + 1, 3, 4]], dtype=np.int8)
    packed = oracle.pack_int4(codes)
    # byte i = low nibble of element 2i | high nibble of element 2i+1
    np.testing.assert_array_equal(packed[0], [0xF1, 0x97, 0x90, 0x43])
    np.testing.assert_array_equal(oracle.unpack_int4(packed), codes)
    rng = np.random.default_rng(2)
    c = rng.integers(-7, 8, size=(10, 128)).astype(np.int8)
    np.testing.assert_array_equal(oracle.unpack_int4(oracle.pack_int4(c)), c)


def test_compress_int4_quantises_the_selected_rows():
    x = make_custom([400, 60, 900], 8, 2, 64, 16, seed=3)
    lens = x.seq_lens.tolist()
    ref = oracle.compress(x.q_win, x.k, x.v, lens, 16, 5, "avg", 128)
    q = oracle.compress_int4(x.q_win, x.k, x.v, lens, 16, 5, "avg", 128)
    np.testing.assert_array_equal(q.out_idx, ref.out_idx)
    assert q.kq.shape == (3, 2, 128, 32) and q.ks.shape == (3, 2, 128)
    deq = oracle.dequantize_int4(q.kq, q.ks)
    kf = oracle.bf16_bits_to_f64(ref.out_k)
    assert (np.abs(deq - kf) <= q.ks[..., None] * (0.5 + 1e-5)).all()
    # padding rows of the short prompt: zero codes and zero scales
    assert (q.ks[1, :, 60:] == 0).all() and (q.kq[1, :, 60:] == 0).all()
    assert (q.vs[1, :, :60] > 0).all()
