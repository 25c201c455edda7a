"""Pins of the oracle's 8-bit (OCP FP8 E4M3) storage of the compressed cache.

The encoding is pinned against torch's float8_e4m3fn conversion (a library
special case) over values spanning the normal and subnormal ranges, by
encodings written out by hand (including ties to even and the largest
value), and by a round trip of every finite code; the row quantisation by
the position of the largest magnitude, the format's error bound and zero
rows.
"""

import numpy as np
import pytest
import torch

import oracle
from synth import bf16_round_bits, make_custom


def test_encoding_matches_torch_float8_e4m3fn():
    rng = np.random.default_rng(0)
    v = rng.standard_normal(200000) * np.exp(rng.uniform(-12, 6, 200000))
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(oracle.e4m3_encode(v), ref)


def test_hand_written_encodings():
    v = np.array([0.0, 1.0, 448.0, -2.75, 2.0 ** -9, 2.0 ** -10, 3 * 2.0 ** -10, 3.3,
                  1.0625, 1.1875, 2.0 ** -6, 416.0], dtype=np.float32)
    want = [0x00, 0x38, 0x7E, 0xC3, 0x01, 0x00, 0x02, 0x45, 0x38, 0x3A, 0x08, 0x7D]
    # 2^-10 is half the smallest subnormal: ties to even gives 0; 3 * 2^-10
    # ties to 2 * 2^-9; 1.0625 = 1 + 1/16 ties to 1.0; 1.1875 ties to 1.25
    np.testing.assert_array_equal(oracle.e4m3_encode(v), want)


def test_every_finite_code_round_trips():
    codes = np.arange(256, dtype=np.uint8)
    vals = oracle.e4m3_decode(codes)
    finite = np.isfinite(vals)
    assert finite.sum() == 254  # 0x7F and 0xFF are NaN
    np.testing.assert_array_equal(oracle.e4m3_encode(vals[finite].astype(np.float32)),
                                  codes[finite])
    assert np.nanmax(vals) == 448.0


def test_out_of_range_is_rejected():
    with pytest.raises(oracle.OracleError):
        oracle.e4m3_encode(np.array([500.0], dtype=np.float32))


def test_row_quantisation_bounds():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((300, 128)) * np.exp(rng.uniform(-8, 8, size=(300, 1)))
    bits = bf16_round_bits(x)
    xf = oracle.bf16_bits_to_f64(bits)
    codes, scales = oracle.quantize_rows_fp8(bits)
    amax = np.abs(xf).max(axis=1)
    np.testing.assert_allclose(scales, amax / 448, rtol=2 ** -23)
    arg = np.abs(xf).argmax(axis=1)
    np.testing.assert_array_equal(codes[np.arange(300), arg] & 0x7F, 0x7E)
    deq = oracle.e4m3_decode(codes) * scales.astype(np.float64)[:, None]
    # 3 mantissa bits: half a step is 2^-4 of the value in the normal range;
    # subnormals (below 2^-6 * scale) are within 2^-10 * scale
    bound = np.maximum(np.abs(xf) * 2.0 ** -4, scales[:, None] * 2.0 ** -10) * (1 + 1e-6)
    assert (np.abs(deq - xf) <= bound).all()


def test_zero_rows_and_cache_layout():
    codes, scales = oracle.quantize_rows_fp8(np.zeros((2, 64), dtype=np.uint16))
    assert (codes == 0).all() and (scales == 0).all()
    x = make_custom([300, 40], 8, 2, 64, 16, seed=2)
    ref = oracle.compress(x.q_win, x.k, x.v, x.seq_lens.tolist(), 16, 5, "max", 64)
    q = oracle.quantize_cache_fp8(ref.out_k, ref.out_v, ref.out_idx)
    assert q.kq.shape == (2, 2, 64, 64) and q.ks.shape == (2, 2, 64)
    assert (q.ks[1, :, 40:] == 0).all() and (q.kq[1, :, 40:] == 0).all()
