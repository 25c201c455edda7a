"""CPU oracle of the compressed cache stored at 4 or 8 bits per value.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may use it.

The Scissorhands page (section "4ビット量子化との併用", and its FAQ on
quantisation) reports that cutting tokens and cutting the bit width of each
stored value are separate levers that combine: a reduced cache stored with
4-bit values kept its accuracy. The page fixes no scheme. Reading taken here
(plainest per-token form, stated once): each kept K or V row of one head
(D values) is quantised symmetrically with its own scale,

    amax  = max_d |x_d|
    inv   = 7 / amax            (float32, round to nearest even)
    code  = rint(x_d * inv)     (float32 product, ties to even), in [-7, 7]
    scale = amax / 7            (float32), so that x_d ~= code * scale

and a row of zeros has codes 0 and scale 0. Codes are two's-complement
nibbles, two per byte, the even element in the low nibble. The arithmetic is
float32 because it decides integers: the kernel and this oracle take those
decisions in the same precision (IEEE operations with round to nearest even
give the same bits everywhere).
"""

from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from .snapkv_oracle import OracleError, bf16_bits_to_f64, compress

QMAX = 7


def quantize_rows_int4(rows_bits: np.ndarray):
    """Codes (int8 [..., D], values in [-7, 7]) and scales (float32 [...]) of
    bfloat16 rows given as bit patterns (uint16 [..., D])."""
    x = bf16_bits_to_f64(rows_bits).astype(np.float32)  # exact: bf16 fits float32
    amax = np.abs(x).max(axis=-1)
    live = amax > 0
    with np.errstate(divide="ignore"):
        inv = np.where(live, np.float32(QMAX) / np.where(live, amax, np.float32(1)),
                       np.float32(0)).astype(np.float32)
    prod = (x * inv[..., None]).astype(np.float32)
    codes = np.clip(np.rint(prod), -QMAX, QMAX).astype(np.int8)
    scales = (amax / np.float32(QMAX)).astype(np.float32)
    return codes, scales


def pack_int4(codes: np.ndarray) -> np.ndarray:
    """Two's-complement nibbles, element 2i in the low half of byte i."""
    c = codes.astype(np.int16) & 0xF
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8)


def unpack_int4(packed: np.ndarray) -> np.ndarray:
    """Inverse of pack_int4 (sign-extends each nibble)."""
    lo = (packed & 0xF).astype(np.int16)
    hi = (packed >> 4).astype(np.int16)
    out = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.int16)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return np.where(out >= 8, out - 16, out).astype(np.int8)


def dequantize_int4(packed: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Values code * scale (float64) of packed rows."""
    return unpack_int4(packed).astype(np.float64) * scales.astype(np.float64)[..., None]


# ---------------------------------------------------------------- fp8 ----
# The same per-row scheme at 8 bits, in the OCP FP8 E4M3 format that
# MI355X's matrix cores consume (1 sign, 4 exponent bits with bias 7, 3
# mantissa bits; no infinities; 448 the largest finite value; subnormals
# m * 2^-9): scale = amax / 448, code = E4M3(x * (448 / amax)) with the
# product in float32 and the conversion rounding to nearest even.
FP8_MAX = 448.0


def e4m3_encode(v: np.ndarray) -> np.ndarray:
    """E4M3 bit patterns (uint8) of float32 values with |v| <= 448 * (1 + 2^-20)
    (round to nearest even; larger magnitudes are rejected)."""
    v = np.asarray(v, dtype=np.float32).astype(np.float64)  # exact
    a = np.abs(v)
    if (a > FP8_MAX * (1 + 2.0 ** -20)).any() or not np.isfinite(a).all():
        raise OracleError("value outside the E4M3 range")
    sign = (np.signbit(v)).astype(np.uint8) << 7
    out = np.zeros(v.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    # subnormals (and zero): m * 2^-9, m = 0 .. 8 (8 is the smallest normal)
    m = np.rint(a[sub] * 2.0 ** 9).astype(np.int64)
    out[sub] = np.where(m == 8, 1 << 3, m).astype(np.uint8)
    nrm = ~sub
    mant, ex = np.frexp(a[nrm])          # a = mant * 2^ex, mant in [0.5, 1)
    e = ex - 1                           # a = (2 * mant) * 2^e, 2 * mant in [1, 2)
    q = np.rint((2.0 * mant - 1.0) * 8.0).astype(np.int64)  # 3 mantissa bits, ties to even
    carry = q == 8
    q = np.where(carry, 0, q)
    e = np.where(carry, e + 1, e)
    code = ((e + 7) << 3) | q
    code = np.minimum(code, 0x7E)        # values rounding past 448 stay at 448
    out[nrm] = code.astype(np.uint8)
    return out | sign


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values (float64) of E4M3 bit patterns (NaN patterns give NaN)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(e == 0, m * 2.0 ** -9, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    val = np.where((e == 0xF) & (m == 0x7), np.nan, val)
    return sign * val


def quantize_rows_fp8(rows_bits: np.ndarray):
    """E4M3 codes (uint8 [..., D]) and scales (float32 [...]) of bfloat16 rows."""
    x = bf16_bits_to_f64(rows_bits).astype(np.float32)
    amax = np.abs(x).max(axis=-1)
    live = amax > 0
    inv = np.where(live, np.float32(FP8_MAX) / np.where(live, amax, np.float32(1)),
                   np.float32(0)).astype(np.float32)
    prod = (x * inv[..., None]).astype(np.float32)
    return e4m3_encode(prod), (amax / np.float32(FP8_MAX)).astype(np.float32)


@dataclass
class Fp8Result:
    kq: np.ndarray  # uint8 [batch, H_kv, B, D]
    ks: np.ndarray  # float32 [batch, H_kv, B]
    vq: np.ndarray
    vs: np.ndarray
    out_idx: np.ndarray


def quantize_cache_fp8(out_k_bits, out_v_bits, out_idx) -> Fp8Result:
    kc, ks = quantize_rows_fp8(out_k_bits)
    vc, vs = quantize_rows_fp8(out_v_bits)
    return Fp8Result(kc, ks, vc, vs, out_idx.copy())


@dataclass
class Int4Result:
    kq: np.ndarray  # uint8 [batch, H_kv, B, D/2]
    ks: np.ndarray  # float32 [batch, H_kv, B]
    vq: np.ndarray
    vs: np.ndarray
    out_idx: np.ndarray  # int32 [batch, H_kv, B]


def quantize_cache(out_k_bits: np.ndarray, out_v_bits: np.ndarray,
                   out_idx: np.ndarray) -> Int4Result:
    """4-bit form of a compressed cache; padding rows (all zero) quantise to
    zero codes and scale 0."""
    kc, ks = quantize_rows_int4(out_k_bits)
    vc, vs = quantize_rows_int4(out_v_bits)
    return Int4Result(pack_int4(kc), ks, pack_int4(vc), vs, out_idx.copy())


def compress_int4(q_win_bits, k_bits, v_bits, seq_lens, window, kernel, pool,
                  budget, lse=None) -> Int4Result:
    """The compression (same selection as compress) with the kept rows
    stored at 4 bits per value."""
    ref = compress(q_win_bits, k_bits, v_bits, seq_lens, window, kernel, pool,
                   budget, keep_scores=False, lse=lse)
    return quantize_cache(ref.out_k, ref.out_v, ref.out_idx)
