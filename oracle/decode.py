"""CPU oracle of one decode step's attention over a KV cache.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may use it.

After compression the decode phase attends over the kept rows only
(glossary page "SnapKV(スナップケーブイ)", section "SnapKVの仕組み", step 4;
the paper page's results report the generation speed-up at 16K input tokens
that this makes possible; the Scissorhands page notes that after eviction
attention is computed as usual over the rows that remain). One decode step,
per prompt b and query head q (KV head h = q // G):

    o[b, q] = sum_t softmax_t( q_dec[b, q] . k_t / sqrt(D) ) v_t

over the n_b cached rows t of head h. Readings: the scale is 1/sqrt(D), as
in prefill; the decode query sees every cached row (no mask); the token being
generated is not in the cache (a caller appends it before the step when it
wants it attended). Computed in float64 from the bf16 inputs.
"""

from __future__ import annotations

import numpy as np

from .snapkv_oracle import OracleError, bf16_bits_to_f64


def attend(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray) -> np.ndarray:
    """softmax(q . k / sqrt(D)) v for queries [G, D] over rows [n, D] (float64)."""
    if k_rows.shape[0] < 1:
        raise OracleError("a decode step needs at least one cached row")
    d = q_rows.shape[-1]
    logits = (q_rows @ k_rows.T) / np.sqrt(d)
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w /= w.sum(axis=1, keepdims=True)
    return w @ v_rows


def decode_compressed(q_bits: np.ndarray, out_k_bits: np.ndarray, out_v_bits: np.ndarray,
                      cache_lens) -> np.ndarray:
    """Decode attention over a compressed cache [batch, H_kv, B, D] whose
    first cache_lens[b] rows are valid. q_bits: [batch, H_q, D]. Returns
    float64 [batch, H_q, D]."""
    batch, h_q, d = q_bits.shape
    h_kv = out_k_bits.shape[1]
    g = h_q // h_kv
    out = np.zeros((batch, h_q, d))
    for b, n in enumerate(np.asarray(cache_lens).tolist()):
        for h in range(h_kv):
            k_rows = bf16_bits_to_f64(out_k_bits[b, h, :n])
            v_rows = bf16_bits_to_f64(out_v_bits[b, h, :n])
            out[b, h * g:(h + 1) * g] = attend(bf16_bits_to_f64(q_bits[b, h * g:(h + 1) * g]),
                                               k_rows, v_rows)
    return out


def decode_packed(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
                  seq_lens) -> np.ndarray:
    """Decode attention over the uncompressed cache, packed [T, H_kv, D] with
    prompts back to back (every prompt row is attended)."""
    batch, h_q, d = q_bits.shape
    h_kv = k_bits.shape[1]
    g = h_q // h_kv
    out = np.zeros((batch, h_q, d))
    off = 0
    for b, n in enumerate(np.asarray(seq_lens).tolist()):
        for h in range(h_kv):
            k_rows = bf16_bits_to_f64(k_bits[off:off + n, h])
            v_rows = bf16_bits_to_f64(v_bits[off:off + n, h])
            out[b, h * g:(h + 1) * g] = attend(bf16_bits_to_f64(q_bits[b, h * g:(h + 1) * g]),
                                               k_rows, v_rows)
        off += n
    return out
