"""CPU oracle of the prefill attention whose by-product SnapKV reads.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite,
the smoke check and the CPU-baseline leg of the benchmark may use it.

The window scores can come out of the ordinary prefill attention at almost
no extra cost (glossary page "SnapKV(スナップケーブイ)", FAQ Q3): prefill
computes, for every prompt row, causal attention over the prompt's keys, and
a row's softmax normaliser (its log-sum-exp) is what the window vote needs.
Per prompt b (length L), query head q (KV head h = q // G) and row i:

    lse[i] = log sum_{j <= i} exp(q_i . k_j / sqrt(D))
    out[i] = sum_{j <= i} exp(q_i . k_j / sqrt(D) - lse[i]) v_j

Readings: scale 1/sqrt(D) and the causal mask j <= i, as for the window
vote; the row normaliser is reported as a natural logarithm. Computed in
float64 from the bf16 inputs; the largest logit is factored out only to keep
exp finite.
"""

from __future__ import annotations

import numpy as np

from .snapkv_oracle import OracleError, bf16_bits_to_f64


def causal_attention(q_rows: np.ndarray, k_rows: np.ndarray, v_rows: np.ndarray):
    """Causal attention of one head of one prompt: q_rows [L, D] (row i at
    position i), k_rows / v_rows [L, D]. Returns (out [L, D], lse [L])."""
    length, d = q_rows.shape
    if k_rows.shape[0] != length or v_rows.shape[0] != length:
        raise OracleError("one key and value row per query row")
    logits = (q_rows @ k_rows.T) / np.sqrt(d)
    visible = np.arange(length)[None, :] <= np.arange(length)[:, None]
    logits = np.where(visible, logits, -np.inf)
    top = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - top)
    s = e.sum(axis=1, keepdims=True)
    out = (e / s) @ v_rows
    lse = (top + np.log(s))[:, 0]
    return out, lse


def prefill_attention(q_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray, seq_lens):
    """Prefill attention of a packed batch.

    q_bits: uint16 [T, H_q, D]; k_bits, v_bits: uint16 [T, H_kv, D]; prompts
    back to back with lengths seq_lens. Returns (out float64 [T, H_q, D],
    lse float64 [T, H_q])."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    total, h_q, d = q_bits.shape
    h_kv = k_bits.shape[1]
    if h_q % h_kv or k_bits.shape != v_bits.shape or k_bits.shape[0] != total:
        raise OracleError("q, k and v shapes disagree")
    if total != int(seq_lens.sum()):
        raise OracleError("rows must equal the sum of seq_lens")
    g = h_q // h_kv
    out = np.zeros((total, h_q, d))
    lse = np.zeros((total, h_q))
    off = 0
    for length in seq_lens.tolist():
        for q in range(h_q):
            o, l_ = causal_attention(bf16_bits_to_f64(q_bits[off:off + length, q]),
                                     bf16_bits_to_f64(k_bits[off:off + length, q // g]),
                                     bf16_bits_to_f64(v_bits[off:off + length, q // g]))
            out[off:off + length, q] = o
            lse[off:off + length, q] = l_
        off += length
    return out, lse


def window_rows(x_rows: np.ndarray, seq_lens, window: int) -> np.ndarray:
    """The last `window` rows of every prompt of a packed [T, H, ...] array,
    as [batch, H, window, ...]; rows before a prompt's start are NaN."""
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    batch = seq_lens.size
    out = np.full((batch, x_rows.shape[1], window) + x_rows.shape[2:], np.nan)
    off = 0
    for b, length in enumerate(seq_lens.tolist()):
        for i in range(window):
            t = length - window + i
            if t >= 0:
                out[b, :, i] = x_rows[off + t]
        off += length
    return out
