"""Plain fp64 CPU oracle of SnapKV's prefill-time KV-cache compression.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously-correct
definition that the GPU path is checked against. Only the test suite, the
smoke check and the CPU-baseline leg of the benchmark may import or run it;
the product path never does. It shares no code with the GPU library.

What it computes, step by step, for each prompt b (length L, window W,
budget B, pooling kernel k, GQA group G = H_q / H_kv):

O1  decode bfloat16 bit patterns exactly to float64;
O2  if L <= B the prompt already fits its budget: keep every position
    (glossary page "SnapKV", section "SnapKVの仕組み", step 3: only a budget of
    B pairs is kept, so a prompt within budget is kept whole);
O3  vote: for KV head h, every query head q in h's group and every window row
    i (absolute position t = P + i, P = L - W) take the causal attention row
    softmax_j( q . k_j / sqrt(D) ) over keys j <= t, and add its entries for
    the prefix keys j < P into s_h[j] (glossary page, "Observation Window"
    paragraph and steps 1-2: the window tokens' attention scores per head are
    aggregated; FAQ Q1: MHA and GQA models; abstract of the SnapKV paper page:
    the pattern is read from an observation window at the end of the prompt);
O3' the same vote from normalisers supplied by the caller's prefill: each
    window row's natural-log normaliser lse_i = log sum_{j <= P+i}
    exp(q_i . k_j / sqrt(D)) (window_lse), and s_h[j] as the sum of
    exp(q_i . k_j / sqrt(D) - lse_i) (window_vote_from_lse) (glossary page
    "SnapKV", FAQ Q3: the scores come out of the ordinary prefill attention
    at almost no extra cost);
O4  pool: smooth s_h along the position axis with a window of k positions,
    stride 1, same length, averaging (dividing by k, positions outside the
    prefix count as zero) or taking the in-range maximum (glossary page,
    "Pooling for Robustness"; paper page, technical approach: max or average
    pooling, kernel 5-13; limitations: pooling can be omitted, i.e. k = 1);
O5  select: the top m = B - W prefix positions by pooled score, ties to the
    lower position, reported in ascending order (glossary page, step 3; paper
    abstract: selection is made for each attention head);
O6  assemble: index list = selection followed by the window positions
    P .. L-1 (B entries), and gather those K and V rows into the compressed
    cache; rows past min(L, B) are zero with index -1 (glossary page, step 4:
    decode then runs on the compressed cache).

Readings where the pages are silent (softmax scale 1/sqrt(D), causal row
including the window's own keys, sum as the aggregation, B counting the window
rows, zero-padded pooling that divides by k, lowest-index ties) are listed in
the design notes of the repository and are marked "reading:" below.
"""

from __future__ import annotations

from dataclasses import dataclass
from typing import List, Optional

import numpy as np
from numpy.lib.stride_tricks import sliding_window_view

POOL_AVG = 0
POOL_MAX = 1
_POOL_NAMES = {"avg": POOL_AVG, "avgpool": POOL_AVG, "max": POOL_MAX,
               "maxpool": POOL_MAX}


class OracleError(ValueError):
    """Raised for arguments the method does not define."""


def pool_code(mode) -> int:
    if isinstance(mode, str):
        if mode not in _POOL_NAMES:
            raise OracleError(f"unknown pooling {mode!r}")
        return _POOL_NAMES[mode]
    if mode not in (POOL_AVG, POOL_MAX):
        raise OracleError(f"unknown pooling {mode!r}")
    return int(mode)


# ---------------------------------------------------------------- O1 decode --
def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact value of bfloat16 bit patterns: the upper half of a float32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    with np.errstate(invalid="ignore"):
        return b.view(np.float32).astype(np.float64)


# ------------------------------------------------------------ O0 validation --
def validate(h_q: int, h_kv: int, d: int, seq_lens, window: int, kernel: int,
             pool, budget: int) -> None:
    """Reject hyperparameters that the method leaves undefined."""
    if h_q < 1 or h_kv < 1 or h_q % h_kv:
        raise OracleError("query heads must be a positive multiple of KV heads")
    if d < 1:
        raise OracleError("head_dim must be positive")
    if window < 1:
        raise OracleError("window must be >= 1")
    if budget <= window:
        raise OracleError("budget must exceed the window (it includes it)")
    if kernel < 1 or kernel % 2 == 0:
        raise OracleError("pooling kernel must be odd and >= 1")
    pool_code(pool)
    lens = np.asarray(seq_lens)
    if lens.ndim != 1 or lens.size < 1 or (lens < 1).any():
        raise OracleError("every prompt needs at least one token")


# ------------------------------------------------------------------ O3 vote --
def causal_window_probs(q_rows: np.ndarray, k_head: np.ndarray,
                        prefix: int) -> np.ndarray:
    """Attention rows of the window queries over the prompt's keys.

    q_rows: [W, D] queries of window positions prefix .. prefix+W-1;
    k_head: [L, D] keys of the prompt (L = prefix + W).
    Row i attends causally to keys 0 .. prefix+i. Reading: the scale is
    1/sqrt(D), the usual prefill attention the scores come from.
    Returns [W, L] probabilities (zero where masked).
    """
    w, d = q_rows.shape
    length = k_head.shape[0]
    logits = (q_rows @ k_head.T) / np.sqrt(d)
    visible = np.arange(length)[None, :] <= (prefix + np.arange(w))[:, None]
    logits = np.where(visible, logits, -np.inf)
    row_max = logits.max(axis=1, keepdims=True)
    e = np.exp(logits - row_max)
    return e / e.sum(axis=1, keepdims=True)


def window_vote(q_group: np.ndarray, k_head: np.ndarray, window: int) -> np.ndarray:
    """Raw score s_h[j], j < P: the window rows' attention summed over rows
    and over the G query heads sharing this KV head.

    q_group: [G, W, D]; k_head: [L, D]. Reading: aggregation is a sum.
    """
    length = k_head.shape[0]
    prefix = length - window
    s = np.zeros(prefix, dtype=np.float64)
    for q_rows in q_group:
        probs = causal_window_probs(q_rows, k_head, prefix)
        s += probs[:, :prefix].sum(axis=0)
    return s


def window_vote_from_lse(q_group: np.ndarray, k_head: np.ndarray, window: int,
                         lse_group: np.ndarray) -> np.ndarray:
    """s_h[j], j < P, from normalisers the caller supplies: the sum over the G
    heads and W rows of exp(q_i . k_j / sqrt(D) - lse_i).

    lse_group: [G, W] natural-log normalisers of the window rows (what
    window_lse returns for this group). Every window row sees every prefix
    key (j < P <= P + i), so no mask enters. With the exact normalisers this
    is window_vote (glossary page "SnapKV", FAQ Q3: the scores can come out of
    the ordinary prefill attention, whose kernels keep each row's log-sum-exp).
    """
    length, d = k_head.shape
    prefix = length - window
    s = np.zeros(prefix, dtype=np.float64)
    for q_rows, lse_rows in zip(q_group, lse_group):
        logits = (q_rows @ k_head[:prefix].T) / np.sqrt(d)
        s += np.exp(logits - np.asarray(lse_rows, dtype=np.float64)[:, None]).sum(axis=0)
    return s


def window_lse(q_win_bits: np.ndarray, k_bits: np.ndarray, seq_lens,
               window: int) -> np.ndarray:
    """Natural-log softmax normaliser of every observation-window row.

    Entry [b, q, i] is log sum_{j <= P+i} exp(q . k_j / sqrt(D)) for prompt b
    (P = L_b - W), query head q against the keys of KV head q // G, window row
    i; NaN where the row's position P + i is negative (a prompt shorter than
    the window has no such query). float64 [batch, H_q, W]. This is the
    quantity a prefill flash-attention kernel keeps per row (glossary page
    "SnapKV", FAQ Q3); the maximum is factored out only to keep exp finite.
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    batch, h_q, w, d = q_win_bits.shape
    h_kv = k_bits.shape[1]
    if w != window or batch != seq_lens.size or h_q % h_kv != 0:
        raise OracleError("q_win, seq_lens and the head counts disagree")
    g = h_q // h_kv
    out = np.full((batch, h_q, w), np.nan)
    offset = 0
    for b, length in enumerate(seq_lens.tolist()):
        prefix = length - window
        rows = [i for i in range(w) if prefix + i >= 0]
        for q in range(h_q):
            k_head = bf16_bits_to_f64(k_bits[offset:offset + length, q // g, :])
            q_rows = bf16_bits_to_f64(q_win_bits[b, q])
            logits = (q_rows @ k_head.T) / np.sqrt(d)
            for i in rows:
                row = logits[i, :prefix + i + 1]
                top = row.max()
                out[b, q, i] = top + np.log(np.exp(row - top).sum())
        offset += length
    return out


# ------------------------------------------------------------------ O4 pool --
def pool_scores(s: np.ndarray, kernel: int, pool) -> np.ndarray:
    """Same-length stride-1 pooling of a score vector with kernel k.

    Reading: r = k // 2 positions of padding on both ends of the prefix
    vector. Average pooling divides the window sum by k (padding counts as
    zero); max pooling takes the maximum over in-range positions only.
    """
    mode = pool_code(pool)
    r = kernel // 2
    if mode == POOL_AVG:
        padded = np.concatenate([np.zeros(r), s, np.zeros(r)])
        return sliding_window_view(padded, kernel).sum(axis=1) / kernel
    padded = np.concatenate([np.full(r, -np.inf), s, np.full(r, -np.inf)])
    return sliding_window_view(padded, kernel).max(axis=1)


# ---------------------------------------------------------------- O5 select --
def select_prefix(c: np.ndarray, m: int) -> np.ndarray:
    """Positions of the m largest pooled scores; ties go to the lower
    position; returned ascending."""
    order = np.lexsort((np.arange(c.size), -c))  # by -c, then by position
    return np.sort(order[:m])


# -------------------------------------------------------------- O6 assemble --
def assemble_indices(length: int, window: int, budget: int,
                     selected: Optional[np.ndarray]) -> np.ndarray:
    """B-entry index list of one head: selection then window, -1 padded."""
    idx = np.full(budget, -1, dtype=np.int32)
    if length <= budget:
        idx[:length] = np.arange(length)
        return idx
    prefix = length - window
    full = np.concatenate([selected, np.arange(prefix, length)])
    assert full.size == budget
    idx[:] = full
    return idx


@dataclass
class OracleResult:
    out_k: np.ndarray  # uint16 [batch, H_kv, B, D]
    out_v: np.ndarray  # uint16 [batch, H_kv, B, D]
    out_idx: np.ndarray  # int32 [batch, H_kv, B]
    raw: List[Optional[np.ndarray]]  # per prompt: [H_kv, P] float64, or None
    pooled: List[Optional[np.ndarray]]  # per prompt: [H_kv, P] float64, or None


def prompt_scores(q_win_bits, k_bits, offset: int, length: int, b: int,
                  h_q: int, h_kv: int, window: int, kernel: int, pool,
                  heads=None, lse=None):
    """Raw and pooled scores of one prompt, per KV head ([H_kv, P]); with
    lse ([H_q, W] normalisers of this prompt) the vote uses them."""
    prefix = length - window
    g = h_q // h_kv
    heads = range(h_kv) if heads is None else heads
    raw = np.zeros((h_kv, prefix))
    pooled = np.zeros((h_kv, prefix))
    for h in heads:
        k_head = bf16_bits_to_f64(k_bits[offset:offset + length, h, :])
        q_group = bf16_bits_to_f64(q_win_bits[b, h * g:(h + 1) * g])
        if lse is None:
            raw[h] = window_vote(q_group, k_head, window)
        else:
            raw[h] = window_vote_from_lse(q_group, k_head, window, lse[h * g:(h + 1) * g])
        pooled[h] = pool_scores(raw[h], kernel, pool)
    return raw, pooled


def compress(q_win_bits: np.ndarray, k_bits: np.ndarray, v_bits: np.ndarray,
             seq_lens, window: int, kernel: int, pool, budget: int,
             keep_scores: bool = True, lse=None) -> OracleResult:
    """Whole compression of one layer.

    q_win_bits: uint16 [batch, H_q, W, D]; k_bits, v_bits: uint16 [T, H_kv, D]
    with the prompts packed back to back; seq_lens: [batch]. lse, when given,
    is [batch, H_q, W] window-row normalisers that the vote takes in place of
    its own (window_vote_from_lse).
    """
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    batch, h_q, w, d = q_win_bits.shape
    h_kv = k_bits.shape[1]
    if w != window:
        raise OracleError("q_win window dimension differs from window")
    if k_bits.shape != v_bits.shape or k_bits.shape[2] != d:
        raise OracleError("K/V shapes disagree")
    if k_bits.shape[0] != int(seq_lens.sum()) or batch != seq_lens.size:
        raise OracleError("K/V rows must equal the sum of seq_lens")
    validate(h_q, h_kv, d, seq_lens, window, kernel, pool, budget)
    m = budget - window
    out_k = np.zeros((batch, h_kv, budget, d), dtype=np.uint16)
    out_v = np.zeros((batch, h_kv, budget, d), dtype=np.uint16)
    out_idx = np.full((batch, h_kv, budget), -1, dtype=np.int32)
    raws: List[Optional[np.ndarray]] = []
    pooleds: List[Optional[np.ndarray]] = []
    offset = 0
    for b, length in enumerate(seq_lens.tolist()):
        prefix = length - window
        raw = pooled = None
        if prefix >= 1 and (length > budget or keep_scores):
            raw, pooled = prompt_scores(q_win_bits, k_bits, offset, length, b,
                                        h_q, h_kv, window, kernel, pool,
                                        lse=None if lse is None else lse[b])
        for h in range(h_kv):
            sel = select_prefix(pooled[h], m) if length > budget else None
            idx = assemble_indices(length, window, budget, sel)
            n = min(length, budget)
            out_idx[b, h] = idx
            out_k[b, h, :n] = k_bits[offset + idx[:n], h, :]
            out_v[b, h, :n] = v_bits[offset + idx[:n], h, :]
        raws.append(raw)
        pooleds.append(pooled)
        offset += length
    return OracleResult(out_k, out_v, out_idx, raws, pooleds)
