"""The oracle's pins have teeth: each test plants one plausible mistake in an
oracle function (a wrong scale, an off-by-one causal bound, a softmax over
the prefix only, a wrong GQA mapping, pooling that divides by the in-range
count, ties to the higher position, truncating quantisation, an unscaled
decode logit, an exclusive normaliser bound, a flipped normaliser sign, a
prefill row that sees the next key, a base-2 normaliser, a strided head
mapping) and
checks that at least one of the pins fails on it. Mistakes are planted in
the oracle, on the CPU, only for the duration of one test.
"""

import numpy as np
import pytest

import oracle
import oracle.decode as odecode
import oracle.kv_quant as oquant
import oracle.snapkv_oracle as orc
import test_oracle_compress as t_compress
import test_oracle_decode as t_decode
import test_oracle_int4 as t_int4
import test_oracle_lse as t_lse
import test_oracle_pool_select as t_pool
import test_oracle_vote as t_vote


def _patch(monkeypatch, name, fn, modules):
    for m in modules:
        if hasattr(m, name):
            monkeypatch.setattr(m, name, fn)


def _caught(*checks):
    """True if at least one check raises an assertion."""
    for check in checks:
        try:
            check()
        except AssertionError:
            return True
    return False


def _probs(q_rows, k_head, prefix, scale=None, visible=None):
    w, d = q_rows.shape
    length = k_head.shape[0]
    logits = (q_rows @ k_head.T) * (1 / np.sqrt(d) if scale is None else scale(d))
    vis = (np.arange(length)[None, :] <= (prefix + np.arange(w))[:, None]) if visible is None \
        else visible(length, prefix, w)
    logits = np.where(vis, logits, -np.inf)
    e = np.exp(logits - logits.max(axis=1, keepdims=True))
    return e / e.sum(axis=1, keepdims=True)


VOTE_PINS = [
    lambda: t_vote.test_rank_one_pins_scale_and_mask(),
    lambda: t_vote.test_zero_queries_give_harmonic_scores(1, 3, 5, 8),
    lambda: t_vote.test_rows_match_torch_softmax(4, 9, 8),
    lambda: t_vote.test_brute_force_tiny(0),
]


@pytest.mark.parametrize("mutant", ["scale_1_over_d", "strict_causal", "prefix_only"])
def test_vote_mutants_are_caught(monkeypatch, mutant):
    if mutant == "scale_1_over_d":
        fn = lambda q, k, p: _probs(q, k, p, scale=lambda d: 1.0 / d)  # noqa: E731
    elif mutant == "strict_causal":
        fn = lambda q, k, p: _probs(  # noqa: E731
            q, k, p, visible=lambda n, pre, w: np.arange(n)[None, :] < (pre + np.arange(w))[:, None])
    else:
        fn = lambda q, k, p: _probs(  # noqa: E731
            q, k, p, visible=lambda n, pre, w: np.repeat((np.arange(n) < pre)[None, :], w, 0))
    _patch(monkeypatch, "causal_window_probs", fn, [orc, oracle, t_vote])
    assert _caught(*VOTE_PINS), mutant


def test_gqa_mapping_mutant_is_caught(monkeypatch):
    real = orc.prompt_scores

    def strided(q_win_bits, k_bits, offset, length, b, h_q, h_kv, window, kernel, pool,
                heads=None, lse=None):
        # query heads h, h + H_kv, ... instead of the contiguous group
        g = h_q // h_kv
        perm = np.concatenate([np.arange(h, h_q, h_kv) for h in range(h_kv)])
        assert perm.size == h_q and g >= 1
        return real(q_win_bits[:, perm], k_bits, offset, length, b, h_q, h_kv, window, kernel,
                    pool, heads=heads, lse=lse)

    _patch(monkeypatch, "prompt_scores", strided, [orc, oracle, t_compress])
    assert _caught(lambda: t_compress.test_prompt_scores_map_query_groups_to_kv_heads())


def test_pool_by_in_range_count_mutant_is_caught(monkeypatch):
    real = orc.pool_scores

    def by_count(s, kernel, pool):
        if orc.pool_code(pool) != orc.POOL_AVG:
            return real(s, kernel, pool)
        r = kernel // 2
        n = np.convolve(np.ones_like(s), np.ones(kernel), mode="same")
        return np.convolve(s, np.ones(kernel), mode="same")[: s.size] / n[: s.size] if r else s

    _patch(monkeypatch, "pool_scores", by_count, [orc, oracle, t_pool])
    assert _caught(lambda: t_pool.test_pool_matches_torch(5, 13),
                   lambda: t_pool.test_constant_input_edges(5))


def test_ties_to_higher_position_mutant_is_caught(monkeypatch):
    def high_ties(c, m):
        order = np.lexsort((-np.arange(c.size), -c))
        return np.sort(order[:m])

    _patch(monkeypatch, "select_prefix", high_ties, [orc, oracle, t_pool])
    assert _caught(lambda: t_pool.test_zero_queries_select_by_pool_edges(5),
                   lambda: t_pool.test_zero_queries_select_by_pool_edges(1))


def test_truncating_quantisation_mutant_is_caught(monkeypatch):
    def trunc(rows_bits):
        x = oracle.bf16_bits_to_f64(rows_bits).astype(np.float32)
        amax = np.abs(x).max(axis=-1)
        inv = np.where(amax > 0, np.float32(7) / np.where(amax > 0, amax, 1), 0).astype(np.float32)
        codes = np.clip(np.trunc(x * inv[..., None]), -7, 7).astype(np.int8)
        return codes, (amax / np.float32(7)).astype(np.float32)

    _patch(monkeypatch, "quantize_rows_int4", trunc, [oquant, oracle, t_int4])
    assert _caught(lambda: t_int4.test_halves_round_to_even(),
                   lambda: t_int4.test_error_bound_and_extremes_on_random_rows())


def test_unscaled_decode_mutant_is_caught(monkeypatch):
    def unscaled(q_rows, k_rows, v_rows):
        logits = q_rows @ k_rows.T
        e = np.exp(logits - logits.max(axis=1, keepdims=True))
        return (e / e.sum(axis=1, keepdims=True)) @ v_rows

    _patch(monkeypatch, "attend", unscaled, [odecode, oracle, t_decode])
    assert _caught(lambda: t_decode.test_two_rows_follow_the_logistic_weight(),
                   lambda: t_decode.test_matches_torch_sdpa_in_float64())


def test_exclusive_normaliser_bound_mutant_is_caught(monkeypatch):
    def exclusive(q_win_bits, k_bits, seq_lens, window):
        seq_lens = np.asarray(seq_lens)
        batch, h_q, w, d = q_win_bits.shape
        g = h_q // k_bits.shape[1]
        out = np.full((batch, h_q, w), np.nan)
        off = 0
        for b, length in enumerate(seq_lens.tolist()):
            p = length - window
            for q in range(h_q):
                kh = oracle.bf16_bits_to_f64(k_bits[off:off + length, q // g])
                lg = (oracle.bf16_bits_to_f64(q_win_bits[b, q]) @ kh.T) / np.sqrt(d)
                for i in range(w):
                    if p + i >= 1:
                        row = lg[i, :p + i]  # misses the row's own key
                        out[b, q, i] = row.max() + np.log(np.exp(row - row.max()).sum())
            off += length
        return out

    _patch(monkeypatch, "window_lse", exclusive, [orc, oracle, t_lse])
    assert _caught(lambda: t_lse.test_zero_operand_gives_log_of_visible_count("k"),
                   lambda: t_lse.test_brute_force_in_50_digits())


def test_flipped_normaliser_sign_mutant_is_caught(monkeypatch):
    def flipped(q_group, k_head, window, lse_group):
        length, d = k_head.shape
        prefix = length - window
        s = np.zeros(prefix)
        for q_rows, lse_rows in zip(q_group, lse_group):
            logits = (q_rows @ k_head[:prefix].T) / np.sqrt(d)
            s += np.exp(np.asarray(lse_rows)[:, None] - logits).sum(axis=0)
        return s

    _patch(monkeypatch, "window_vote_from_lse", flipped, [orc, oracle, t_lse])
    assert _caught(lambda: t_lse.test_vote_from_exact_normalisers_equals_vote(),
                   lambda: t_lse.test_shifted_normalisers_scale_the_vote())


def test_truncating_fp8_mutant_is_caught(monkeypatch):
    import test_oracle_fp8 as t_fp8
    real = oquant.e4m3_encode

    def truncating(v):
        # round toward zero: shave a quarter step before rounding to nearest
        v = np.asarray(v, dtype=np.float32)
        a = np.abs(v.astype(np.float64))
        step = np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 3)
        return real((np.sign(v) * np.maximum(a - 0.499 * step, 0)).astype(np.float32))

    _patch(monkeypatch, "e4m3_encode", truncating, [oquant, oracle, t_fp8])
    assert _caught(lambda: t_fp8.test_encoding_matches_torch_float8_e4m3fn(),
                   lambda: t_fp8.test_hand_written_encodings())


# ------------------------------------------------------------ prefill ------
import oracle.prefill as oprefill  # noqa: E402
import test_oracle_prefill as t_prefill  # noqa: E402


def _attention_mutant(kind):
    def mutant(q_rows, k_rows, v_rows):
        length, d = q_rows.shape
        scale = 1 / d if kind == "scale_1_over_d" else 1 / np.sqrt(d)
        logits = (q_rows @ k_rows.T) * scale
        bound = 1 if kind == "sees_next_key" else 0
        visible = np.arange(length)[None, :] <= np.arange(length)[:, None] + bound
        logits = np.where(visible, logits, -np.inf)
        top = logits.max(axis=1, keepdims=True)
        e = np.exp(logits - top)
        s = e.sum(axis=1, keepdims=True)
        lse = (top + np.log(s))[:, 0]
        if kind == "log2_normaliser":
            lse = lse / np.log(2.0)
        return (e / s) @ v_rows, lse
    return mutant


PREFILL_PINS = [
    lambda: t_prefill.test_matches_torch_causal_attention(40, 64),
    lambda: t_prefill.test_zero_queries_give_running_means(),
    lambda: t_prefill.test_equal_keys_give_running_means_and_shifted_normalisers(),
    lambda: t_prefill.test_brute_force_tiny(),
]


@pytest.mark.parametrize("mutant", ["scale_1_over_d", "sees_next_key", "log2_normaliser"])
def test_prefill_pins_catch(monkeypatch, mutant):
    fn = _attention_mutant(mutant)
    monkeypatch.setattr(oprefill, "causal_attention", fn)
    monkeypatch.setattr(oracle, "causal_attention", fn)
    assert _caught(*PREFILL_PINS)


def test_prefill_gqa_pin_catches_a_strided_mapping(monkeypatch):
    # head q reads KV head q % H_kv instead of q // G
    def _strided(q_bits, k_bits, v_bits, seq_lens):
        total, h_q, d = q_bits.shape
        h_kv = k_bits.shape[1]
        out = np.zeros((total, h_q, d))
        lse = np.zeros((total, h_q))
        off = 0
        for length in np.asarray(seq_lens).tolist():
            for q in range(h_q):
                o, l_ = oprefill.causal_attention(
                    oracle.bf16_bits_to_f64(q_bits[off:off + length, q]),
                    oracle.bf16_bits_to_f64(k_bits[off:off + length, q % h_kv]),
                    oracle.bf16_bits_to_f64(v_bits[off:off + length, q % h_kv]))
                out[off:off + length, q] = o
                lse[off:off + length, q] = l_
            off += length
        return out, lse

    monkeypatch.setattr(oprefill, "prefill_attention", _strided)
    monkeypatch.setattr(oracle, "prefill_attention", _strided)
    assert _caught(t_prefill.test_packed_prompts_and_gqa_mapping)
