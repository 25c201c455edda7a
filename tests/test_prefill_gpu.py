"""GPU parity of snapkv_prefill_attention: causal attention of every prompt
row with each row's normaliser, and the window outputs it hands to
snapkv_compress_from_lse.

Tolerances (derived from the kernel's arithmetic): the probabilities enter
the P . V products rounded to bf16 (relative error <= 2^-9 each) while the
normaliser sums the unrounded float32 values, and each output row is rounded
once to bf16, so |out - oracle| <= 2 * 2^-9 * max_j |v_j| + 2^-9 * |oracle|
(about 0.006 of the largest |v| of the head), asserted as
3e-3 * |oracle| + 5e-3 * max |v|; the normalisers are float32 sums of
exp2 terms, asserted within 2e-5 * (1 + |lse|). Small shapes compare every
element; the 16K layer compares every window row's normaliser and a sample
of output rows, each against the oracle's attention of that row alone.
"""

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
import oracle
from parity import (bits_from_device, bits_to_device, check_index_sets, check_selected_scores,
                    check_structure_and_gather, check_topk_exact, run_gpu)
from synth import WORKLOADS, bf16_round_bits, make_custom, make_layer

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

OUT_REL, OUT_ABS_FRAC, LSE_TOL = 3e-3, 5e-3, 2e-5


def _queries(lens, hq, d, seed, q_win=None):
    """Packed queries [T, H_q, D] (bf16 bits), N(0, 1/D) with a stronger
    spread; with q_win ([batch, H_q, W, D]) the last W rows of each prompt are
    those window queries."""
    rng = np.random.default_rng(seed)
    total = sum(lens)
    q = bf16_round_bits(rng.standard_normal((total, hq, d)).astype(np.float32) * (2.0 / np.sqrt(d)))
    if q_win is not None:
        w = q_win.shape[2]
        off = 0
        for b, length in enumerate(lens):
            for i in range(w):
                t = length - w + i
                if t >= 0:
                    q[off + t] = q_win[b, :, i]
            off += length
    return q


def _check_out(got_bits, ref, v_bits, lens, hkv):
    got = oracle.bf16_bits_to_f64(got_bits)
    g = got.shape[1] // hkv
    vmax = np.zeros(got.shape[1])
    off = 0
    for length in lens:
        for q in range(got.shape[1]):
            vmax[q] = np.abs(oracle.bf16_bits_to_f64(v_bits[off:off + length, q // g])).max()
            err = np.abs(got[off:off + length, q] - ref[off:off + length, q])
            bound = OUT_REL * np.abs(ref[off:off + length, q]) + OUT_ABS_FRAC * vmax[q]
            assert (err <= bound).all(), (q, float((err / bound).max()))
        off += length


CASES = [
    # lens, h_q, h_kv, d, window
    ([1], 4, 2, 128, 8),                   # one row
    ([200], 8, 2, 128, 16),                # two items, a partial key tile
    ([300, 37, 1, 130], 8, 8, 64, 32),     # ragged, MHA, D = 64, prompts shorter than W
    ([513], 32, 4, 128, 64),               # G = 8, five items
    ([129, 64], 6, 2, 128, 20),            # G = 3
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_every_row_matches_the_oracle(case):
    lens, hq, hkv, d, window = case
    print(f"[prefill] {case}", flush=True)
    x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 61)
    q_bits = _queries(lens, hq, d, seed=sum(lens))
    out, lse_w, q_win = skv.snapkv_prefill_attention(
        bits_to_device(q_bits), bits_to_device(x.k), bits_to_device(x.v), lens, window)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle.prefill_attention(q_bits, x.k, x.v, lens)
    _check_out(bits_from_device(out), ref_out, x.v, lens, hkv)
    want = oracle.window_rows(ref_lse, lens, window)
    got = lse_w.cpu().numpy().astype(np.float64)
    np.testing.assert_array_equal(np.isnan(got), np.isnan(want))
    ok = ~np.isnan(want)
    assert (np.abs(got[ok] - want[ok]) <= LSE_TOL * (1 + np.abs(want[ok]))).all()
    # the window queries, bit for bit (zero rows before a prompt's start)
    want_q = oracle.window_rows(q_bits.astype(np.float64), lens, window)
    got_q = bits_from_device(q_win).astype(np.float64)
    np.testing.assert_array_equal(got_q[~np.isnan(want_q)], want_q[~np.isnan(want_q)])
    assert (got_q[np.isnan(want_q)] == 0).all()


@needs_gpu
def test_repeated_calls_are_bitwise_identical():
    lens = [700, 90]
    x = make_custom(lens, 8, 2, 128, 32, seed=3)
    q = bits_to_device(_queries(lens, 8, 128, seed=4))
    k, v = bits_to_device(x.k), bits_to_device(x.v)
    a = skv.snapkv_prefill_attention(q, k, v, lens, 32)
    b = skv.snapkv_prefill_attention(q, k, v, lens, 32)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta,
                           tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb)


@needs_gpu
def test_llama3_8b_16k_window_normalisers_and_sampled_rows():
    # the 16K layer with its window queries as the prompt's last rows: every
    # window row's normaliser against oracle.window_lse, and output rows
    # sampled across the prompt against the oracle's attention of that row
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    lens = x.seq_lens.tolist()
    L = lens[0]
    q_bits = _queries(lens, w.h_q, w.head_dim, seed=16, q_win=x.q_win)
    print("[prefill] llama3_8b_16k", flush=True)
    out, lse_w, q_win = skv.snapkv_prefill_attention(
        bits_to_device(q_bits), bits_to_device(x.k), bits_to_device(x.v), lens, w.window)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bits_from_device(q_win), x.q_win)
    want = oracle.window_lse(x.q_win, x.k, lens, w.window)
    got = lse_w.cpu().numpy().astype(np.float64)
    assert (np.abs(got - want) <= LSE_TOL * (1 + np.abs(want))).all()
    got_out = oracle.bf16_bits_to_f64(bits_from_device(out))
    g = w.h_q // w.h_kv
    rng = np.random.default_rng(17)
    rows = np.unique(np.concatenate([[0, 1, 127, 128, L - 1], rng.integers(0, L, 27)]))
    for q in range(0, w.h_q, 5):
        kh = oracle.bf16_bits_to_f64(x.k[:, q // g])
        vh = oracle.bf16_bits_to_f64(x.v[:, q // g])
        vmax = np.abs(vh).max()
        for i in rows.tolist():
            ref = oracle.attend(oracle.bf16_bits_to_f64(q_bits[i:i + 1, q]), kh[:i + 1], vh[:i + 1])[0]
            err = np.abs(got_out[i, q] - ref)
            assert (err <= OUT_REL * np.abs(ref) + OUT_ABS_FRAC * vmax).all(), (q, i)


@needs_gpu
@pytest.mark.parametrize("name", ["llama3_8b_16k", "tiny_mha_1k"])
def test_prefill_then_compress_from_lse(name):
    # the pipeline the normalisers are for: prefill attention hands its window
    # normalisers and window queries to snapkv_compress_from_lse; the result
    # matches the oracle's compression and, where the oracle leaves no near-tie,
    # snapkv_compress's own selection
    w = WORKLOADS[name]
    x = make_layer(w)
    lens = x.seq_lens.tolist()
    q_bits = _queries(lens, w.h_q, w.head_dim, seed=18, q_win=x.q_win)
    k, v = bits_to_device(x.k), bits_to_device(x.v)
    print(f"[prefill] then compress {name}", flush=True)
    _, lse_w, q_win = skv.snapkv_prefill_attention(bits_to_device(q_bits), k, v, lens, w.window)
    ok, ov, oi, sc = skv.snapkv_compress_with_scores(q_win, k, v, lens, w.window, w.kernel, w.pool,
                                                     w.budget, window_lse=lse_w)
    torch.cuda.synchronize()
    res = dict(out_k=bits_from_device(ok), out_v=bits_from_device(ov), out_idx=oi.cpu().numpy(),
               sel_scores=sc.cpu().numpy().astype(np.float64))
    ref = oracle.compress(x.q_win, x.k, x.v, lens, w.window, w.kernel, w.pool, w.budget)
    check_structure_and_gather(res, x, w.window, w.budget)
    check_selected_scores(res["sel_scores"], ref.pooled, lens, w.window, w.budget)
    check_topk_exact(res, lens, w.window, w.budget)
    check_index_sets(res["out_idx"], ref.pooled, lens, w.window, w.budget)
    plain = run_gpu(x, w.window, w.kernel, w.pool, w.budget)
    m = w.budget - w.window
    for b in range(len(lens)):
        for h, o in enumerate(ref.pooled[b]):
            srt = np.sort(o)[::-1]
            if srt[m - 1] - srt[m] > 1e-3 * srt[m - 1] + 1e-6 * srt[0]:
                np.testing.assert_array_equal(res["out_idx"][b, h], plain["out_idx"][b, h])
