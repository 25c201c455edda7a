"""GPU parity of snapkv_decode_attention: one decode step's attention over a
compressed cache (the layout snapkv_compress writes) or over the packed
prefill cache.

The caches fed to the GPU are the oracle's own (its compression's out_k /
out_v) or the synthetic inputs, so the check is independent of the
compression kernels. Tolerance, from the float32 arithmetic: each weight
carries a relative error of about (|logit| + log n) * 2^-23 (below 1e-5 at
these sizes) and the weighted sum adds rounding of the same order, so
|gpu - oracle| <= 1e-4 * max |v| of the head + 1e-4 * |oracle| leaves a
tenfold margin.
"""

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
import oracle
from parity import bits_to_device
from synth import WORKLOADS, bf16_round_bits, make_custom, make_layer

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _query(batch, hq, d, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    return bf16_round_bits((rng.standard_normal((batch, hq, d)) * scale).astype(np.float32))


def _check(gpu, ref, v_rows_max, hkv):
    batch, hq, d = ref.shape
    g = hq // hkv
    for b in range(batch):
        for h in range(hkv):
            sl = slice(h * g, (h + 1) * g)
            bound = 1e-4 * v_rows_max[b][h] + 1e-4 * np.abs(ref[b, sl])
            err = np.abs(gpu[b, sl] - ref[b, sl])
            assert (err <= bound).all(), (b, h, float(err.max()), float(bound.min()))


def _compressed_case(lens, hq, hkv, d, window, budget, seed, garbage=True):
    x = make_custom(lens, hq, hkv, d, window, seed=seed)
    ref = oracle.compress(x.q_win, x.k, x.v, lens, window, 5, "avg", budget, keep_scores=False)
    n = [min(L, budget) for L in lens]
    kc, vc = ref.out_k.copy(), ref.out_v.copy()
    if garbage:  # rows past each cache length must not be read: NaN there
        for b, nb in enumerate(n):
            kc[b, :, nb:] = 0x7FC0
            vc[b, :, nb:] = 0x7FC0
    qd = _query(len(lens), hq, d, seed + 1)
    want = oracle.decode_compressed(qd, ref.out_k, ref.out_v, n)
    got = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(kc), bits_to_device(vc),
                                      n).cpu().numpy().astype(np.float64)
    vmax = [[np.abs(oracle.bf16_bits_to_f64(ref.out_v[b, h, :nb])).max() for h in range(hkv)]
            for b, nb in enumerate(n)]
    _check(got, want, vmax, hkv)
    assert np.isfinite(got).all()
    return got


CASES = [
    # lens, h_q, h_kv, d, window, budget
    ([3000], 32, 8, 128, 32, 1024),           # G = 4
    ([5000, 17, 1, 700], 8, 8, 64, 16, 256),  # MHA, D = 64, ragged, 1-row cache
    ([2000, 900], 16, 8, 128, 32, 512),       # G = 2
    ([4000], 64, 8, 128, 64, 1024),           # G = 8
    ([1500], 24, 8, 128, 16, 300),            # G = 3 (masked query slots)
    ([1200, 2500], 12, 2, 64, 16, 400),       # G = 6, D = 64
]


@needs_gpu
@pytest.mark.parametrize("case", CASES, ids=[f"case{i}" for i in range(len(CASES))])
def test_decode_over_compressed_cache(case):
    lens, hq, hkv, d, window, budget = case
    print(f"[decode] compressed {case}", flush=True)
    _compressed_case(lens, hq, hkv, d, window, budget, seed=sum(lens) % 71)


@needs_gpu
@pytest.mark.parametrize("lens", [[16384], [5000, 17, 1, 3000]])
def test_decode_over_packed_cache(lens):
    print(f"[decode] packed {lens}", flush=True)
    x = make_custom(lens, 32, 8, 128, 32, seed=len(lens))
    qd = _query(len(lens), 32, 128, 7)
    want = oracle.decode_packed(qd, x.k, x.v, lens)
    got = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(x.k),
                                      bits_to_device(x.v), lens).cpu().numpy().astype(np.float64)
    vmax, off = [], 0
    for L in lens:
        vmax.append([np.abs(oracle.bf16_bits_to_f64(x.v[off:off + L, h])).max() for h in range(8)])
        off += L
    _check(got, want, vmax, 8)


@needs_gpu
def test_decode_llama3_8b_16k_compressed_and_full():
    # the benchmark workload: the oracle's compressed cache (B = 1024) and the
    # full 16K cache, same decode queries
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    lens = x.seq_lens.tolist()
    ref = oracle.compress(x.q_win, x.k, x.v, lens, w.window, w.kernel, w.pool, w.budget,
                          keep_scores=False)
    qd = _query(1, w.h_q, w.head_dim, 8)
    n = [min(lens[0], w.budget)]
    got_c = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(ref.out_k),
                                        bits_to_device(ref.out_v), n).cpu().numpy()
    got_f = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(x.k),
                                        bits_to_device(x.v), lens).cpu().numpy()
    want_c = oracle.decode_compressed(qd, ref.out_k, ref.out_v, n)
    want_f = oracle.decode_packed(qd, x.k, x.v, lens)
    vmax = [[np.abs(oracle.bf16_bits_to_f64(x.v[:, h])).max() for h in range(w.h_kv)]]
    _check(got_c.astype(np.float64), want_c, vmax, w.h_kv)
    _check(got_f.astype(np.float64), want_f, vmax, w.h_kv)


@needs_gpu
def test_dominant_row_and_zero_query():
    # a zero query averages V; a query aligned with one key returns its V row
    lens, hq, hkv, d = [600], 8, 2, 128
    x = make_custom(lens, hq, hkv, d, 16, seed=31)
    qd = np.zeros((1, hq, d), dtype=np.uint16)
    got = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(x.k),
                                      bits_to_device(x.v), lens).cpu().numpy()
    for h in range(hkv):
        mean = oracle.bf16_bits_to_f64(x.v[:, h]).mean(axis=0)
        np.testing.assert_allclose(got[0, 4 * h:4 * h + 4], np.repeat(mean[None], 4, 0),
                                   rtol=1e-4, atol=1e-5)
    k = x.k.copy()
    k[123, :, :] = bf16_round_bits(np.full((hkv, d), 0.5, np.float32))
    qd = bf16_round_bits(np.full((1, hq, d), 2.0, np.float32))  # logit 128/sqrt(128) ~ 11.3 x 8
    got = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(k),
                                      bits_to_device(x.v), lens).cpu().numpy()
    want = oracle.decode_packed(qd, k, x.v, lens)
    for h in range(hkv):
        np.testing.assert_allclose(got[0, 4 * h:4 * h + 4], want[0, 4 * h:4 * h + 4],
                                   rtol=1e-4, atol=1e-4)


@needs_gpu
def test_decode_repeatable():
    lens = [9000, 4000]
    x = make_custom(lens, 32, 8, 128, 32, seed=33)
    qd, k, v = bits_to_device(_query(2, 32, 128, 34)), bits_to_device(x.k), bits_to_device(x.v)
    a = skv.snapkv_decode_attention(qd, k, v, lens)
    b = skv.snapkv_decode_attention(qd, k, v, lens)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


@needs_gpu
def test_decode_70b_shape_128k_packed_and_compressed():
    # G = 8 query heads per KV head over a 131K-row cache and its compression
    w = WORKLOADS["llama3_70b_128k_x80"]
    x = make_layer(w, 0)
    lens = x.seq_lens.tolist()
    print("[decode] 70b 128k", flush=True)
    qd = _query(1, w.h_q, w.head_dim, 9)
    got = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(x.k), bits_to_device(x.v),
                                      lens).cpu().numpy().astype(np.float64)
    want = oracle.decode_packed(qd, x.k, x.v, lens)
    vmax = [[np.abs(oracle.bf16_bits_to_f64(x.v[:, h])).max() for h in range(w.h_kv)]]
    _check(got, want, vmax, w.h_kv)
    # a compressed layout of B rows per head taken at fixed positions (the
    # decode step does not depend on how the rows were chosen)
    pos = np.linspace(0, lens[0] - 1, w.budget).astype(np.int64)
    kc = np.ascontiguousarray(x.k[pos].transpose(1, 0, 2))[None]
    vc = np.ascontiguousarray(x.v[pos].transpose(1, 0, 2))[None]
    got_c = skv.snapkv_decode_attention(bits_to_device(qd), bits_to_device(kc), bits_to_device(vc),
                                        [w.budget]).cpu().numpy()
    want_c = oracle.decode_compressed(qd, kc, vc, [w.budget])
    _check(got_c.astype(np.float64), want_c, vmax, w.h_kv)


FORM_CASES = [
    # (cache_lens, h_q, h_kv, d, capacity or None for the packed layout)
    ([4096] * 8, 32, 8, 128, 4096),          # 16 chunks per head, one launch
    ([1024, 1, 300, 1024], 32, 8, 128, 1024),  # one-chunk prompts written directly
    ([2048], 8, 8, 64, None),                # packed, 16 chunks
    ([1500, 100, 9], 24, 8, 128, None),      # packed, G = 3, ragged
]


def _random_cache(lens, hkv, d, capacity, seed):
    rng = np.random.default_rng(seed)
    if capacity is None:
        shape = (sum(lens), hkv, d)
    else:
        shape = (len(lens), hkv, capacity, d)
    k = bf16_round_bits(rng.standard_normal(shape).astype(np.float32) * 0.3)
    v = bf16_round_bits(rng.standard_normal(shape).astype(np.float32))
    return k, v


@needs_gpu
@pytest.mark.parametrize("case", FORM_CASES, ids=[f"form{i}" for i in range(len(FORM_CASES))])
def test_one_launch_and_two_launch_forms_give_identical_bits(case, monkeypatch):
    # the one-launch form (an item that finds every chunk done merges) folds
    # the chunks in the merge kernel's order, so both forms agree bit for bit
    lens, hq, hkv, d, cap = case
    layout = skv.SNAPKV_CACHE_PACKED if cap is None else skv.SNAPKV_CACHE_COMPRESSED
    print(f"[decode] forms {case}", flush=True)
    k, v = _random_cache(lens, hkv, d, cap, seed=len(lens) + hq)
    qd = _query(len(lens), hq, d, seed=5)
    qg, kg, vg = bits_to_device(qd), bits_to_device(k), bits_to_device(v)
    assert skv.snapkv_decode_kernels(hq, hkv, d, lens, layout, cap or 0) == 1
    one = skv.snapkv_decode_attention(qg, kg, vg, lens)
    monkeypatch.setenv("SNAPKV_NO_FUSED_DECODE", "1")
    assert skv.snapkv_decode_kernels(hq, hkv, d, lens, layout, cap or 0) == 2
    two = skv.snapkv_decode_attention(qg, kg, vg, lens)
    torch.cuda.synchronize()
    assert torch.equal(one, two)
    if cap is None:
        want = oracle.decode_packed(qd, k, v, lens)
        vmax = [[np.abs(oracle.bf16_bits_to_f64(v[sum(lens[:b]):sum(lens[:b + 1]), h])).max()
                 for h in range(hkv)] for b in range(len(lens))]
    else:
        want = oracle.decode_compressed(qd, k, v, lens)
        vmax = [[np.abs(oracle.bf16_bits_to_f64(v[b, h, :n])).max() for h in range(hkv)]
                for b, n in enumerate(lens)]
    _check(one.cpu().numpy().astype(np.float64), want, vmax, hkv)


@needs_gpu
def test_one_launch_marks_need_no_clearing_across_calls_and_shapes():
    # one workspace reused by calls of different chunk counts: each call's
    # done marks carry its own epoch, so stale marks never start a merge
    cases = [([2048] * 2, 2048), ([1024, 1024], 1024), ([1900, 200], 2048)]
    ws = torch.empty(1 << 22, dtype=torch.uint8, device="cuda")
    data = []
    for i, (lens, cap) in enumerate(cases):
        assert skv.snapkv_decode_kernels(32, 8, 128, lens, skv.SNAPKV_CACHE_COMPRESSED, cap) == 1
        k, v = _random_cache(lens, 8, 128, cap, seed=40 + i)
        q = bits_to_device(_query(len(lens), 32, 128, seed=50 + i))
        data.append((q, bits_to_device(k), bits_to_device(v), lens))
    fresh = [skv.snapkv_decode_attention(*x[:3], x[3]) for x in data]
    for _ in range(3):
        for x, want in zip(data, fresh):
            got = skv.snapkv_decode_attention(*x[:3], x[3], workspace=ws)
            torch.cuda.synchronize()
            assert torch.equal(got, want)


@needs_gpu
def test_timed_step_records_the_dispatch_events_and_gives_the_same_bits():
    lens = [1024]
    k, v = _random_cache(lens, 8, 128, 1024, seed=61)
    q = bits_to_device(_query(1, 32, 128, seed=62))
    kg, vg = bits_to_device(k), bits_to_device(v)
    plain = skv.snapkv_decode_attention(q, kg, vg, lens)
    start, stop = (torch.cuda.Event(enable_timing=True) for _ in range(2))
    start.record()
    stop.record()  # the events exist before the dispatches record them
    torch.cuda.synchronize()
    step = skv.prepare_decode(q, kg, vg, lens, events=(start, stop))
    timed = step()
    torch.cuda.synchronize()
    assert torch.equal(plain, timed)
    ms = start.elapsed_time(stop)
    assert 0.0 < ms < 10.0
