"""GPU parity of snapkv_compress / snapkv_window_scores against the oracle.

Named workloads at their full sizes (the large stacks on sampled layers), plus
edge cases: prompts at, just over and under the budget, shorter than the
window, a one-token prefix, no pooling, kernels wider than the prefix, MHA,
head_dim 64, window rows that are not a multiple of 32, the 512-row maximum,
ragged batches mixing kept-whole and compressed prompts, and prefixes longer
than the register-resident selection (the sliced selection), with exact ties.
"""

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
from synth.device import layer_lengths
from synth import WORKLOADS, make_custom, make_layer

from parity import bits_from_device, full_check, run_gpu, upload

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")


def _named(name, layer=0):
    w = WORKLOADS[name]
    x = make_layer(w, layer)
    print(f"[parity] {name} layer {layer} lens={x.seq_lens.tolist()}", flush=True)
    return w, x


@needs_gpu
def test_tiny_mha_1k():
    w, x = _named("tiny_mha_1k")
    full_check(x, w.window, w.kernel, w.pool, w.budget)


@needs_gpu
def test_llama3_8b_16k():
    w, x = _named("llama3_8b_16k")
    full_check(x, w.window, w.kernel, w.pool, w.budget)


@needs_gpu
@pytest.mark.parametrize("layer", [0, 31])
def test_llama3_8b_32k_layers(layer):
    w, x = _named("llama3_8b_32k_x32", layer)
    full_check(x, w.window, w.kernel, w.pool, w.budget)


@needs_gpu
def test_llama3_8b_ragged8():
    w, x = _named("llama3_8b_ragged8")
    assert (x.seq_lens < w.budget).sum() == 1
    full_check(x, w.window, w.kernel, w.pool, w.budget)


@needs_gpu
def test_llama3_70b_128k_layer0():
    w, x = _named("llama3_70b_128k_x80", 0)
    full_check(x, w.window, w.kernel, w.pool, w.budget)


@needs_gpu
def test_longest_context_of_the_pages():
    # One 380,000-token prompt, the longest context the paper page reports on
    # a single 80 GB device (paper page "SnapKV: LLM Knows What You are
    # Looking for Before Generation", sections "핵심 기여도" and "주요 결과"),
    # on a Llama-3-8B-shaped layer. 47 chunks of 8192 keys per head are more
    # items than CUs (two score kernels), and the 379,968-position prefix
    # takes 93 selection slices per head (the three-kernel sliced form); the
    # last chunk, tile and slice are ragged.
    lens, hq, hkv, d, window, kernel, pool, budget = [380000], 32, 8, 128, 32, 7, "max", 4096
    print(f"[parity] longest context lens={lens}", flush=True)
    if torch.cuda.get_device_properties(0).multi_processor_count < 376:
        assert skv.snapkv_score_kernels(hq, hkv, d, lens, window, kernel) == 2
    if torch.cuda.get_device_properties(0).multi_processor_count < 744:
        assert skv.snapkv_select_kernels(hq, hkv, d, lens, window, budget) == 3
    x = make_custom(lens, hq, hkv, d, window, seed=5, planting="spans64")
    full_check(x, window, kernel, pool, budget)


EDGE = [
    # lens, h_q, h_kv, d, window, kernel, pool, budget
    ([256], 4, 2, 128, 16, 5, "avg", 256),        # L == B: kept whole
    ([257], 4, 2, 128, 16, 5, "max", 256),        # L == B + 1
    ([10], 4, 2, 128, 16, 5, "avg", 64),          # L < W
    ([17], 4, 2, 128, 16, 3, "max", 16 + 1),      # P == 1 is kept whole (L <= B)
    ([200], 4, 2, 128, 16, 1, "avg", 64),         # no pooling
    ([150], 8, 8, 64, 32, 1, "max", 48),          # MHA, D = 64, raw scores
    ([300], 4, 4, 64, 16, 13, "avg", 40),         # MHA, W = 16: 16 padded rows
    ([500], 6, 2, 128, 20, 7, "avg", 100),        # R = 60 rows
    ([700], 6, 2, 64, 24, 9, "max", 80),          # R = 72, D = 64
    ([1200], 64, 8, 128, 64, 7, "max", 300),      # R = 512 (maximum)
    ([97], 32, 8, 128, 32, 201, "avg", 60),       # kernel wider than the prefix
    ([97], 32, 8, 128, 32, 2049, "max", 60),      # widest kernel
    ([64, 300, 65, 5, 1000], 8, 2, 128, 32, 5, "avg", 96),  # ragged, mixed
    ([1, 1, 2], 4, 4, 128, 16, 5, "max", 32),     # one-token prompts
    ([40000], 8, 2, 128, 16, 7, "max", 2048),     # prefix > register-resident selection
    # a prefix past the register-resident length sends the whole call through
    # the sliced selection: short, kept-whole and one-slice prompts beside it
    ([40000, 3000, 400, 35000, 4100], 8, 2, 128, 16, 5, "avg", 512),
    ([3000, 2500], 16, 4, 128, 64, 5, "avg", 1024),
    # window rows forming 3 and 5 row tiles (G = 3 and 5, W = 32): some
    # waves hold two row tiles, so short prompts take the streaming form
    ([300], 12, 4, 128, 32, 5, "avg", 64),         # R = 96
    ([700, 90], 20, 4, 128, 32, 7, "max", 128),    # R = 160, ragged
]


@needs_gpu
@pytest.mark.parametrize("case", EDGE, ids=[f"edge{i}" for i in range(len(EDGE))])
def test_edge_cases(case):
    lens, hq, hkv, d, window, kernel, pool, budget = case
    print(f"[parity] edge {case}", flush=True)
    x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 97)
    full_check(x, window, kernel, pool, budget)


@needs_gpu
def test_no_planting_flat_scores():
    # without planted structure scores are near-uniform: many near-ties, the
    # band rule and the exact topk self-check carry the comparison
    x = make_custom([5000], 32, 8, 128, 32, seed=3, planting="none")
    full_check(x, 32, 5, "avg", 512)


@needs_gpu
@pytest.mark.parametrize("lens", [[3000, 2100], [36000, 2100]], ids=["resident", "sliced"])
@pytest.mark.parametrize("pool", ["max", "avg"])
def test_exact_ties_go_to_lowest_positions(pool, lens):
    # zero queries make every logit 0: all prefix votes are equal, so the
    # selection is decided by ties alone (lowest positions first); avg pooling
    # lowers the first and last r positions through its zero padding. A
    # prefix past the register-resident length takes the sliced selection.
    x = make_custom(lens, 16, 4, 128, 32, seed=9)
    x.q_win[:] = 0
    print(f"[parity] ties {pool} {lens}", flush=True)
    out = full_check(x, 32, 5, pool, 512)
    idx = out["res"]["out_idx"]
    m = 512 - 32
    r = 5 // 2
    for b in range(2):
        for h in range(4):
            if pool == "max":
                np.testing.assert_array_equal(idx[b, h, :m], np.arange(m))
            else:
                np.testing.assert_array_equal(idx[b, h, :m], np.arange(r, r + m))


@needs_gpu
def test_raw_scores_without_pooling_match_oracle_vote():
    import oracle
    x = make_custom([3000], 32, 8, 128, 32, seed=5)
    q, k, _ = upload(x)
    g = skv.snapkv_window_scores(q, k, [3000], 32, 1, "avg").cpu().numpy().astype(np.float64)
    for h in range(8):
        kh = oracle.bf16_bits_to_f64(x.k[:, h])
        qg = oracle.bf16_bits_to_f64(x.q_win[0, 4 * h:4 * h + 4])
        s = oracle.window_vote(qg, kh, 32)
        np.testing.assert_allclose(g[0, h], s, rtol=1e-3, atol=1e-6 * s.max())


@needs_gpu
def test_deterministic_bitwise():
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    dev = upload(x)
    a = run_gpu(x, w.window, w.kernel, w.pool, w.budget, dev)
    b = run_gpu(x, w.window, w.kernel, w.pool, w.budget, dev)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])


@needs_gpu
def test_guard_bands_untouched():
    lens = [700, 40, 333]
    hq, hkv, d, window, budget = 8, 2, 128, 32, 128
    x = make_custom(lens, hq, hkv, d, window, seed=21)
    q, k, v = upload(x)
    batch = len(lens)
    guard = 4096
    nk = batch * hkv * budget * d
    ni = batch * hkv * budget
    kbuf = torch.full((nk + 2 * guard,), 7, dtype=torch.int16, device="cuda")
    vbuf = torch.full((nk + 2 * guard,), 7, dtype=torch.int16, device="cuda")
    ibuf = torch.full((ni + 2 * guard,), 12345, dtype=torch.int32, device="cuda")
    ws_bytes = skv.snapkv_workspace_size(hq, hkv, d, lens, window)
    wbuf = torch.full((ws_bytes + 2 * guard,), 0xA5, dtype=torch.uint8, device="cuda")
    out_k = kbuf[guard:guard + nk].view(torch.bfloat16).view(batch, hkv, budget, d)
    out_v = vbuf[guard:guard + nk].view(torch.bfloat16).view(batch, hkv, budget, d)
    out_i = ibuf[guard:guard + ni].view(batch, hkv, budget)
    ws = wbuf[guard:guard + ws_bytes]
    skv.snapkv_compress(q, k, v, lens, window, 5, "avg", budget, out_k=out_k, out_v=out_v,
                        out_idx=out_i, workspace=ws)
    torch.cuda.synchronize()
    for buf, val in ((kbuf, 7), (vbuf, 7), (ibuf, 12345), (wbuf, 0xA5)):
        assert (buf[:guard] == val).all() and (buf[-guard:] == val).all()
    res = dict(out_k=bits_from_device(out_k), out_v=bits_from_device(out_v),
               out_idx=out_i.cpu().numpy())
    from parity import check_structure_and_gather
    check_structure_and_gather(res, x, window, budget)


@needs_gpu
def test_workspace_reused_across_calls_and_shapes():
    # one buffer, sized for the largest shape and never cleared, serves a
    # sequence of calls of different shapes: intermediates from one call
    # must not leak into the next
    from parity import run_gpu
    shapes = [([3000, 500], 16, 4, 128, 32, 7, "max", 256),
              ([900], 8, 8, 64, 16, 5, "avg", 128),
              ([3000, 500], 16, 4, 128, 32, 7, "max", 256),
              ([70, 2000, 40], 32, 8, 128, 64, 13, "avg", 512)]
    size = max(skv.snapkv_workspace_size(hq, hkv, d, lens, w)
               for lens, hq, hkv, d, w, *_ in shapes)
    ws = torch.full((size,), 0x5A, dtype=torch.uint8, device="cuda")
    for i, (lens, hq, hkv, d, w, kern, pool, budget) in enumerate(shapes):
        print(f"[parity] reuse call {i} {lens}", flush=True)
        x = make_custom(lens, hq, hkv, d, w, seed=40 + i)
        res = run_gpu(x, w, kern, pool, budget, workspace=ws)
        full_check(x, w, kern, pool, budget, res=res)


@pytest.mark.skip(reason="the single-launch persistent kernel (spin-waiting work items) did "
                         "not finish on its first two hardware runs (tiny MHA workload); the "
                         "cause was never established and the kernel was removed from the "
                         "library. The fused score kernels that wait on other items now do "
                         "so only when every item fits the device at once, with a bounded "
                         "spin that gives up with NaN scores (tested above)")
def test_persistent_single_launch_path():
    raise AssertionError("not enabled")


@needs_gpu
def test_validation_error_surfaces_through_binding():
    # an even pooling kernel is rejected on the host before anything is queued
    x = make_custom([100], 4, 2, 128, 8, seed=1)
    q, k, v = upload(x)
    with pytest.raises(skv.SnapKVError) as e:
        skv.snapkv_compress(q, k, v, [100], 8, 4, "avg", 32)
    assert e.value.status == skv.SNAPKV_ERR_INVALID_ARGUMENT


@needs_gpu
def test_caller_stream_is_used():
    # work enqueued on a side stream: results equal the default stream's once
    # that stream is synchronised
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    dev = upload(x)
    lens = x.seq_lens.tolist()
    ref = skv.snapkv_compress(*dev, lens, w.window, w.kernel, w.pool, w.budget)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        out = skv.snapkv_compress(*dev, lens, w.window, w.kernel, w.pool, w.budget, stream=side)
        dq = dev[0][:, :, -1].contiguous()
        dec = skv.snapkv_decode_attention(dq, out[0], out[1], [w.budget], stream=side)
    side.synchronize()
    dec_ref = skv.snapkv_decode_attention(dq, ref[0], ref[1], [w.budget])
    torch.cuda.synchronize()
    for a, b in zip(out, ref):
        assert torch.equal(a, b)
    assert torch.equal(dec, dec_ref)


@needs_gpu
def test_score_kernel_count_by_shape():
    # the 16K layer (8 heads x 32 chunks of 512 keys, one item per CU) runs
    # statistics and vote as one kernel; longer prompts, head_dim 64, wide
    # pooling and more items than CUs take the two kernels. The parity cases
    # above cover both paths, and the score export (always two kernels)
    # reproduces the fused path's selection exactly in full_check.
    w = WORKLOADS["llama3_8b_16k"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    one = cus >= 256  # every workload below has at most 256 scoring items
    fused = skv.snapkv_score_kernels(w.h_q, w.h_kv, w.head_dim, [16384], w.window, w.kernel)
    assert fused == (1 if one else 2)
    # chunks too long for LDS, head_dim 64, or a wide pooling halo: keys
    # streamed twice in one launch
    assert skv.snapkv_score_kernels(32, 8, 128, [32768], 32, 5) == (3 if one else 2)
    assert skv.snapkv_score_kernels(64, 8, 128, [131072], 64, 7) == (3 if one else 2)
    assert skv.snapkv_score_kernels(32, 8, 64, [16384], 32, 7) == (3 if one else 2)
    assert skv.snapkv_score_kernels(32, 8, 128, [16384], 32, 35) == (3 if one else 2)
    assert skv.snapkv_score_kernels(8, 8, 128, [1000], 32, 33) == 1
    # short prompts keep their keys in LDS only with one row tile per wave:
    # 128 window rows (4 row tiles) do, 96 and 160 (3 and 5) stream instead
    assert skv.snapkv_score_kernels(8, 2, 128, [300], 32, 5) == (1 if one else 2)
    assert skv.snapkv_score_kernels(12, 4, 128, [300], 32, 5) == (3 if one else 2)
    assert skv.snapkv_score_kernels(20, 4, 128, [700, 90], 32, 7) == (3 if one else 2)
    # a ragged batch: the chunk is lengthened until the (prompt, chunk, head)
    # items fit one round, so the statistics and vote run in one launch
    assert skv.snapkv_score_kernels(32, 8, 128, [20000] * 8, 64, 13) == (3 if one else 2)
    r = WORKLOADS["llama3_8b_ragged8"]
    lens = layer_lengths(r, 0)
    assert skv.snapkv_score_kernels(r.h_q, r.h_kv, r.head_dim, lens, r.window,
                                    r.kernel) == (3 if one else 2)
    # more scoring items than compute units even with the longest chunks:
    # two kernels
    assert skv.snapkv_score_kernels(32, 8, 128, [100000] * 8, 64, 13) == 2


@needs_gpu
def test_selection_inside_gather_by_shape():
    w = WORKLOADS["llama3_8b_16k"]
    cus = torch.cuda.get_device_properties(0).multi_processor_count
    got = skv.snapkv_gather_selects(w.h_q, w.h_kv, w.head_dim, [16384], w.window, w.budget)
    assert got == (1 if cus >= 256 else 0)
    # 32K layer: 64-row items (32 per head) fit the CUs
    assert skv.snapkv_gather_selects(32, 8, 128, [32768], 32, 2048) == (1 if cus >= 256 else 0)
    # a prefix past the register-resident length takes the sliced selection
    assert skv.snapkv_gather_selects(64, 8, 128, [131072], 64, 1024) == 0
    # too many gather items for the device at once
    assert skv.snapkv_gather_selects(32, 8, 128, [20000] * 8, 64, 4096) == 0
    # the selection stage's own kernels: none (inside the gather), one
    # workgroup per head, the sliced selection in one launch
    assert skv.snapkv_select_kernels(w.h_q, w.h_kv, w.head_dim, [16384], w.window,
                                     w.budget) == (0 if cus >= 256 else 1)
    assert skv.snapkv_select_kernels(32, 8, 128, [20000] * 8, 64, 4096) == 1
    assert skv.snapkv_select_kernels(64, 8, 128, [131072], 64, 1024) == (2 if cus >= 256 else 3)
    assert skv.snapkv_select_kernels(8, 2, 128, [40000], 16, 2048) == (2 if cus >= 20 else 3)


@needs_gpu
def test_select_kernels_switch_off(monkeypatch):
    # with the fused forms switched off the sliced selection takes its three
    # kernels (bit-identity of the two forms: test_fused_paths_identical_on_edge_shapes)
    monkeypatch.setenv("SNAPKV_NO_FUSED_SELECT", "1")
    assert skv.snapkv_select_kernels(64, 8, 128, [131072], 64, 1024) == 3
    assert skv.snapkv_select_kernels(32, 8, 128, [16384], 32, 1024) == 1


@needs_gpu
@pytest.mark.parametrize("name", ["llama3_8b_16k", "llama3_8b_32k_x32", "tiny_mha_1k"])
def test_fused_and_separate_paths_give_identical_bits(name, monkeypatch):
    # the same call with the fused score kernel and the selection inside the
    # gather, and with both switched off: every output bit equal
    w = WORKLOADS[name]
    x = make_layer(w)
    print(f"[parity] fused vs separate {name}", flush=True)
    dev = upload(x)
    q, k, v = dev
    lens = x.seq_lens.tolist()
    a = skv.snapkv_compress(q, k, v, lens, w.window, w.kernel, w.pool, w.budget)
    torch.cuda.synchronize()
    monkeypatch.setenv("SNAPKV_NO_FUSED_SCORE", "1")
    monkeypatch.setenv("SNAPKV_NO_FUSED_SELECT", "1")
    assert skv.snapkv_score_kernels(w.h_q, w.h_kv, w.head_dim, lens, w.window, w.kernel) == 2
    assert skv.snapkv_gather_selects(w.h_q, w.h_kv, w.head_dim, lens, w.window, w.budget) == 0
    b = skv.snapkv_compress(q, k, v, lens, w.window, w.kernel, w.pool, w.budget)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta,
                           tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb)


@needs_gpu
def test_cooperative_launch_gives_identical_bits(monkeypatch):
    # the fused score kernels launched cooperatively (runtime-guaranteed
    # co-residency) give the same bits as the ordinary launch
    w = WORKLOADS["llama3_8b_16k"]
    x = make_layer(w)
    q, k, v = upload(x)
    lens = x.seq_lens.tolist()
    print("[parity] cooperative launch 16k", flush=True)
    a = skv.snapkv_compress(q, k, v, lens, w.window, w.kernel, w.pool, w.budget)
    monkeypatch.setenv("SNAPKV_COOPERATIVE", "1")
    b = skv.snapkv_compress(q, k, v, lens, w.window, w.kernel, w.pool, w.budget)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta,
                           tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb)


GIVE_UP = [
    # (workload name or custom shape): fused resident scoring with the
    # selection in the gather (16K), fused streaming scoring (32K), and
    # prefixes past the register-resident selection, whose sliced selection
    # then recounts the first digit over the whole prefix
    "llama3_8b_16k",
    "llama3_8b_32k_x32",
    ([40000], 8, 2, 128, 16, 7, "max", 2048),
    ([70000], 8, 2, 128, 16, 5, "avg", 1024),
    # the ragged batch on the compact (prompt chunk, head) grid, one prompt
    # kept whole (no items of its own)
    "llama3_8b_ragged8",
]


@needs_gpu
@pytest.mark.parametrize("case", GIVE_UP,
                         ids=["16k", "32k", "resident_sliced", "stream_sliced", "ragged"])
def test_fused_wait_gives_up_with_identical_results(case, monkeypatch):
    # the fused score kernels' wait for the other items of a head is bounded;
    # with the bound forced to zero polls from the host, an item gives up at
    # its first look at an unset flag, computes those chunks' statistics
    # itself, and marks the head's first-digit histogram for a recount when
    # item 0's clearing was not seen. Every output bit, the selected-from
    # scores included, must equal the call in which nobody gave up, and the
    # whole result must pass the oracle comparison.
    if isinstance(case, str):
        w = WORKLOADS[case]
        x = make_layer(w)
        window, kernel, pool, budget = w.window, w.kernel, w.pool, w.budget
        hq, hkv, d = w.h_q, w.h_kv, w.head_dim
    else:
        lens, hq, hkv, d, window, kernel, pool, budget = case
        x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 71)
    lens = x.seq_lens.tolist()
    assert skv.snapkv_score_kernels(hq, hkv, d, lens, window, kernel) != 2
    dev = upload(x)
    print(f"[parity] forced give-up {lens}", flush=True)
    a = run_gpu(x, window, kernel, pool, budget, dev)
    monkeypatch.setenv("SNAPKV_SPIN_LIMIT", "0")
    b = run_gpu(x, window, kernel, pool, budget, dev)
    for key in a:
        np.testing.assert_array_equal(a[key], b[key])
    full_check(x, window, kernel, pool, budget, res=b)


@needs_gpu
@pytest.mark.parametrize("case", [EDGE[12], EDGE[9], EDGE[8], EDGE[13], EDGE[16], EDGE[10],
                                  EDGE[17], EDGE[18], EDGE[14], EDGE[15]],
                         ids=["ragged_mixed", "rows512", "d64_rows72", "one_token", "batch2_w64",
                              "wide_kernel", "rows96", "rows160", "sliced", "sliced_mixed"])
def test_fused_paths_identical_on_edge_shapes(case, monkeypatch):
    # small ragged, row-padded, head_dim-64 and one-token batches take the
    # fused forms (one-launch scoring, selection inside the gather, the
    # sliced selection of long prefixes in one launch) by default; with them
    # switched off every output bit is the same
    lens, hq, hkv, d, window, kernel, pool, budget = case
    x = make_custom(lens, hq, hkv, d, window, seed=sum(lens) % 89)
    q, k, v = upload(x)
    print(f"[parity] fused vs separate {lens} hq={hq} hkv={hkv} d={d}", flush=True)
    a = skv.snapkv_compress(q, k, v, lens, window, kernel, pool, budget)
    torch.cuda.synchronize()
    monkeypatch.setenv("SNAPKV_NO_FUSED_SCORE", "1")
    monkeypatch.setenv("SNAPKV_NO_FUSED_SELECT", "1")
    b = skv.snapkv_compress(q, k, v, lens, window, kernel, pool, budget)
    torch.cuda.synchronize()
    for ta, tb in zip(a, b):
        assert torch.equal(ta.view(torch.int16) if ta.dtype == torch.bfloat16 else ta,
                           tb.view(torch.int16) if tb.dtype == torch.bfloat16 else tb)
