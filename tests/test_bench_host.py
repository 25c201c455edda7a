"""Host-side logic of bench.py that runs without a GPU: the one-GPU guard,
the algorithmic byte counts its roofline is priced with, and the rule that
counter-derived HBM traffic is reported only for the kernel sources it was
measured on."""

import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
from synth import WORKLOADS  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=60)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""  # no JSON line


def test_stage_bytes_of_the_16k_layer():
    # Q_win [32 heads, 32 rows, 128] and K [16384 keys, 8 heads, 128] in bf16,
    # K read once by the fused score kernel; the vote reads the P = L - W prefix
    w = WORKLOADS["llama3_8b_16k"]
    lens = [16384]
    sb = bench.stage_bytes(w, lens)
    q = 32 * 32 * 128 * 2
    assert sb["snapkv_score_fused"] == q + 8 * 16384 * 128 * 2 == 33816576
    assert sb["snapkv_score_stats"] == sb["snapkv_score_fused"]
    assert sb["snapkv_score_vote"] == q + 8 * (16384 - 32) * 128 * 2
    # kept rows: 1024 per head, K and V read and written, plus the index list
    gather = 4 * 8 * 1024 * 128 * 2 + 4 * 8 * 1024
    assert sb["snapkv_gather"] == gather
    assert sb["snapkv_gather_select"] == gather + 8 * (16384 - 32) * 4
    score, g = bench.algorithmic_bytes(w, lens)
    assert (score, g) == (sb["snapkv_score_fused"], gather)


def test_prompts_within_the_budget_move_only_their_rows():
    # a prompt of L <= B is kept whole: no scoring bytes, its L rows copied
    w = WORKLOADS["llama3_8b_16k"]
    score, g = bench.algorithmic_bytes(w, [w.budget, 100])
    assert score == 0
    assert g == sum(4 * w.h_kv * n * w.head_dim * 2 + 4 * w.h_kv * n for n in (w.budget, 100))
    assert bench.score_flops(w, [w.budget, 100]) == 0


def test_traffic_is_reported_only_for_the_measured_sources(monkeypatch, tmp_path):
    prof = tmp_path / "profiles"
    prof.mkdir()
    key = "llama3_8b_16k:snapkv_score_fused"
    rec = {key: {"source_hash": "abc", "hbm_bytes_per_launch": 123}}
    (prof / "traffic.json").write_text(json.dumps(rec))
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "_source_hash", lambda names: "abc")
    assert bench._traffic(key) == 123
    assert bench._traffic("llama3_8b_16k:snapkv_gather") is None
    assert bench._traffic("llama3_70b_128k_x80:snapkv_score_fused") is None
    monkeypatch.setattr(bench, "_source_hash", lambda names: "changed")
    assert bench._traffic(key) is None
    (prof / "traffic.json").unlink()
    assert bench._traffic(key) is None


def test_valu_floor_of_the_score_passes():
    # statistics over all L keys and vote over the P = L - W prefix keys, for
    # all H_q * W window rows; 16 SIMD cycles per 64 updates (fma 4, exp2 8,
    # add 4) on 1024 SIMDs at 2.4 GHz; prompts kept whole add nothing
    w = WORKLOADS["llama3_8b_16k"]
    assert bench.score_logit_updates(w, [16384]) == 32 * 32 * (16384 + 16384 - 32)
    assert bench.score_logit_updates(w, [16384, w.budget]) == bench.score_logit_updates(w, [16384])
    assert abs(bench.VALU_LOGIT_PEAK - 1024 * 2.4e9 * 64 / 16) < 1.0
    h = WORKLOADS["llama3_70b_128k_x80"]
    floor_us = bench.score_logit_updates(h, [131072]) / bench.VALU_LOGIT_PEAK * 1e6
    assert 109 < floor_us < 110


def test_headline_is_the_largest_single_gpu_workload():
    # the 70B-shaped 128K stack has the most prompt tokens per layer and is
    # priced against the matrix cores (one pass of Q_win . K^T)
    w = WORKLOADS[bench.HEADLINE]
    assert bench.HEADLINE == "llama3_70b_128k_x80" and w.layers == 80
    assert all(WORKLOADS[s].name != bench.HEADLINE for s in bench.SUBS)
    assert bench.score_flops(w, [131072]) == 2 * 64 * 64 * 128 * 131072
    assert bench.HEADLINE in bench.MFMA_BOUND


def test_cpu_baseline_splits_a_layer_into_one_job_per_kv_head():
    # the oracle's per-head work on single-head slices: together they are the
    # layer's oracle call (heads are independent)
    import numpy as np
    import oracle
    from synth import make_custom
    from synth.workloads import Workload
    w = Workload(name="t", ident=99, h_q=8, h_kv=2, head_dim=64, window=16, kernel=5,
                 pool="avg", budget=64, layers=1, batch=1, planting="points16", length=300)
    x = make_custom([300], 8, 2, 64, 16, seed=4)
    jobs = bench._head_slices(w, x)
    assert len(jobs) == 2
    full = oracle.compress(x.q_win, x.k, x.v, [300], 16, 5, "avg", 64)
    for h, (q, k, v, lens, *rest) in enumerate(jobs):
        part = oracle.compress(q, k, v, lens, *rest)
        np.testing.assert_array_equal(part.out_idx[:, 0], full.out_idx[:, h])
        np.testing.assert_array_equal(part.out_k[:, 0], full.out_k[:, h])


def test_source_hash_covers_every_kernel_source():
    # every source of the compression kernels (the decode and prefill
    # attention kernels are separate launches with no counters recorded)
    csrc = os.path.join(ROOT, "long_context_kv_snapkv_amd", "csrc")
    device_sources = {f for f in os.listdir(csrc) if f.startswith("snapkv_")
                      and f.endswith((".h", ".hip", ".cpp")) and "decode" not in f
                      and "prefill" not in f}
    missing = device_sources - set(bench.KERNEL_SOURCES)
    assert not missing, missing
