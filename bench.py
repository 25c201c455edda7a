"""Throughput of SnapKV prefill-time KV-cache compression on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                    [--subs NAME,NAME|none] [--no-cpu-baseline]

A step is one snapkv_compress call (vote statistics, vote with pooling,
selection, gather: four kernels, or fewer when statistics and vote run as
one fused score kernel and the selection runs inside the gather) on one
layer of synthetic, seeded input already resident in HBM. The headline
workload is the largest single-GPU one, the 70B-shaped 80-layer stack at
L = 131072 (64 query / 8 KV heads, W = 64, maxpool 7, B = 1024): each step
compresses the next of its distinct-seed layers, so every step streams its
K from HBM. The other workloads (8B-shaped 16K layer, 32K 32-layer stack,
ragged batch of 8 prompts) are measured the same way as sub-records, each
rotating over distinct-seed layers or input variants that together exceed
the 256 MB Infinity Cache.

Prints one JSON line: value = prompt tokens compressed per second per layer
on the headline workload; `roofline` of its dominant kernel (per-kernel
durations from HIP events that each dispatch records at its kernel's start
and end, priced with the kernel's algorithmic work per launch); and
`cpu_baseline`, the fp64 CPU oracle timed on this host over a bounded sample
of the same workload, spread over worker processes one KV head per job.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0     # MI355X dense bf16 MFMA
# VALU issue floor of the score passes: every logit takes an fma, an exp2
# and an add in each pass. A gfx950 SIMD issues a wave64 fp32 fma or add
# every 4 cycles (16 lanes) and a wave64 v_exp_f32 every 8 (half rate;
# measured: 8.5 shader cycles per exp2 against 4.4 per fma), so 16 cycles
# per 64 logit updates; 256 CUs x 4 SIMDs at 2.4 GHz
VALU_LOGIT_PEAK = 256 * 4 * 2.4e9 * 64 / 16  # logit updates per second
METRIC = "prompt tokens compressed/sec per layer; achieved HBM GB/s vs MI355X peak"
CACHE_BYTES = 256 << 20       # Infinity Cache
HEADLINE = "llama3_70b_128k_x80"
SUBS = ("llama3_8b_16k", "llama3_8b_32k_x32", "llama3_8b_ragged8")
# workloads whose score kernels sit above the HBM/MFMA balance point: their
# roofline is the bf16 matrix cores (one pass of Q_win . K^T)
MFMA_BOUND = ("llama3_70b_128k_x80",)
KERNEL_SOURCES = ("snapkv_api.cpp", "snapkv_kernels.h", "snapkv_kernels.hip", "snapkv_score.h",
                  "snapkv_select.h", "snapkv_gather.h", "snapkv_device.h", "snapkv_static.hip")


def algorithmic_bytes(w, seq_lens):
    """Bytes one call must move at minimum: Q and K read once for every
    compressed prompt, the kept K/V rows read and written, the index list."""
    score = gather = 0
    for L in seq_lens:
        n = min(L, w.budget)
        if L > w.budget:
            score += w.h_q * w.window * w.head_dim * 2 + w.h_kv * L * w.head_dim * 2
        gather += 4 * w.h_kv * n * w.head_dim * 2 + 4 * w.h_kv * n
    return score, gather


def stage_bytes(w, seq_lens):
    """Algorithmic bytes of each stage kernel for one call (per launch):
    stats reads Q and all L keys; vote reads Q and the P prefix keys; the
    fused score kernels (both in one launch) read Q and all L keys once;
    select reads the P pooled scores and writes the index list; gather moves
    the kept rows (the gather term of algorithmic_bytes)."""
    d, q_bytes = w.head_dim, w.h_q * w.window * w.head_dim * 2
    gather = algorithmic_bytes(w, seq_lens)[1]
    out = {"snapkv_score_stats": 0, "snapkv_score_vote": 0, "snapkv_score_fused": 0,
           "snapkv_score_fused_stream": 0, "snapkv_select": 0, "snapkv_select_slices": 0,
           "snapkv_select_sliced": 0, "snapkv_gather": gather, "snapkv_gather_select": gather}
    for L in seq_lens:
        if L > w.budget:
            P = L - w.window
            out["snapkv_score_stats"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_fused"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_fused_stream"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_vote"] += q_bytes + w.h_kv * P * d * 2
            out["snapkv_select"] += w.h_kv * (P * 4 + w.budget * 4)
            out["snapkv_select_slices"] += w.h_kv * (P * 4 + w.budget * 4)
            out["snapkv_select_sliced"] += w.h_kv * (P * 4 + w.budget * 4)
            out["snapkv_gather_select"] += w.h_kv * P * 4  # the pooled scores, read once
    return out


def score_logit_updates(w, seq_lens):
    """Logit updates of the two score passes: every window row against all
    L keys (statistics) and against the P = L - W prefix keys (vote)."""
    rows = w.h_q * w.window
    return sum(rows * (2 * L - w.window) for L in seq_lens if L > w.budget)


def score_flops(w, seq_lens):
    """One pass of Q_win . K^T over every compressed prompt's keys."""
    return sum(2 * w.h_q * w.window * w.head_dim * L for L in seq_lens if L > w.budget)


def _source_hash(names):
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "long_context_kv_snapkv_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _traffic(kernel_key):
    """HBM bytes per launch from the committed rocprofv3 counter summary (key
    "<workload>:<kernel>"), or None when the kernel sources changed since the
    counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_hash") != _source_hash(KERNEL_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


# ------------------------------------------------------------ CPU baseline --
_JOBS = None  # per-worker copy of the sample's head slices (small layers)


def _init_worker(jobs=None):
    global _JOBS
    _JOBS = jobs
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:
        pass
    import oracle  # noqa: F401  (imported before any job is timed)


def _oracle_head_job(job):
    """One full oracle compression of one KV head (the oracle's per-head work
    on a single-KV-head slice of the layer); returns its wall time. `job` is
    the slice itself, or its index into the worker's copy."""
    import oracle
    args = _JOBS[job] if isinstance(job, int) else job
    q, k, v, lens, window, kernel, pool, budget = args
    t = time.perf_counter()
    oracle.compress(q, k, v, lens, window, kernel, pool, budget, keep_scores=False)
    return time.perf_counter() - t


def _head_slices(w, x):
    import numpy as np
    g = w.h_q // w.h_kv
    lens = x.seq_lens.tolist()
    return [(np.ascontiguousarray(x.q_win[:, h * g:(h + 1) * g]),
             np.ascontiguousarray(x.k[:, h:h + 1]), np.ascontiguousarray(x.v[:, h:h + 1]),
             lens, w.window, w.kernel, w.pool, w.budget) for h in range(w.h_kv)]


def cpu_baseline(w, cpu_seconds=12.0):
    """The oracle as it stands, timed on this host: layer 0 of the workload
    (the parity tests' input bits) split into one job per KV head, repeated
    until the sample holds about `cpu_seconds` of single-threaded work, run
    on a pool of worker processes (one BLAS thread each, up to 16, the host's
    core count permitting). Input generation, pool start-up and handing the
    inputs to the workers are outside the timed region (small layers are
    copied to every worker once; a large layer's head slices travel with
    their jobs)."""
    import multiprocessing
    from concurrent.futures import ProcessPoolExecutor

    from synth import make_layer

    x = make_layer(w, 0)
    jobs = _head_slices(w, x)
    host_cores = len(os.sched_getaffinity(0))
    workers = max(1, min(16, host_cores))
    tokens = int(x.seq_lens.sum())
    layer_bytes = x.q_win.nbytes + x.k.nbytes + x.v.nbytes
    resident = layer_bytes <= (64 << 20)
    with ProcessPoolExecutor(max_workers=workers, mp_context=multiprocessing.get_context("spawn"),
                             initializer=_init_worker,
                             initargs=(jobs if resident else None,)) as ex:
        ids = list(range(len(jobs))) if resident else jobs
        # warm-up: every worker started and through one job; a second round
        # sizes the sample
        list(ex.map(_oracle_head_job, [ids[0]] * workers))
        t_head = min(ex.map(_oracle_head_job, [ids[0]] * workers))
        reps = max(1, int(round(cpu_seconds / (t_head * len(jobs)))))
        sample = ids * reps
        t0 = time.perf_counter()
        busy = sum(ex.map(_oracle_head_job, sample))
        wall = time.perf_counter() - t0
    used = min(workers, len(sample))
    return {"value": round(reps * tokens / wall, 1), "unit": "tokens/s/layer", "cores": used,
            "kind": "oracle",
            "sample": f"{w.name} layer 0 ({tokens} tokens): {reps} x {len(jobs)} one-KV-head "
                      f"full oracle calls ({reps} layer(s) of work, {busy:.1f} s of CPU) in "
                      f"{wall:.2f} s on {used} worker processes",
            "host_cores": host_cores, "blas_threads_per_worker": 1}


# ----------------------------------------------------------------- GPU ------
def _input_sets(w, steps, warmup, dev):
    """Distinct-seed inputs for the rotation: the stack's own layers when it
    has several, else variants of its one layer; at least enough to exceed
    four times the Infinity Cache, and for the stacks one layer per step up to
    all of them."""
    import torch  # noqa: F401

    from synth.device import layer_lengths, make_layer_device

    lens = layer_lengths(w, 0)
    kv_bytes = 2 * sum(lens) * w.h_kv * w.head_dim * 2
    need = max(2, -(-4 * CACHE_BYTES // kv_bytes))
    if w.layers > 1:
        n = min(w.layers, max(need, steps + warmup))
        return [make_layer_device(w, layer, dev) for layer in range(n)], "layers"
    n = min(64, need)
    return [make_layer_device(w, 0, dev, variant=i) for i in range(n)], "variants"


def measure(w, args, dev, stream, extras=False):
    import numpy as np
    import torch

    import long_context_kv_snapkv_amd as skv

    sets, kind = _input_sets(w, args.steps, args.warmup, dev)
    batch, hkv, d, B = len(sets[0][3]), w.h_kv, w.head_dim, w.budget
    outs = [(torch.empty((batch, hkv, B, d), dtype=torch.bfloat16, device=dev),
             torch.empty((batch, hkv, B, d), dtype=torch.bfloat16, device=dev),
             torch.empty((batch, hkv, B), dtype=torch.int32, device=dev)) for _ in range(2)]
    ws = skv.new_workspace(w.h_q, hkv, d, sets[0][3], w.window, dev)
    nsets = len(sets)

    def step(i, staged=False, events=None):
        q, k, v, lens = sets[i % nsets]
        ok, ov, oi = outs[i % 2]
        skv.snapkv_compress(q, k, v, lens, w.window, w.kernel, w.pool, B, out_k=ok, out_v=ov,
                            out_idx=oi, workspace=ws, stream=stream, staged=staged,
                            stage_events=events)

    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)

    def timed(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            fn(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        return t_start.elapsed_time(t_end) / args.steps

    ms_step = timed(step)

    # per-kernel durations: snapkv_compress_staged has each stage's dispatch
    # record the caller's events at its kernel's start and end
    nprof = min(args.steps, 200)
    nst = skv.SNAPKV_NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)] for _ in range(nprof)]
    for row in evs:  # materialise the HIP events before handing them over
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(nprof):
        step(i, staged=True, events=evs[i])
    torch.cuda.synchronize()
    lens0 = sets[0][3]
    score_kernels = skv.snapkv_score_kernels(w.h_q, hkv, d, lens0, w.window, w.kernel)
    fused = score_kernels != 2
    fused_name = "snapkv_score_fused" if score_kernels == 1 else "snapkv_score_fused_stream"
    sel_in_gather = skv.snapkv_gather_selects(w.h_q, hkv, d, lens0, w.window, B) == 1
    select_kernels = skv.snapkv_select_kernels(w.h_q, hkv, d, lens0, w.window, B)
    stage_ms = {}
    for s_ in range(nst):
        if (fused and s_ == 1) or (sel_in_gather and s_ == 2):
            continue
        vals = [row[2 * s_].elapsed_time(row[2 * s_ + 1]) for row in evs]
        name = skv.snapkv_stage_name(s_)
        if fused and s_ == 0:
            name = fused_name
        if sel_in_gather and s_ == 3:
            name = "snapkv_gather_select"
        if s_ == 2:  # the selection stage's own kernel(s)
            name = {2: "snapkv_select_slices", 3: "snapkv_select_sliced"}.get(select_kernels, name)
        stage_ms[name] = float(np.mean(vals))

    sbytes = stage_bytes(w, lens0)
    dominant = max(stage_ms, key=stage_ms.get)
    kernel_ms = stage_ms[dominant]
    score_b, gather_b = algorithmic_bytes(w, lens0)
    total_b = score_b + gather_b
    flops = score_flops(w, lens0)
    score_ms = (stage_ms[fused_name] if fused else
                stage_ms["snapkv_score_stats"] + stage_ms["snapkv_score_vote"])
    hbm_gbps = sbytes[dominant] / (kernel_ms * 1e-3) / 1e9
    traffic = _traffic(f"{w.name}:{dominant}")
    if w.name in MFMA_BOUND and dominant in (fused_name, "snapkv_score_stats",
                                             "snapkv_score_vote"):
        tflops = flops / (kernel_ms * 1e-3) / 1e12
        roofline = {"kernel": dominant, "bound": "mfma", "achieved": round(tflops, 1),
                    "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": round(tflops / BF16_PEAK_TFLOPS, 4), "traffic": traffic,
                    "flops_per_launch": flops, "bytes_per_launch": sbytes[dominant],
                    "launch_ms": round(kernel_ms, 5), "hbm_gbps": round(hbm_gbps, 1),
                    "hbm_frac": round(hbm_gbps / HBM_PEAK_GBPS, 4)}
    else:
        roofline = {"kernel": dominant, "bound": "hbm", "achieved": round(hbm_gbps, 1),
                    "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                    "frac": round(hbm_gbps / HBM_PEAK_GBPS, 4), "traffic": traffic,
                    "bytes_per_launch": sbytes[dominant], "launch_ms": round(kernel_ms, 5)}
    tokens = sum(lens0)
    rec = {
        "value": round(tokens / (ms_step * 1e-3), 1), "unit": "tokens/s/layer",
        "ms_per_step": round(ms_step, 5),
        "config": {"workload": w.name, "batch": batch,
                   "seq_len": lens0 if batch > 1 else lens0[0],
                   "num_q_heads": w.h_q, "num_kv_heads": hkv, "head_dim": d,
                   "window": w.window, "kernel_size": w.kernel, "pooling": w.pool + "pool",
                   "budget": B, "layers": w.layers,
                   "rotating_inputs": f"{nsets} distinct-seed {kind}"},
        "hbm_gbps_whole_call": round(total_b / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac_whole_call": round(total_b / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_call": total_b,
        "mfma_util_score": {"algorithmic_1pass": round(flops / (score_ms * 1e-3) / 1e12 /
                                                       BF16_PEAK_TFLOPS, 4),
                            "issued_2pass": round(2 * flops / (score_ms * 1e-3) / 1e12 /
                                                  BF16_PEAK_TFLOPS, 4)},
        # the score kernels against their VALU issue floor (fma, exp2 at half
        # rate, add per logit and pass), the bound they meet first
        "valu_floor_score": {"logit_updates": score_logit_updates(w, lens0),
                             "floor_us": round(score_logit_updates(w, lens0) / VALU_LOGIT_PEAK
                                               * 1e6, 1),
                             "frac": round(score_logit_updates(w, lens0) / VALU_LOGIT_PEAK /
                                           (score_ms * 1e-3), 4)},
        "score_kernels": score_kernels,
        "score_kernel": fused_name if fused else "snapkv_score_stats + snapkv_score_vote",
        "selection_in_gather": sel_in_gather,
        "stage_kernels": {k: {"ms": round(v, 5), "alg_bytes": sbytes[k],
                              "gbps": round(sbytes[k] / (v * 1e-3) / 1e9, 1)}
                          for k, v in stage_ms.items()},
        "roofline": roofline,
    }
    if extras:
        rec.update(measure_extras(w, args, dev, stream, sets, outs, ws, timed))
    del sets, outs, ws
    torch.cuda.synchronize()
    torch.cuda.empty_cache()
    return rec


def _window_lse(q, k, lens, window):
    """Natural-log normaliser of every window row, float32 [batch, H_q, W],
    with plain torch ops on the device (the prefill attention's by-product
    that snapkv_compress_from_lse consumes)."""
    import torch
    batch, hq, w, d = q.shape
    hkv = k.shape[1]
    g = hq // hkv
    out = torch.empty((batch, hq, w), dtype=torch.float32, device=q.device)
    off = 0
    for b, length in enumerate(lens):
        i = torch.arange(w, device=q.device).repeat(g)
        visible = torch.arange(length, device=q.device)[None, :] <= (length - w + i)[:, None]
        for h in range(hkv):
            kh = k[off:off + length, h].float().t().contiguous()
            logits = (q[b, h * g:(h + 1) * g].float().reshape(g * w, d) @ kh) / (d ** 0.5)
            out[b, h * g:(h + 1) * g] = torch.logsumexp(
                logits.masked_fill(~visible, float("-inf")), dim=1).reshape(g, w)
        off += length
    return out


def measure_extras(w, args, dev, stream, sets, outs, ws, timed):
    """The same workload through snapkv_compress_from_lse, _int4 and _fp8,
    and one decode step's attention over the compressed and the full cache."""
    import torch

    import long_context_kv_snapkv_amd as skv

    nsets = len(sets)
    batch, hkv, d, B = len(sets[0][3]), w.h_kv, w.head_dim, w.budget
    lens = sets[0][3]
    # the caller's prefill would hand over the normalisers: computed here
    # beforehand, outside the timed region, for every input set
    lses = [_window_lse(q, k, ls, w.window) for q, k, _, ls in sets]

    def step_lse(i):
        q, k, v, ls = sets[i % nsets]
        ok, ov, oi = outs[i % 2]
        skv.snapkv_compress_from_lse(q, k, v, ls, w.window, lses[i % nsets], w.kernel, w.pool, B,
                                     out_k=ok, out_v=ov, out_idx=oi, workspace=ws, stream=stream)

    ms_lse = timed(step_lse)
    quant = {}
    for form, per_byte in (("int4", 2), ("fp8", 1)):
        kq = [torch.empty((batch, hkv, B, d // per_byte), dtype=torch.uint8, device=dev)
              for _ in range(2)]
        vq = [torch.empty_like(t) for t in kq]
        ks = [torch.empty((batch, hkv, B), dtype=torch.float32, device=dev) for _ in range(2)]
        vs = [torch.empty_like(t) for t in ks]
        fn = skv.snapkv_compress_int4 if form == "int4" else skv.snapkv_compress_fp8

        def step_q(i, fn=fn, kq=kq, vq=vq, ks=ks, vs=vs):
            q, k, v, ls = sets[i % nsets]
            j = i % 2
            fn(q, k, v, ls, w.window, w.kernel, w.pool, B,
               out=(kq[j], ks[j], vq[j], vs[j], outs[j][2]), workspace=ws, stream=stream)

        ms = timed(step_q)
        quant[form] = {"ms_per_step": round(ms, 5),
                       "value": round(sum(lens) / (ms * 1e-3), 1), "unit": "tokens/s/layer",
                       "cache_bytes": 2 * batch * hkv * B * (d // per_byte + 4)}
    quant["int4"]["note"] = ("snapkv_compress_int4: kept rows stored as 4-bit codes with a "
                             "float32 scale per row")
    quant["fp8"]["note"] = ("snapkv_compress_fp8: kept rows stored as FP8 E4M3 bytes with a "
                            "float32 scale per row")

    # one decode step's attention over the compressed cache against the full
    # prefill cache, each streamed from HBM: enough distinct compressed caches
    # (the gathered rows of different input sets) to exceed the Infinity Cache
    n_kept = [min(L, B) for L in lens]
    qdec = torch.randn((batch, w.h_q, d), device=dev).to(torch.bfloat16)
    dout = torch.empty((batch, w.h_q, d), dtype=torch.float32, device=dev)
    comp_bytes = 2 * batch * hkv * B * d * 2
    ncomp = max(2, -(-4 * CACHE_BYTES // comp_bytes))
    comp = []
    for i in range(ncomp):
        q, k, v, ls = sets[i % nsets]
        ok = torch.empty((batch, hkv, B, d), dtype=torch.bfloat16, device=dev)
        ov = torch.empty_like(ok)
        skv.snapkv_compress(q, k, v, ls, w.window, w.kernel, w.pool, B, out_k=ok, out_v=ov,
                            workspace=ws, stream=stream)
        comp.append((ok, ov))
    torch.cuda.synchronize()
    ws_c = torch.empty(max(16, skv.snapkv_decode_workspace_size(
        w.h_q, hkv, d, n_kept, skv.SNAPKV_CACHE_COMPRESSED, B)), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(16, skv.snapkv_decode_workspace_size(
        w.h_q, hkv, d, lens, skv.SNAPKV_CACHE_PACKED)), dtype=torch.uint8, device=dev)

    # each step prepared once (arguments checked, one C call per step), as a
    # serving loop would; the host-driven rate is the loop's, the device time
    # comes from events the step's dispatches record at its first kernel's
    # start and last kernel's end
    def make_comp(i, events=None):
        kc, vc = comp[i % ncomp]
        return skv.prepare_decode(qdec, kc, vc, n_kept, out=dout, workspace=ws_c, stream=stream,
                                  events=events)

    def make_full(i, events=None):
        _, k, v, ls = sets[i % nsets]
        return skv.prepare_decode(qdec, k, v, ls, out=dout, workspace=ws_f, stream=stream,
                                  events=events)

    def device_ms(make):
        n = min(args.steps, 200)
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for a, b in evs:  # materialise the HIP events before handing them over
            a.record(stream)
            b.record(stream)
        torch.cuda.synchronize()
        runs = [make(i, evs[i]) for i in range(n)]
        for r in runs:
            r()
        torch.cuda.synchronize()
        t = sorted(a.elapsed_time(b) for a, b in evs)
        return sum(t) / n, t[n // 2]

    dec_steps = {"compressed": [make_comp(i) for i in range(ncomp)],
                 "full": [make_full(i) for i in range(nsets)]}
    dec_ms = {key: timed(lambda i, st=st: st[i % len(st)]()) for key, st in dec_steps.items()}
    dec_dev = {"compressed": device_ms(make_comp), "full": device_ms(make_full)}
    dec_dev_ms = {k: v[0] for k, v in dec_dev.items()}
    dec_dev_med = {k: v[1] for k, v in dec_dev.items()}
    dec_kernels = {"compressed": skv.snapkv_decode_kernels(w.h_q, hkv, d, n_kept,
                                                           skv.SNAPKV_CACHE_COMPRESSED, B),
                   "full": skv.snapkv_decode_kernels(w.h_q, hkv, d, lens,
                                                     skv.SNAPKV_CACHE_PACKED)}
    del dec_steps

    # the prefill attention whose by-product the compression reads: causal
    # attention of every prompt row (queries drawn here, N(0, 1/D)), with the
    # window normalisers and window queries it hands to
    # snapkv_compress_from_lse; alone, and followed by that compression
    npre = 2
    total = sum(lens)
    qfull = [(torch.randn((total, w.h_q, d), device=dev) / d ** 0.5).to(torch.bfloat16)
             for _ in range(npre)]
    pre_out = torch.empty((total, w.h_q, d), dtype=torch.bfloat16, device=dev)
    pre_lse = torch.empty((batch, w.h_q, w.window), dtype=torch.float32, device=dev)
    pre_qw = torch.empty((batch, w.h_q, w.window, d), dtype=torch.bfloat16, device=dev)

    def step_pre(i):
        _, k, v, ls = sets[i % nsets]
        skv.snapkv_prefill_attention(qfull[i % npre], k, v, ls, w.window, out=pre_out,
                                     window_lse=pre_lse, q_win=pre_qw, stream=stream)

    def step_pipe(i):
        step_pre(i)
        _, k, v, ls = sets[i % nsets]
        ok, ov, oi = outs[i % 2]
        skv.snapkv_compress_from_lse(pre_qw, k, v, ls, w.window, pre_lse, w.kernel, w.pool, B,
                                     out_k=ok, out_v=ov, out_idx=oi, workspace=ws, stream=stream)

    ms_pre = timed(step_pre)
    ms_pipe = timed(step_pipe)
    pre_flops = sum(4 * d * w.h_q * L * (L + 1) // 2 for L in lens)
    del qfull
    dec_bytes = {"compressed": 2 * hkv * sum(n_kept) * d * 2, "full": 2 * hkv * sum(lens) * d * 2}
    del comp
    pre_tflops = pre_flops / (ms_pre * 1e-3) / 1e12
    return {
        "prefill": {
            "note": "snapkv_prefill_attention: causal attention of every prompt row (bf16 MFMA), "
                    "emitting the window normalisers and queries; then "
                    "snapkv_compress_from_lse on them",
            "prefill_ms": round(ms_pre, 4), "prefill_tflops": round(pre_tflops, 1),
            "prefill_mfma_frac": round(pre_tflops / BF16_PEAK_TFLOPS, 4),
            "prefill_flops": pre_flops,
            "prefill_then_compress_ms": round(ms_pipe, 4),
            "compress_share_of_pipeline": round((ms_pipe - ms_pre) / ms_pipe, 4)},
        "from_lse": {"ms_per_step": round(ms_lse, 5),
                     "value": round(sum(lens) / (ms_lse * 1e-3), 1), "unit": "tokens/s/layer",
                     "note": "snapkv_compress_from_lse: window-row log-sum-exp supplied by "
                             "the caller's prefill, computed before the timed region"},
        "decode": {
            "note": "snapkv_decode_attention: one decode step's attention per layer over the "
                    "compressed cache (B rows per head) and over the full prefill cache; "
                    "*_us: host-driven loop of prepared steps (events around the loop), "
                    "*_device_us: the step's dispatch events (first kernel start to last "
                    "kernel end), mean (and median) over the steps",
            "compressed_us": round(dec_ms["compressed"] * 1e3, 3),
            "full_us": round(dec_ms["full"] * 1e3, 3),
            "speedup": round(dec_ms["full"] / dec_ms["compressed"], 2),
            "compressed_device_us": round(dec_dev_ms["compressed"] * 1e3, 3),
            "full_device_us": round(dec_dev_ms["full"] * 1e3, 3),
            "device_speedup": round(dec_dev_ms["full"] / dec_dev_ms["compressed"], 2),
            "compressed_device_median_us": round(dec_dev_med["compressed"] * 1e3, 3),
            "full_device_median_us": round(dec_dev_med["full"] * 1e3, 3),
            "kernels": dec_kernels,
            "compressed_gbps": round(dec_bytes["compressed"] / (dec_dev_ms["compressed"] * 1e-3) /
                                     1e9, 1),
            "full_gbps": round(dec_bytes["full"] / (dec_dev_ms["full"] * 1e-3) / 1e9, 1),
            "full_hbm_frac": round(dec_bytes["full"] / (dec_dev_ms["full"] * 1e-3) / 1e9 /
                                   HBM_PEAK_GBPS, 4),
            "cache_bytes": dec_bytes},
        "int4": quant["int4"],
        "fp8": quant["fp8"],
    }


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--subs", default=",".join(SUBS),
                    help="comma-separated workloads measured as sub-records, or 'none'")
    ap.add_argument("--extras-on", default="llama3_8b_16k",
                    help="workload that also times from_lse, int4, fp8 and decode")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0,
                    help="single-threaded oracle work per CPU baseline sample")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the compression path runs on a single "
              "MI355X and launches no multi-GPU work (--gpus must be 1).",
              file=sys.stderr)
        sys.exit(2)

    import torch

    import long_context_kv_snapkv_amd as skv
    from synth import WORKLOADS

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skv.load_library()
    stream = torch.cuda.current_stream(dev)
    subs = [] if args.subs in ("", "none") else [s for s in args.subs.split(",") if s]

    w = WORKLOADS[args.workload]
    head = measure(w, args, dev, stream, extras=(w.name == args.extras_on))
    records = {}
    for name in subs:
        if name == w.name:
            continue
        records[name] = measure(WORKLOADS[name], args, dev, stream,
                                extras=(name == args.extras_on))
        print(f"[bench] {name}: {records[name]['ms_per_step'] * 1e3:.1f} us per call",
              file=sys.stderr, flush=True)

    out = {
        "metric": METRIC, "value": head["value"], "unit": "tokens/s/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": head["ms_per_step"], "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
    }
    out.update({k: v for k, v in head.items() if k not in ("value", "unit", "ms_per_step")})
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
        for name, rec in records.items():
            rec["cpu_baseline"] = cpu_baseline(WORKLOADS[name], args.cpu_seconds)
    else:
        out["cpu_baseline"] = None
    out["workloads"] = records
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
