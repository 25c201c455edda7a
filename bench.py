"""Throughput of SnapKV prefill-time KV-cache compression on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

A step is one snapkv_compress call (vote statistics, vote with pooling,
selection, gather: four kernels, or fewer when statistics and vote run as
the fused score kernel and the selection runs inside the gather) on one
layer of synthetic, seeded input
already resident in HBM. Inputs and outputs rotate over enough buffer sets to
exceed the 256 MB Infinity Cache, so every step streams its K from HBM.
Prints one JSON line: value = prompt tokens compressed per second per layer;
the roofline of the dominant kernel, timed per kernel with HIP events on the
library's stream through snapkv_compress_staged (one kernel per stage) and
priced with its algorithmic bytes per launch; and the fp64 CPU oracle timed
on a bounded sample of the same workload on this host.
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
METRIC = "prompt tokens compressed/sec per layer; achieved HBM GB/s vs MI355X peak"
CACHE_BYTES = 256 << 20       # Infinity Cache
KERNEL_SOURCES = ("snapkv_api.cpp", "snapkv_kernels.h", "snapkv_kernels.hip", "snapkv_score.h",
                  "snapkv_select.h", "snapkv_gather.h", "snapkv_device.h")


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
    fused score kernel (both in one launch) reads Q and all L keys once;
    select reads the P pooled scores and writes the index list; gather moves
    the kept rows (the gather term of algorithmic_bytes)."""
    d, q_bytes = w.head_dim, w.h_q * w.window * w.head_dim * 2
    gather = algorithmic_bytes(w, seq_lens)[1]
    out = {"snapkv_score_stats": 0, "snapkv_score_vote": 0, "snapkv_score_fused": 0,
           "snapkv_score_fused_stream": 0, "snapkv_select": 0, "snapkv_gather": gather, "snapkv_gather_select": gather}
    for L in seq_lens:
        if L > w.budget:
            P = L - w.window
            out["snapkv_score_stats"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_fused"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_fused_stream"] += q_bytes + w.h_kv * L * d * 2
            out["snapkv_score_vote"] += q_bytes + w.h_kv * P * d * 2
            out["snapkv_select"] += w.h_kv * (P * 4 + w.budget * 4)
            out["snapkv_gather_select"] += w.h_kv * P * 4  # the pooled scores, read once
    return out


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
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when the kernel source changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f).get(kernel_key)
    if not rec or rec.get("source_hash") != _source_hash(KERNEL_SOURCES):
        return None
    return rec.get("hbm_bytes_per_launch")


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


def cpu_baseline(w, x, budget_s=10.0):
    import numpy as np  # noqa: F401

    import oracle
    threads = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads", 0) for i in threadpool_info() if i.get("user_api") == "blas"]
        threads = max(blas) if blas else 1
    except Exception:
        pass
    lens = x.seq_lens.tolist()
    t0 = time.perf_counter()
    calls = 0
    while True:
        oracle.compress(x.q_win, x.k, x.v, lens, w.window, w.kernel, w.pool, w.budget,
                        keep_scores=False)
        calls += 1
        if time.perf_counter() - t0 > budget_s:
            break
    dt = (time.perf_counter() - t0) / calls
    return {"value": sum(lens) / dt, "unit": "tokens/s/layer", "cores": threads,
            "kind": "oracle",
            "sample": f"{w.name} layer 0, all {w.h_kv} KV heads, {calls} full oracle "
                      f"call(s) in {dt * calls:.1f} s ({dt:.2f} s per layer)"}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--workload", default="llama3_8b_16k")
    ap.add_argument("--sets", type=int, default=0, help="rotating input sets (0: auto)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain device copy of known size (counter scaling)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the compression path runs on a single "
              "MI355X and launches no multi-GPU work (--gpus must be 1).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import long_context_kv_snapkv_amd as skv
    from synth import WORKLOADS, make_layer

    w = WORKLOADS[args.workload]
    x = make_layer(w, 0)
    lens = x.seq_lens.tolist()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    skv.load_library()

    def up(bits):
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(
            torch.bfloat16).to(dev)

    q0, k0, v0 = up(x.q_win), up(x.k), up(x.v)
    kv_bytes = 2 * k0.numel() * 2
    nsets = args.sets or max(2, min(64, -(-4 * CACHE_BYTES // kv_bytes)))
    batch, hkv, d, B = len(lens), w.h_kv, w.head_dim, w.budget
    sets = []
    for i in range(nsets):
        sets.append(dict(q=q0.clone(), k=k0.clone(), v=v0.clone(),
                         ok=torch.empty((batch, hkv, B, d), dtype=torch.bfloat16, device=dev),
                         ov=torch.empty((batch, hkv, B, d), dtype=torch.bfloat16, device=dev),
                         oi=torch.empty((batch, hkv, B), dtype=torch.int32, device=dev)))
    del q0, k0, v0
    ws = skv.new_workspace(w.h_q, hkv, d, lens, w.window, dev)
    stream = torch.cuda.current_stream(dev)

    def step(i, staged=False, events=None):
        s = sets[i % nsets]
        skv.snapkv_compress(s["q"], s["k"], s["v"], lens, w.window, w.kernel, w.pool, B,
                            out_k=s["ok"], out_v=s["ov"], out_idx=s["oi"], workspace=ws,
                            stream=stream, staged=staged, stage_events=events)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t_start = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    t_start.record(stream)
    for i in range(args.steps):
        step(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_total = t_start.elapsed_time(t_end)
    ms_step = ms_total / args.steps

    # per-kernel durations: snapkv_compress_staged has each stage's dispatch
    # record the caller's events at its kernel's start and end
    nprof = min(args.steps, 200)
    nst = skv.SNAPKV_NUM_STAGES
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(2 * nst)]
           for _ in range(nprof)]
    for row in evs:  # materialise the HIP events before handing them over
        for e in row:
            e.record(stream)
    torch.cuda.synchronize()
    for i in range(nprof):
        step(i, staged=True, events=evs[i])
    torch.cuda.synchronize()
    # with a fused score kernel, stage 0 is that kernel and stage 1 is empty
    # and with the selection inside the gather, stage 3 is that kernel and
    # stage 2 is empty
    score_kernels = skv.snapkv_score_kernels(w.h_q, hkv, d, lens, w.window, w.kernel)
    fused = score_kernels != 2
    fused_name = "snapkv_score_fused" if score_kernels == 1 else "snapkv_score_fused_stream"
    sel_in_gather = skv.snapkv_gather_selects(w.h_q, hkv, d, lens, w.window, B) == 1
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
        stage_ms[name] = float(np.mean(vals))

    # the same compression when the caller's prefill attention hands over
    # each window row's log-sum-exp (snapkv_compress_from_lse): the
    # normalisers are computed here beforehand, outside the timed region, as
    # a prefill kernel would have produced them
    lse = _window_lse(sets[0]["q"], sets[0]["k"], lens, w.window)

    def step_lse(i):
        s = sets[i % nsets]
        skv.snapkv_compress_from_lse(s["q"], s["k"], s["v"], lens, w.window, lse, w.kernel,
                                     w.pool, B, out_k=s["ok"], out_v=s["ov"], out_idx=s["oi"],
                                     workspace=ws, stream=stream)

    for i in range(args.warmup):
        step_lse(i)
    torch.cuda.synchronize()
    t_start.record(stream)
    for i in range(args.steps):
        step_lse(i)
    t_end.record(stream)
    torch.cuda.synchronize()
    ms_step_lse = t_start.elapsed_time(t_end) / args.steps

    # the same compression storing the kept rows at 4 bits per value
    # (snapkv_compress_int4)
    for s_ in sets:
        s_["kq"] = torch.empty((batch, hkv, B, d // 2), dtype=torch.uint8, device=dev)
        s_["vq"] = torch.empty_like(s_["kq"])
        s_["ks"] = torch.empty((batch, hkv, B), dtype=torch.float32, device=dev)
        s_["vs"] = torch.empty_like(s_["ks"])

    def step_int4(i):
        s = sets[i % nsets]
        skv.snapkv_compress_int4(s["q"], s["k"], s["v"], lens, w.window, w.kernel, w.pool, B,
                                 out=(s["kq"], s["ks"], s["vq"], s["vs"], s["oi"]),
                                 workspace=ws, stream=stream)

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

    ms_step_int4 = timed(step_int4)
    # and as FP8 E4M3 bytes (snapkv_compress_fp8)
    for s_ in sets:
        s_["kq8"] = torch.empty((batch, hkv, B, d), dtype=torch.uint8, device=dev)
        s_["vq8"] = torch.empty_like(s_["kq8"])

    def step_fp8(i):
        s = sets[i % nsets]
        skv.snapkv_compress_fp8(s["q"], s["k"], s["v"], lens, w.window, w.kernel, w.pool, B,
                                out=(s["kq8"], s["ks"], s["vq8"], s["vs"], s["oi"]),
                                workspace=ws, stream=stream)

    ms_step_fp8 = timed(step_fp8)
    for s_ in sets:
        del s_["kq8"], s_["vq8"]

    # one decode step's attention over the compressed cache against the full
    # prefill cache (snapkv_decode_attention), each cache streamed from HBM:
    # enough distinct compressed caches rotate to exceed the Infinity Cache
    n_kept = [min(L, B) for L in lens]
    qdec = torch.randn((batch, w.h_q, d), device=dev).to(torch.bfloat16)
    dout = torch.empty((batch, w.h_q, d), dtype=torch.float32, device=dev)
    comp_bytes = 2 * batch * hkv * B * d * 2
    ncomp = max(2, -(-4 * CACHE_BYTES // comp_bytes))
    comp = [(sets[i % nsets]["ok"].clone(), sets[i % nsets]["ov"].clone()) for i in range(ncomp)]
    ws_c = torch.empty(max(16, skv.snapkv_decode_workspace_size(
        w.h_q, hkv, d, n_kept, skv.SNAPKV_CACHE_COMPRESSED, B)), dtype=torch.uint8, device=dev)
    ws_f = torch.empty(max(16, skv.snapkv_decode_workspace_size(
        w.h_q, hkv, d, lens, skv.SNAPKV_CACHE_PACKED)), dtype=torch.uint8, device=dev)

    def dec_comp(i):
        kc, vc = comp[i % ncomp]
        skv.snapkv_decode_attention(qdec, kc, vc, n_kept, out=dout, workspace=ws_c, stream=stream)

    def dec_full(i):
        s = sets[i % nsets]
        skv.snapkv_decode_attention(qdec, s["k"], s["v"], lens, out=dout, workspace=ws_f,
                                    stream=stream)

    dec_ms = {}
    for name, fn in (("compressed", dec_comp), ("full", dec_full)):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t_start.record(stream)
        for i in range(args.steps):
            fn(i)
        t_end.record(stream)
        torch.cuda.synchronize()
        dec_ms[name] = t_start.elapsed_time(t_end) / args.steps
    dec_bytes = {"compressed": 2 * hkv * sum(n_kept) * d * 2,
                 "full": 2 * hkv * sum(lens) * d * 2}
    del comp

    sbytes = stage_bytes(w, lens)
    dominant = max(stage_ms, key=stage_ms.get)
    kernel_ms = stage_ms[dominant]
    achieved = sbytes[dominant] / (kernel_ms * 1e-3) / 1e9
    score_b, gather_b = algorithmic_bytes(w, lens)
    total_b = score_b + gather_b
    flops = score_flops(w, lens)
    score_ms = (stage_ms[fused_name] if fused else
                stage_ms["snapkv_score_stats"] + stage_ms["snapkv_score_vote"])
    tokens = sum(lens)
    value = tokens / (ms_step * 1e-3)
    roofline = {
        "kernel": dominant, "bound": "hbm",
        "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
        "frac": round(achieved / HBM_PEAK_GBPS, 4),
        "traffic": _traffic(dominant),
        "bytes_per_launch": sbytes[dominant], "launch_ms": round(kernel_ms, 5),
    }
    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s/layer",
        "n_gpus": 1, "steps": args.steps, "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w.name, "batch": batch, "seq_len": lens if batch > 1 else lens[0],
                   "num_q_heads": w.h_q, "num_kv_heads": hkv, "head_dim": d,
                   "window": w.window, "kernel_size": w.kernel, "pooling": w.pool + "pool",
                   "budget": B, "rotating_sets": nsets},
        "hbm_gbps_whole_call": round(total_b / (ms_step * 1e-3) / 1e9, 1),
        "hbm_frac_whole_call": round(total_b / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "algorithmic_bytes_per_call": total_b,
        "mfma_util_score": {"algorithmic_1pass": round(flops / (score_ms * 1e-3) / 1e12 /
                                                       BF16_PEAK_TFLOPS, 4),
                            "issued_2pass": round(2 * flops / (score_ms * 1e-3) / 1e12 /
                                                  BF16_PEAK_TFLOPS, 4)},
        "score_kernels": 1 if fused else 2,
        "score_kernel": fused_name if fused else "snapkv_score_stats + snapkv_score_vote",
        "selection_in_gather": sel_in_gather,
        "stage_kernels": {k: {"ms": round(v, 5), "alg_bytes": sbytes[k],
                              "gbps": round(sbytes[k] / (v * 1e-3) / 1e9, 1)}
                          for k, v in stage_ms.items()},
        "roofline": roofline,
        "from_lse": {"ms_per_step": round(ms_step_lse, 5),
                     "value": round(sum(lens) / (ms_step_lse * 1e-3), 1),
                     "unit": "tokens/s/layer",
                     "note": "snapkv_compress_from_lse: window-row log-sum-exp supplied by "
                             "the caller's prefill, computed before the timed region"},
        "decode": {
            "note": "snapkv_decode_attention: one decode step's attention per layer over the "
                    "compressed cache (B rows per head) and over the full prefill cache",
            "compressed_us": round(dec_ms["compressed"] * 1e3, 3),
            "full_us": round(dec_ms["full"] * 1e3, 3),
            "speedup": round(dec_ms["full"] / dec_ms["compressed"], 2),
            "compressed_gbps": round(dec_bytes["compressed"] / (dec_ms["compressed"] * 1e-3) / 1e9,
                                     1),
            "full_gbps": round(dec_bytes["full"] / (dec_ms["full"] * 1e-3) / 1e9, 1),
            "full_hbm_frac": round(dec_bytes["full"] / (dec_ms["full"] * 1e-3) / 1e9 /
                                   HBM_PEAK_GBPS, 4),
            "cache_bytes": dec_bytes},
        "int4": {"ms_per_step": round(ms_step_int4, 5),
                 "value": round(sum(lens) / (ms_step_int4 * 1e-3), 1),
                 "unit": "tokens/s/layer",
                 "cache_bytes": 2 * batch * hkv * B * (d // 2 + 4),
                 "note": "snapkv_compress_int4: kept rows stored as 4-bit codes with a "
                         "float32 scale per row"},
        "fp8": {"ms_per_step": round(ms_step_fp8, 5),
                "value": round(sum(lens) / (ms_step_fp8 * 1e-3), 1),
                "unit": "tokens/s/layer",
                "cache_bytes": 2 * batch * hkv * B * (d + 4),
                "note": "snapkv_compress_fp8: kept rows stored as FP8 E4M3 bytes with a "
                        "float32 scale per row"},
    }
    if args.copy_calibration:
        src = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        out["copy_calibration_bytes"] = src.numel()
    if not args.no_cpu_baseline:
        out["cpu_baseline"] = cpu_baseline(w, x)
    else:
        out["cpu_baseline"] = None
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
