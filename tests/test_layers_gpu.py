"""GPU parity on every layer of the two multi-layer workloads: the 32-layer
Llama-3-8B-shaped stack at L = 32768 (per-layer heavy-hitter density from
0.1% to 1%) and the 80-layer 70B-shaped stack at L = 131072.

Each layer is compressed through snapkv_compress_with_scores, so the scores
compared are the ones the selection read (from the one-launch scoring
kernels these shapes take on a full MI355X). Per layer and KV head:
  * pooled scores within 1e-3 relative (+1e-6 of the head's maximum) of the
    fp64 oracle;
  * the oracle's selection rule on those scores gives the index list exactly;
  * every clearly-kept position is kept and no clearly-dropped one is, and
    where the oracle's threshold gap exceeds the tolerance the index list is
    the oracle's;
  * out_k / out_v rows are bit copies of K / V at the indices (on the device).
The oracle runs in a pool of worker processes, one layer per job, started
when the first test of this file runs; the layers are checked in order as
their jobs finish.
"""

import multiprocessing
import os
from concurrent.futures import ProcessPoolExecutor

import numpy as np
import pytest
import torch

import long_context_kv_snapkv_amd as skv
from parity import bits_to_device, check_index_sets, check_selected_scores, check_topk_exact
from synth import WORKLOADS

import layer_oracle

pytestmark = pytest.mark.gpu

needs_gpu = pytest.mark.skipif(not torch.cuda.is_available(), reason="needs a GPU")

STACKS = ("llama3_8b_32k_x32", "llama3_70b_128k_x80")
LAYERS = [(name, layer) for name in STACKS for layer in range(WORKLOADS[name].layers)]


@pytest.fixture(scope="module")
def oracle_jobs():
    workers = max(1, min(16, len(os.sched_getaffinity(0))))
    ex = ProcessPoolExecutor(max_workers=workers,
                             mp_context=multiprocessing.get_context("spawn"),
                             initializer=layer_oracle.init_worker)
    print(f"[layers] oracle pool of {workers} workers for {len(LAYERS)} layers", flush=True)
    futures = {key: ex.submit(layer_oracle.layer_job, *key) for key in LAYERS}
    yield futures
    for f in futures.values():
        f.cancel()
    ex.shutdown(wait=True, cancel_futures=True)


@needs_gpu
@pytest.mark.parametrize("name,layer", LAYERS, ids=[f"{n}-L{l}" for n, l in LAYERS])
def test_layer_matches_oracle(oracle_jobs, name, layer):
    w = WORKLOADS[name]
    job = oracle_jobs.pop((name, layer)).result(timeout=900)
    lens = job["lens"]
    print(f"[layers] {name} layer {layer} lens={lens}", flush=True)
    q, k, v = bits_to_device(job["q"]), bits_to_device(job["k"]), bits_to_device(job["v"])
    del job["q"], job["k"], job["v"]
    out_k, out_v, out_idx, sel = skv.snapkv_compress_with_scores(
        q, k, v, lens, w.window, w.kernel, w.pool, w.budget)
    torch.cuda.synchronize()
    res = dict(out_idx=out_idx.cpu().numpy(), sel_scores=sel.cpu().numpy().astype(np.float64))
    check_selected_scores(res["sel_scores"], job["pooled"], lens, w.window, w.budget)
    check_topk_exact(res, lens, w.window, w.budget)
    check_index_sets(res["out_idx"], job["pooled"], lens, w.window, w.budget)
    # the gathered rows, compared on the device (batch 1: prompt 0 only)
    assert len(lens) == 1
    idx = out_idx[0].long()
    n = min(lens[0], w.budget)
    assert (res["out_idx"][0, :, n:] == -1).all()
    for h in range(w.h_kv):
        rows = idx[h, :n]
        assert torch.equal(out_k[0, h, :n].view(torch.int16), k[rows, h].view(torch.int16))
        assert torch.equal(out_v[0, h, :n].view(torch.int16), v[rows, h].view(torch.int16))
    np.testing.assert_array_equal(res["out_idx"][0, :, w.budget - w.window:],
                                  job["out_idx"][0, :, w.budget - w.window:])
