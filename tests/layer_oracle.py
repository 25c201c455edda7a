"""Oracle side of the per-layer parity tests, run in worker processes.

One job builds one layer of a named workload from its seed and runs the
fp64 oracle on it (single-threaded BLAS, so that a pool of workers shares the
host's cores). It returns the layer's input bits (which the GPU side uploads)
and the oracle's pooled scores and index lists. Nothing here touches a GPU.
"""

from __future__ import annotations

import numpy as np

import oracle
from synth import WORKLOADS, make_layer


def init_worker() -> None:
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(1)
    except Exception:  # without threadpoolctl the BLAS default stands
        pass


def layer_job(name: str, layer: int) -> dict:
    w = WORKLOADS[name]
    x = make_layer(w, layer)
    lens = x.seq_lens.tolist()
    ref = oracle.compress(x.q_win, x.k, x.v, lens, w.window, w.kernel, w.pool, w.budget,
                          keep_scores=False)
    return dict(q=x.q_win, k=x.k, v=x.v, lens=lens,
                pooled=[None if p is None else np.asarray(p) for p in ref.pooled],
                out_idx=ref.out_idx)
