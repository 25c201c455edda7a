"""Seeded synthetic workloads shaped like the SnapKV evaluation settings.

The SnapKV pages evaluate on LLaMA-3-8B-Instruct (32 query heads, 8 KV heads,
head_dim 128) at long context and run a 70B-class model up to hundreds of
thousands of tokens (SnapKV abstract, page "SnapKV: LLM Knows What You are
Looking for Before Generation"; glossary page "SnapKV", section on evaluation).
Neither the datasets nor the weights are available here, so these generators
stand in for them: Gaussian Q/K/V at the models' head shapes, with "clustered
important positions" (abstract: SnapKV keeps clustered important KV positions
per head) emulated by planting a per-head direction into chosen key positions
and into every observation-window query of that head's group.

Recipe (every value is deterministic in the seed):

* one ``numpy.random.Generator(PCG64(seed))`` per prompt, with
  ``seed = 1_000_000 * ident + 1000 * layer + prompt``;
* draw order per prompt: ``q_win`` [H_q, W, D], then ``k`` [L, H_kv, D], then
  ``v`` [L, H_kv, D], all ``standard_normal(float32) / sqrt(D)``; then, per
  KV head h in order, a unit direction ``u_h`` (float64 Gaussian, normalised)
  followed by that head's planted positions;
* ``4 * u_h`` is added to K at the planted positions of head h and to every
  window row of every query head in h's group (V is never planted);
* the result is rounded once to bfloat16 with round-to-nearest-even and handed
  over as raw uint16 bit patterns, so every consumer sees identical bits.

Nothing here computes attention, pooling or selection.
"""

from __future__ import annotations

from dataclasses import dataclass, field
from typing import List, Optional, Sequence

import numpy as np

PLANT_SCALE = 4.0


@dataclass(frozen=True)
class Workload:
    """Shape and hyperparameters of one synthetic workload."""

    name: str
    ident: int
    h_q: int
    h_kv: int
    head_dim: int
    window: int
    kernel: int
    pool: str  # "avg" or "max"
    budget: int
    layers: int
    batch: int
    planting: str
    length: Optional[int]  # fixed prompt length, None for the ragged batch
    description: str = ""

    @property
    def group(self) -> int:
        return self.h_q // self.h_kv


WORKLOADS = {
    "tiny_mha_1k": Workload(
        name="tiny_mha_1k", ident=1, h_q=8, h_kv=8, head_dim=64, window=32,
        kernel=5, pool="avg", budget=256, layers=1, batch=1,
        planting="points16", length=1024,
        description="tiny MHA layer, L=1024, W=32, avgpool 5, B=256"),
    "llama3_8b_16k": Workload(
        name="llama3_8b_16k", ident=2, h_q=32, h_kv=8, head_dim=128, window=32,
        kernel=7, pool="max", budget=1024, layers=1, batch=1,
        planting="spans64", length=16384,
        description="Llama-3-8B-shaped layer (32q/8kv, d=128), L=16384, W=32, "
                    "maxpool 7, B=1024"),
    "llama3_8b_32k_x32": Workload(
        name="llama3_8b_32k_x32", ident=3, h_q=32, h_kv=8, head_dim=128,
        window=32, kernel=5, pool="avg", budget=2048, layers=32, batch=1,
        planting="density", length=32768,
        description="Llama-3-8B-shaped 32-layer stack, L=32768, W=32, "
                    "avgpool 5, B=2048"),
    "llama3_8b_ragged8": Workload(
        name="llama3_8b_ragged8", ident=4, h_q=32, h_kv=8, head_dim=128,
        window=64, kernel=13, pool="avg", budget=4096, layers=1, batch=8,
        planting="ragged_spans", length=None,
        description="ragged batch of 8 prompts (7 in [4096,32768], one < B), "
                    "W=64, avgpool 13, B=4096"),
    "llama3_70b_128k_x80": Workload(
        name="llama3_70b_128k_x80", ident=5, h_q=64, h_kv=8, head_dim=128,
        window=64, kernel=7, pool="max", budget=1024, layers=80, batch=1,
        planting="spans128_edges", length=131072,
        description="70B-shaped layers (64q/8kv, d=128), L=131072, W=64, "
                    "maxpool 7, B=1024, 80 layers"),
}


def workload(name: str) -> Workload:
    return WORKLOADS[name]


@dataclass
class LayerInputs:
    """One layer's inputs as raw bfloat16 bit patterns (uint16)."""

    q_win: np.ndarray  # uint16 [batch, H_q, W, D]
    k: np.ndarray  # uint16 [T, H_kv, D], prompts packed back to back
    v: np.ndarray  # uint16 [T, H_kv, D]
    seq_lens: np.ndarray  # int32 [batch]
    planted: List[List[np.ndarray]] = field(default_factory=list)  # [prompt][head]

    @property
    def offsets(self) -> np.ndarray:
        return np.concatenate([[0], np.cumsum(self.seq_lens)[:-1]]).astype(np.int64)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return bits."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    out = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    return out.astype(np.uint16)


def _seed(ident: int, layer: int, prompt: int) -> int:
    return 1_000_000 * ident + 1000 * layer + prompt


def _unit(rng: np.random.Generator, d: int) -> np.ndarray:
    u = rng.standard_normal(d)
    return u / np.linalg.norm(u)


def _spans(rng, p: int, count: Optional[int], cover: Optional[int],
           edges: bool, lo: int = 3, hi: int = 9) -> np.ndarray:
    """Non-overlapping spans (at least one free slot between spans) in [0, p).

    Either ``count`` spans or spans until ``cover`` positions are covered.
    With ``edges`` the first span starts at 0 and the second ends at p-1.
    """
    occ = np.zeros(p, dtype=bool)
    placed = 0

    def free(s: int, n: int) -> bool:
        a, b = max(0, s - 1), min(p, s + n + 1)
        return not occ[a:b].any()

    def put(s: int, n: int) -> None:
        nonlocal placed
        occ[s:s + n] = True
        placed += 1

    if edges:
        n0 = min(int(rng.integers(lo, hi + 1)), p)
        put(0, n0)
        n1 = int(rng.integers(lo, hi + 1))
        if p - n1 > n0 + 1:
            put(p - n1, n1)
    covered = int(occ.sum())
    tries = 0
    while True:
        if count is not None and placed >= count:
            break
        if cover is not None and covered >= cover:
            break
        tries += 1
        if tries > 100000:
            break
        n = int(rng.integers(lo, hi + 1))
        if n > p:
            break
        s = int(rng.integers(0, p - n + 1))
        if free(s, n):
            put(s, n)
            covered += n
    return np.flatnonzero(occ).astype(np.int64)


def _plant_positions(rng, kind: str, p: int, layer: int, layers: int) -> np.ndarray:
    if p < 1:
        return np.zeros(0, dtype=np.int64)
    if kind == "points16":
        return np.sort(rng.choice(p, size=min(16, p), replace=False)).astype(np.int64)
    if kind in ("spans64", "ragged_spans"):
        return _spans(rng, p, count=64, cover=None, edges=False)
    if kind == "spans128_edges":
        return _spans(rng, p, count=128, cover=None, edges=True)
    if kind == "density":
        frac = 0.001 + 0.009 * (layer / max(1, layers - 1))
        return _spans(rng, p, count=None, cover=int(round(frac * p)), edges=False)
    if kind == "none":
        return np.zeros(0, dtype=np.int64)
    raise ValueError(f"unknown planting {kind!r}")


def _ragged_lengths(w: Workload, layer: int) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(_seed(w.ident, layer, 999)))
    lens = rng.integers(4096, 32768 + 1, size=w.batch)
    short = int(rng.integers(0, w.batch))
    lens[short] = int(rng.integers(w.window + 1, w.budget))  # W < L < B
    return lens.astype(np.int32)


def _make(seq_lens: Sequence[int], h_q: int, h_kv: int, d: int, window: int,
          ident: int, layer: int, planting: str, layers: int = 1) -> LayerInputs:
    seq_lens = np.asarray(seq_lens, dtype=np.int32)
    batch = len(seq_lens)
    g = h_q // h_kv
    total = int(seq_lens.sum())
    q_out = np.empty((batch, h_q, window, d), dtype=np.uint16)
    k_out = np.empty((total, h_kv, d), dtype=np.uint16)
    v_out = np.empty((total, h_kv, d), dtype=np.uint16)
    inv = np.float32(1.0 / np.sqrt(d))
    planted_all = []
    off = 0
    for b, length in enumerate(seq_lens.tolist()):
        rng = np.random.Generator(np.random.PCG64(_seed(ident, layer, b)))
        q = rng.standard_normal((h_q, window, d), dtype=np.float32) * inv
        k = rng.standard_normal((length, h_kv, d), dtype=np.float32) * inv
        v = rng.standard_normal((length, h_kv, d), dtype=np.float32) * inv
        p = length - window
        planted = []
        for h in range(h_kv):
            u = (PLANT_SCALE * _unit(rng, d)).astype(np.float32)
            pos = _plant_positions(rng, planting, p, layer, layers)
            if pos.size:
                k[pos, h, :] += u
                q[h * g:(h + 1) * g, :, :] += u
            planted.append(pos)
        planted_all.append(planted)
        q_out[b] = bf16_round_bits(q)
        k_out[off:off + length] = bf16_round_bits(k)
        v_out[off:off + length] = bf16_round_bits(v)
        off += length
    return LayerInputs(q_win=q_out, k=k_out, v=v_out, seq_lens=seq_lens,
                       planted=planted_all)


def make_layer(w: Workload, layer: int = 0) -> LayerInputs:
    """Inputs of one layer of a named workload."""
    if not 0 <= layer < w.layers:
        raise ValueError(f"layer {layer} out of range for {w.name}")
    if w.length is None:
        lens = _ragged_lengths(w, layer)
    else:
        lens = np.full(w.batch, w.length, dtype=np.int32)
    return _make(lens, w.h_q, w.h_kv, w.head_dim, w.window, w.ident, layer,
                 w.planting, w.layers)


def make_custom(seq_lens: Sequence[int], h_q: int, h_kv: int, head_dim: int,
                window: int, seed: int = 0, planting: str = "points16") -> LayerInputs:
    """Inputs of an arbitrary shape with the same recipe (for edge cases)."""
    return _make(seq_lens, h_q, h_kv, head_dim, window, ident=100 + seed,
                 layer=0, planting=planting)
