"""The synthetic workloads' recipe with the bulk values drawn on the device.

For timing, where many distinct layers or input sets must sit in device
memory at once and drawing 10^8..10^9 Gaussians on the host would take
minutes: the same shapes, distributions and planting as ``workloads.py``,
but the Gaussian values of Q_win, K and V come from torch's generator on the
device (seeded per prompt), so the bits differ from ``make_layer``'s. The
planting structure (the unit direction of each KV head, the planted
positions, the ragged lengths) is drawn on the host exactly as in
``workloads.py``, from the same ``PCG64`` seeds after an offset that keeps
each ``variant`` distinct. Parity tests use ``make_layer``; only timing uses
this module. Nothing here computes attention, pooling or selection.
"""

from __future__ import annotations

import numpy as np

from .workloads import PLANT_SCALE, Workload, _plant_positions, _ragged_lengths, _seed

VARIANT_STRIDE = 100_000_000  # seed offset between variants of one layer


def layer_lengths(w: Workload, layer: int = 0) -> list:
    """Prompt lengths of a layer, as make_layer draws them."""
    if w.length is None:
        return _ragged_lengths(w, layer).tolist()
    return [w.length] * w.batch


def make_layer_device(w: Workload, layer: int, device, variant: int = 0):
    """(q_win, k, v, seq_lens): bf16 device tensors [batch, H_q, W, D] and
    [T, H_kv, D] (prompts packed), and the lengths, for one layer (and input
    variant) of a named workload. Values are N(0, 1/D) plus the planted
    head directions, rounded once to bf16 (round to nearest even)."""
    import torch

    lens = layer_lengths(w, layer)
    g_size = w.h_q // w.h_kv
    d = w.head_dim
    inv = 1.0 / np.sqrt(d)
    total = int(sum(lens))
    q_out = torch.empty((len(lens), w.h_q, w.window, d), dtype=torch.bfloat16, device=device)
    k_out = torch.empty((total, w.h_kv, d), dtype=torch.bfloat16, device=device)
    v_out = torch.empty((total, w.h_kv, d), dtype=torch.bfloat16, device=device)
    off = 0
    for b, length in enumerate(lens):
        seed = _seed(w.ident, layer, b) + VARIANT_STRIDE * variant
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)
        q = torch.randn((w.h_q, w.window, d), generator=gen, device=device) * inv
        k = torch.randn((length, w.h_kv, d), generator=gen, device=device) * inv
        rng = np.random.Generator(np.random.PCG64(seed))
        p = length - w.window
        for h in range(w.h_kv):
            u = rng.standard_normal(d)
            u = PLANT_SCALE * u / np.linalg.norm(u)
            pos = _plant_positions(rng, w.planting, p, layer, w.layers)
            if pos.size:
                ut = torch.from_numpy(u.astype(np.float32)).to(device)
                k[torch.from_numpy(pos).to(device), h, :] += ut
                q[h * g_size:(h + 1) * g_size] += ut
        q_out[b] = q.to(torch.bfloat16)
        k_out[off:off + length] = k.to(torch.bfloat16)
        del k
        v = torch.randn((length, w.h_kv, d), generator=gen, device=device) * inv
        v_out[off:off + length] = v.to(torch.bfloat16)
        del v, q
        off += length
    return q_out, k_out, v_out, lens
