"""The synthetic input generator: determinism, shapes, rounding, planting."""

import numpy as np
import pytest
import torch

from synth import WORKLOADS, bf16_round_bits, make_custom, make_layer


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32) * 3,
                        np.float32([0.0, -0.0, 1.0, 1.00390625, 1.01171875])])
    # force exact ties: float32 values whose lower 16 bits are 0x8000
    hi = rng.integers(0x3800, 0x4800, 2000, dtype=np.uint32)
    ties = ((hi << np.uint32(16)) | np.uint32(0x8000)).view(np.float32)
    x = np.concatenate([x, ties])
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(bf16_round_bits(x), ref)


def test_deterministic_per_seed():
    a = make_custom([100, 40], 4, 2, 16, 8, seed=5)
    b = make_custom([100, 40], 4, 2, 16, 8, seed=5)
    c = make_custom([100, 40], 4, 2, 16, 8, seed=6)
    for f in ("q_win", "k", "v"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    assert not np.array_equal(a.k, c.k)


def test_tiny_workload_shapes_and_planting():
    w = WORKLOADS["tiny_mha_1k"]
    x = make_layer(w)
    assert x.q_win.shape == (1, 8, 32, 64) and x.k.shape == (1024, 8, 64)
    assert x.q_win.dtype == np.uint16
    for pos in x.planted[0]:
        assert len(pos) == 16 and pos.max() < 1024 - 32


def test_ragged_workload_has_one_identity_prompt():
    w = WORKLOADS["llama3_8b_ragged8"]
    # lengths only (cheap): reuse the generator's private length draw
    from synth.workloads import _ragged_lengths
    lens = _ragged_lengths(w, 0)
    assert len(lens) == 8
    short = lens < w.budget
    assert short.sum() == 1 and lens[short][0] > w.window
    assert ((lens[~short] >= 4096) & (lens[~short] <= 32768)).all()


def test_edge_spans_touch_both_prefix_ends():
    from synth.workloads import _spans
    rng = np.random.default_rng(0)
    pos = _spans(rng, 5000, count=128, cover=None, edges=True)
    assert pos[0] == 0 and pos[-1] == 4999
    # 128 separated spans of 3..9 positions
    starts = np.flatnonzero(np.diff(np.concatenate([[-10], pos])) > 1)
    assert len(starts) == 128


@pytest.mark.parametrize("layer,expect", [(0, 0.001), (31, 0.010)])
def test_density_planting(layer, expect):
    from synth.workloads import _plant_positions
    rng = np.random.default_rng(layer)
    pos = _plant_positions(rng, "density", 32736, layer, 32)
    assert abs(len(pos) - expect * 32736) <= 9
