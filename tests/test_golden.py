"""Fixtures under tests/golden: the pages' printed hyperparameters and an
oracle regression record (written by tests/golden/make_oracle_fixture.py)."""

import json
import os

import numpy as np

from oracle import compress, pool_code, validate
from synth import make_custom

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _load(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def test_snippet_parameters_are_a_valid_configuration():
    p = _load("glossary_snippet_params.json")
    assert pool_code(p["pooling"]) == 0  # "avgpool" is average pooling
    validate(32, 8, 128, [8192], p["window_size"], p["kernel_size"], p["pooling"],
             p["max_capacity_prompt"])


def test_page_ranges_are_valid_configurations():
    r = _load("hyperparameter_ranges.json")
    for w in r["window"]:
        for k in range(r["kernel"][0], r["kernel"][1] + 1, 2):
            for pool in r["pooling"]:
                for b in r["budget"] + r["extra_budgets"]:
                    validate(32, 8, 128, [b + 1], w, k, pool, b)


def test_oracle_regression_record():
    for rec in _load("oracle_tiny_regression.json"):
        c = rec["case"]
        x = make_custom(c["lens"], c["h_q"], c["h_kv"], c["d"], c["window"], seed=c["seed"])
        r = compress(x.q_win, x.k, x.v, x.seq_lens, c["window"], c["kernel"], c["pool"],
                     c["budget"])
        np.testing.assert_array_equal(r.out_idx, np.array(rec["out_idx"]))
