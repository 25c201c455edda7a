"""Writes oracle_tiny_regression.json: the oracle's selection on a small
seeded input, kept so that any later change to the oracle's arithmetic shows
up as a diff. Calls only the oracle and the seeded input generator."""

import json
import os
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle import compress  # noqa: E402
from synth import make_custom  # noqa: E402

CASES = [
    dict(lens=[300, 70], h_q=8, h_kv=2, d=32, window=16, kernel=5, pool="avg", budget=96, seed=11),
    dict(lens=[257], h_q=4, h_kv=4, d=64, window=32, kernel=7, pool="max", budget=128, seed=12),
]


def main():
    out = []
    for c in CASES:
        x = make_custom(c["lens"], c["h_q"], c["h_kv"], c["d"], c["window"], seed=c["seed"])
        r = compress(x.q_win, x.k, x.v, x.seq_lens, c["window"], c["kernel"], c["pool"], c["budget"])
        out.append(dict(case=c, out_idx=r.out_idx.tolist()))
    with open(os.path.join(HERE, "oracle_tiny_regression.json"), "w") as f:
        json.dump(out, f)


if __name__ == "__main__":
    main()
