"""Write tests/golden/formula_cases.json: oracle outputs on small inputs given by a
closed formula.

Only the CPU oracle (``oracle/attention_ref.py``) computes the stored values; the
inputs come from the formula below, not from any generator, so the file is
reproducible on any machine.  Every input value is a small multiple of 1/8, exact
in bf16 and fp32, so the same inputs serve the fp32 and the bf16 GPU paths.

The pages print no worked numerical example of attention, so no fixture here
quotes them; these are regression fixtures for the oracle and small parity cases
for the GPU path.

    python tests/golden/make_golden.py
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.dirname(os.path.dirname(HERE)))

from oracle.attention_ref import attention_forward  # noqa: E402

CASES = [
    # name, N, d, mask_kind, window
    ("none_n7_d64", 7, 64, 0, 0),
    ("causal_n7_d64", 7, 64, 1, 0),
    ("window2_n9_d64", 9, 64, 2, 2),
    ("causal_n5_d128", 5, 128, 1, 0),
    ("window0_n4_d128", 4, 128, 2, 0),
]


def formula_qkv(N: int, d: int):
    """q, k, v as float64 [1, 1, N, d]; entries are multiples of 1/8 in [-6/8, 6/8]
    (q, k) and multiples of 1/4 in [-1, 1] (v)."""
    i = np.arange(N)[:, None]
    c = np.arange(d)[None, :]
    q = (((3 * i + 5 * c + (i * c) % 7 + 1) % 11) - 5) / 8.0
    k = (((7 * i + 2 * c + (3 * i * c) % 5 + 3) % 13) - 6) / 8.0
    v = (((5 * i + 7 * c + (i * c) % 4 + 2) % 9) - 4) / 4.0
    return q[None, None], k[None, None], v[None, None]


def main() -> None:
    out = {"about": __doc__.strip().splitlines()[0], "cases": []}
    for name, N, d, mk, w in CASES:
        q, k, v = formula_qkv(N, d)
        scale = float(np.float32(1.0 / np.sqrt(d)))
        O, L = attention_forward(q, k, v, scale, mk, w)
        out["cases"].append({"name": name, "N": N, "d": d, "mask_kind": mk, "window": w, "scale": scale,
                             "O": O[0, 0].tolist(), "LSE": L[0, 0].tolist()})
    with open(os.path.join(HERE, "formula_cases.json"), "w", encoding="utf-8") as f:
        f.write('{"about": %s,\n "cases": [\n' % json.dumps(out["about"]))
        f.write(",\n".join("  " + json.dumps(c) for c in out["cases"]))
        f.write("\n]}\n")


if __name__ == "__main__":
    main()
