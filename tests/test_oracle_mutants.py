"""Planted mistakes in the oracle's own source must each fail at least one pin.

Each mutant is a textual edit of oracle/attention_ref.py (a dropped term, a wrong
sign or index, a transposed operand, an off-by-one in a mask).  The edited source
is compiled into a throw-away namespace on the CPU; the real oracle is untouched.
"""
import os

import numpy as np
import pytest

from tests.oracle_pins import ALL_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "attention_ref.py")

MUTANTS = {
    "scale_dropped": ("S = s32 * (q[b, h, rr] @ K.T)", "S = (q[b, h, rr] @ K.T)"),
    "scores_transposed": ("S = s32 * (q[b, h, rr] @ K.T)", "S = s32 * (K[rr] @ q[b, h].T)"),
    "scale_not_float32": ("s32 = float(np.float32(scale))", "s32 = float(scale)"),
    "causal_flipped": ("return j <= i", "return j >= i"),
    "causal_strict": ("return j <= i", "return j < i"),
    "window_exclusive": ("return np.abs(i - j) <= window", "return np.abs(i - j) < window"),
    "window_one_wider": ("return np.abs(i - j) <= window", "return np.abs(i - j) <= window + 1"),
    "window_one_sided": ("return np.abs(i - j) <= window", "return (j - i <= window) & (j >= i)"),
    "no_max_shift": ("P = np.exp(S - m)", "P = np.exp(S)"),
    "exp2_for_exp": ("P = np.exp(S - m)", "P = np.exp2(S - m)"),
    "no_normalisation": ("out[b, h, r0:r0 + len(rr)] = (P @ V) / l", "out[b, h, r0:r0 + len(rr)] = (P @ V)"),
    "lse_without_max": ("(m + np.log(l))[:, 0]", "(np.log(l))[:, 0]"),
    "lse_log2": ("(m + np.log(l))[:, 0]", "(m + np.log2(l))[:, 0]"),
    "v_wrong_head": ("V = v[b, h]", "V = v[b, 0]"),
    "k_wrong_batch": ("K = k[b, h]", "K = k[0, h]"),
    "q_rows_ignored": ("q[b, h, rr] @ K.T", "q[b, h, :len(rr)] @ K.T"),
}


def _mutant_forward(old, new):
    src = open(SRC_PATH, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    ns = {"__name__": "oracle_mutant"}
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), ns)
    return ns["attention_forward"]


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    fwd = _mutant_forward(*MUTANTS[name])
    caught = []
    with np.errstate(all="ignore"):
        for pin in ALL_PINS:
            try:
                pin(fwd)
            except Exception as exc:  # noqa: BLE001 - any failure of a pin counts
                caught.append((pin.__name__, type(exc).__name__))
                break
    assert caught, f"mutant {name} passed every pin"
