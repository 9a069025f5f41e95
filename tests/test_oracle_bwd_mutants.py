"""Planted mistakes in the backward oracle's source must each fail at least one pin
(a textual edit compiled into a throw-away namespace; the real oracle is untouched)."""
import os
import sys
import types

import pytest

from tests.oracle_bwd_pins import ALL_BWD_PINS

SRC_PATH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                        "attention_bwd_ref.py")

MUTANTS = {
    "dv_rows_reversed": ("dv[b, h] += P.T @ dO[rr]", "dv[b, h] += P.T @ dO[rr][::-1]"),
    "dv_half": ("dv[b, h] += P.T @ dO[rr]", "dv[b, h] += 0.5 * (P.T @ dO[rr])"),
    "dp_missing": ("dS = P * (dP - D)", "dS = P * (-D)"),
    "d_term_dropped": ("dS = P * (dP - D)", "dS = P * dP"),
    "d_sign": ("dS = P * (dP - D)", "dS = P * (dP + D)"),
    "dq_scale_dropped": ("dq[b, h, rr] = s32 * (dS @ K)", "dq[b, h, rr] = (dS @ K)"),
    "dk_scale_dropped": ("dk[b, h] += s32 * (dS.T @ Q[rr])", "dk[b, h] += (dS.T @ Q[rr])"),
    "dk_wrong_operand": ("dk[b, h] += s32 * (dS.T @ Q[rr])", "dk[b, h] += s32 * (dS.T @ dO[rr])"),
    "dq_wrong_operand": ("dq[b, h, rr] = s32 * (dS @ K)", "dq[b, h, rr] = s32 * (dS @ V)"),
    "p_unnormalised": ("P = E / E.sum(axis=1, keepdims=True)", "P = E"),
    "mask_ignored": ("S = np.where(allowed_mask(rr, N, mask_kind, window), S, -np.inf)", "S = S"),
    "scale_not_float32": ("s32 = float(np.float32(scale))", "s32 = float(scale) * (1 + 1e-3)"),
    "dv_wrong_head": ("Q, K, V, dO = q[b, h], k[b, h], v[b, h], dout[b, h]",
                      "Q, K, V, dO = q[b, h], k[b, h], v[b, h], dout[b, 0]"),
}


def _mutant_backward(old, new):
    src = open(SRC_PATH, encoding="utf-8").read()
    assert src.count(old) == 1, f"mutation anchor not found once: {old!r}"
    import oracle.attention_ref as fwd_mod
    mod = types.ModuleType("oracle.bwd_mutant")
    mod.__package__ = "oracle"
    sys.modules.setdefault("oracle.attention_ref", fwd_mod)
    exec(compile(src.replace(old, new), "oracle_bwd_mutant", "exec"), mod.__dict__)
    return mod.attention_backward


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_fails_a_pin(name):
    bwd = _mutant_backward(*MUTANTS[name])
    failed = []
    for pin in ALL_BWD_PINS:
        try:
            pin(bwd)
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, f"mutant {name} passes every pin"
