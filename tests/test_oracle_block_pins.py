"""The CPU oracle of block-sparse attention, against its pins, and planted mutants
of its source, each of which must fail at least one pin."""
import os
import types

import pytest

from oracle.attention_block_ref import attention_forward_block_sparse
from tests.oracle_block_pins import ALL_BLOCK_PINS


def _fwd(q, k, v, scale, layout, block, causal):
    return attention_forward_block_sparse(q, k, v, scale, layout, block, causal)


@pytest.mark.parametrize("pin", ALL_BLOCK_PINS, ids=[p.__name__ for p in ALL_BLOCK_PINS])
def test_block_oracle_pin(pin):
    pin(_fwd)


MUTANTS = {
    "layout_transposed": ("np.asarray(layout_h)[i // block, j // block]", "np.asarray(layout_h)[j // block, i // block]"),
    "causal_ignored": ("        allowed = allowed & (j <= i)", "        allowed = allowed"),
    "causal_strict": ("allowed & (j <= i)", "allowed & (j < i)"),
    "key_block_from_row": ("np.asarray(layout_h)[i // block, j // block]", "np.asarray(layout_h)[i // block, i // block]"),
    "empty_rows_nan": ("                some = allowed.any(axis=1)", "                some = np.ones(len(rr), dtype=bool)"),
    "head_zero_layout": ("allowed = block_allowed(layout[h], rr, N, block, causal)",
                         "allowed = block_allowed(layout[0], rr, N, block, causal)"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_block_mutant_fails_a_pin(name):
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                            "attention_block_ref.py"), encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1, name
    mod = types.ModuleType("oracle.block_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "block_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in ALL_BLOCK_PINS:
        try:
            pin(lambda q, k, v, s, lay, blk, c: mod.attention_forward_block_sparse(q, k, v, s, lay, blk, c))
        except (AssertionError, ValueError, IndexError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, name
