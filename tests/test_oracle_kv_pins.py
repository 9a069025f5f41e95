"""The CPU oracle of attention with fewer queries than keys, against its pins."""
import pytest

from oracle.attention_kv_ref import attention_forward_kv
from tests.oracle_kv_pins import ALL_KV_PINS


def _fwd_kv(q, k, v, scale, mask, w, off):
    return attention_forward_kv(q, k, v, scale, mask, w, off)


@pytest.mark.parametrize("pin", ALL_KV_PINS, ids=[p.__name__ for p in ALL_KV_PINS])
def test_kv_oracle_pin(pin):
    pin(_fwd_kv)


MUTANTS = {
    "offset_ignored": ("allowed_mask(rr + q_offset, Nk, mask_kind, window)", "allowed_mask(rr, Nk, mask_kind, window)"),
    "offset_off_by_one": ("allowed_mask(rr + q_offset, Nk, mask_kind, window)",
                          "allowed_mask(rr + q_offset + 1, Nk, mask_kind, window)"),
    "keys_truncated": ("K, V = k[b, h], v[b, h]", "K, V = k[b, h, :Nq], v[b, h, :Nq]"),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_kv_mutant_fails_a_pin(name):
    import os
    import types
    src = open(os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle",
                            "attention_kv_ref.py"), encoding="utf-8").read()
    old, new = MUTANTS[name]
    assert src.count(old) == 1
    mod = types.ModuleType("oracle.kv_mutant")
    mod.__package__ = "oracle"
    exec(compile(src.replace(old, new), "kv_mutant", "exec"), mod.__dict__)
    failed = []
    for pin in ALL_KV_PINS:
        try:
            pin(lambda q, k, v, s, m, w, o: mod.attention_forward_kv(q, k, v, s, m, w, o))
        except (AssertionError, ValueError, IndexError):
            failed.append(pin.__name__)
    assert failed, name
