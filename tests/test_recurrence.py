"""The blockwise online-softmax recurrence (CPU, float64) reaches the plain
definition for every tile shape, ragged N and mask (the causal window included),
and visits exactly the key tiles that hold an allowed key; its bf16 rounding
helper rounds to nearest, ties to even.  CPU only."""
import os

import numpy as np
import pytest
import torch

from oracle.attention_ref import allowed_mask, attention_forward
from oracle.recurrence_ref import _round_bf16, blockwise_forward, kv_tile_range

NONE, CAUSAL, WINDOW, CAUSAL_WINDOW = 0, 1, 2, 3


def _qkv(B, H, N, d, seed, mult=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, d)) * mult, g.standard_normal((B, H, N, d)),
            g.standard_normal((B, H, N, d)))


@pytest.mark.parametrize("br,bc", [(1, 1), (7, 16), (16, 7), (64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("mask,w", [(NONE, 0), (CAUSAL, 0), (WINDOW, 0), (WINDOW, 1), (WINDOW, 13), (WINDOW, 64),
                                    (CAUSAL_WINDOW, 0), (CAUSAL_WINDOW, 1), (CAUSAL_WINDOW, 15), (CAUSAL_WINDOW, 16),
                                    (CAUSAL_WINDOW, 63), (CAUSAL_WINDOW, 64), (CAUSAL_WINDOW, 200)])
def test_recurrence_equals_definition(br, bc, mask, w):
    N = 131 if br > 1 else 37   # ragged with respect to every tile size
    q, k, v = _qkv(1, 2, N, 16, seed=br * 1000 + bc + w, mult=2.0)
    O, L = attention_forward(q, k, v, 0.25, mask, w)
    Ob, Lb = blockwise_forward(q, k, v, 0.25, mask, w, block_rows=br, block_cols=bc)
    assert np.max(np.abs(Ob - O)) <= 1e-12
    assert np.max(np.abs(Lb - L)) <= 1e-12


def test_recurrence_overflow_stress():
    # Q x 8 style: large scores, the running max must keep every exp argument <= 0
    q, k, v = _qkv(1, 1, 200, 32, seed=5, mult=40.0)
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 17), (CAUSAL_WINDOW, 17)):
        O, L = attention_forward(q, k, v, 1.0 / np.sqrt(32), mask, w)
        Ob, Lb = blockwise_forward(q, k, v, 1.0 / np.sqrt(32), mask, w, block_rows=64, block_cols=32)
        assert np.all(np.isfinite(Ob))
        assert np.max(np.abs(Ob - O)) <= 1e-11
        assert np.max(np.abs(Lb - L)) <= 1e-9


@pytest.mark.parametrize("N", [1, 5, 64, 65, 200, 257])
@pytest.mark.parametrize("br,bc", [(16, 16), (64, 32), (128, 64), (32, 128)])
@pytest.mark.parametrize("mask,w", [(NONE, 0), (CAUSAL, 0), (WINDOW, 0), (WINDOW, 3), (WINDOW, 40), (WINDOW, 1000),
                                    (CAUSAL_WINDOW, 0), (CAUSAL_WINDOW, 1), (CAUSAL_WINDOW, 15), (CAUSAL_WINDOW, 16),
                                    (CAUSAL_WINDOW, 31), (CAUSAL_WINDOW, 32), (CAUSAL_WINDOW, 33), (CAUSAL_WINDOW, 40),
                                    (CAUSAL_WINDOW, 127), (CAUSAL_WINDOW, 128), (CAUSAL_WINDOW, 1000)])
def test_tile_range_is_exact(N, br, bc, mask, w):
    """Visited tiles are exactly those holding at least one allowed key for some
    row of the query block (whole-tile skipping loses nothing, wastes nothing)."""
    for q0 in range(0, N, br):
        q1 = min(q0 + br, N)
        allow = allowed_mask(np.arange(q0, q1), N, mask, w)
        need = sorted({j // bc for j in np.nonzero(allow.any(axis=0))[0]})
        lo, hi = kv_tile_range(q0, q1, N, bc, mask, w)
        assert list(range(lo, hi + 1)) == need


def test_bf16_probability_rounding_budget():
    """Rounding P to bf16 before P.V (as a bf16 MFMA does) stays far inside the
    2e-2 bf16 output bound at the small workloads' shapes."""
    q, k, v = _qkv(1, 2, 512, 64, seed=9)
    O, L = attention_forward(q, k, v, 0.125, NONE, 0)
    Ob, Lb = blockwise_forward(q, k, v, 0.125, NONE, 0, block_rows=128, block_cols=64, round_p_bf16=True)
    err = np.max(np.abs(Ob - O))
    assert err < 2e-3, err
    assert np.max(np.abs(Lb - L)) <= 1e-12   # l is summed before rounding


def test_causal_window_tile_range_by_hand():
    """Causal window, 32-key tiles, 128-row blocks, w = 40: the block of rows
    128..255 needs keys 88..255, i.e. tiles 2..7; the first block needs keys 0..127
    (tiles 0..3); a window wider than the sequence reduces to the causal range."""
    assert kv_tile_range(128, 256, 1024, 32, CAUSAL_WINDOW, 40) == (2, 7)
    assert kv_tile_range(0, 128, 1024, 32, CAUSAL_WINDOW, 40) == (0, 3)
    assert kv_tile_range(512, 640, 1024, 32, CAUSAL_WINDOW, 5000) == kv_tile_range(512, 640, 1024, 32, CAUSAL, 0)
    # w = 0: only the block's own diagonal tiles
    assert kv_tile_range(96, 100, 1024, 32, CAUSAL_WINDOW, 0) == (3, 3)
    # ragged last block: rows 960..999 of N = 1000 see keys 960 - w .. 999
    assert kv_tile_range(960, 1000, 1000, 32, CAUSAL_WINDOW, 64) == (28, 31)


# ---------------------------------------------------------------- the bf16 rounding helper
# Values that are exact in float32, with the bf16 value round-to-nearest-even gives
# them, worked out from the definition: bf16 keeps 8 significant bits, so between
# 1 and 2 its spacing is 2**-7, and a value exactly half way between two neighbours
# goes to the one whose last kept bit is 0.
_F32_CASES = [
    (1.0, 1.0),
    (1 + 2.0 ** -8, 1.0),                                  # tie: 1.0 (last bit 0) over 1 + 2**-7
    (1 + 3 * 2.0 ** -8, 1 + 2.0 ** -6),                    # tie: 1 + 2**-7 has last bit 1
    (1 + 2.0 ** -8 + 2.0 ** -20, 1 + 2.0 ** -7),           # just above the tie
    (1 + 2.0 ** -8 - 2.0 ** -20, 1.0),                     # just below the tie
    (2 - 2.0 ** -8, 2.0),                                  # tie with carry into the exponent
    (255.5, 256.0),                                        # 255 = 1.1111111b x 2**7 is odd
    (254.5, 254.0),                                        # 254 is even
    (-(1 + 2.0 ** -8), -1.0),                              # sign is kept
    (0.0, 0.0),
    (2.0 ** -134, 0.0),                                    # half the smallest bf16 subnormal: to 0
    (3 * 2.0 ** -134, 2.0 ** -132),                        # subnormal tie: 2**-133 is odd
    (5 * 2.0 ** -134, 2.0 ** -132),                        # subnormal tie: 2**-132 is even
    (2.0 ** -126 * (1 + 2.0 ** -8), 2.0 ** -126),          # smallest normal, tie
    ((2 - 2.0 ** -8) * 2.0 ** 127, float("inf")),          # above the largest bf16: tie rounds to inf
    ((2 - 2.0 ** -7) * 2.0 ** 127, (2 - 2.0 ** -7) * 2.0 ** 127),   # the largest bf16 itself
]


def _pin_round_bf16(fn):
    got = fn(np.array([x for x, _ in _F32_CASES], dtype=np.float64))
    want = np.array([y for _, y in _F32_CASES], dtype=np.float64)
    assert np.array_equal(got, want), (got, want)
    # Against torch's float32 -> bfloat16 conversion (round to nearest even) on bit
    # patterns dense in ties and near-ties, normal and subnormal, both signs.
    g = np.random.default_rng(11)
    hi = g.integers(0, 1 << 16, size=20000, dtype=np.uint64)
    hi = hi[(hi & 0x7F80) != 0x7F80]                       # no inf / NaN exponents
    lo = np.concatenate([np.full(hi.size // 4, 0x8000), np.full(hi.size // 4, 0x7FFF),
                         np.full(hi.size // 4, 0x8001),
                         g.integers(0, 1 << 16, size=hi.size - 3 * (hi.size // 4))]).astype(np.uint64)
    bits = ((hi << 16) | lo).astype(np.uint32)
    f32 = bits.view(np.float32)
    ref = torch.from_numpy(f32.copy()).to(torch.bfloat16).to(torch.float64).numpy()
    got = fn(f32.astype(np.float64))
    same = (got == ref) | (np.isnan(got) & np.isnan(ref))
    assert same.all(), f32[~same][:8]


def test_round_bf16_pinned():
    _pin_round_bf16(_round_bf16)


_RB_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "recurrence_ref.py")
_RB_ANCHOR = "u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000"
_RB_MUTANTS = {
    "half_up": "u = (u + 0x8000) & 0xFFFF0000",
    "truncate": "u = u & 0xFFFF0000",
    "half_down": "u = (u + 0x7FFF) & 0xFFFF0000",
    "ties_to_odd": "u = (u + 0x7FFF + (1 - ((u >> 16) & 1))) & 0xFFFF0000",
    "parity_of_wrong_bit": "u = (u + 0x7FFF + ((u >> 15) & 1)) & 0xFFFF0000",
}


@pytest.mark.parametrize("name", sorted(_RB_MUTANTS))
def test_round_bf16_mutant_is_caught(name):
    src = open(_RB_SRC, encoding="utf-8").read()
    assert src.count(_RB_ANCHOR) == 1
    ns = {"__name__": "oracle.recurrence_mutant", "__package__": "oracle"}
    exec(compile(src.replace(_RB_ANCHOR, _RB_MUTANTS[name]), "recurrence_mutant", "exec"), ns)
    with pytest.raises(AssertionError):
        _pin_round_bf16(ns["_round_bf16"])
