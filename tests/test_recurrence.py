"""The blockwise online-softmax recurrence (CPU, float64) reaches the plain
definition for every tile shape, ragged N and mask, and visits exactly the key
tiles that hold an allowed key.  CPU only."""
import numpy as np
import pytest

from oracle.attention_ref import allowed_mask, attention_forward
from oracle.recurrence_ref import blockwise_forward, kv_tile_range

NONE, CAUSAL, WINDOW = 0, 1, 2


def _qkv(B, H, N, d, seed, mult=1.0):
    g = np.random.default_rng(seed)
    return (g.standard_normal((B, H, N, d)) * mult, g.standard_normal((B, H, N, d)),
            g.standard_normal((B, H, N, d)))


@pytest.mark.parametrize("br,bc", [(1, 1), (7, 16), (16, 7), (64, 64), (128, 64), (64, 128), (128, 128)])
@pytest.mark.parametrize("mask,w", [(NONE, 0), (CAUSAL, 0), (WINDOW, 0), (WINDOW, 1), (WINDOW, 13), (WINDOW, 64)])
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
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 17)):
        O, L = attention_forward(q, k, v, 1.0 / np.sqrt(32), mask, w)
        Ob, Lb = blockwise_forward(q, k, v, 1.0 / np.sqrt(32), mask, w, block_rows=64, block_cols=32)
        assert np.all(np.isfinite(Ob))
        assert np.max(np.abs(Ob - O)) <= 1e-11
        assert np.max(np.abs(Lb - L)) <= 1e-9


@pytest.mark.parametrize("N", [1, 5, 64, 65, 200, 257])
@pytest.mark.parametrize("br,bc", [(16, 16), (64, 32), (128, 64), (32, 128)])
@pytest.mark.parametrize("mask,w", [(NONE, 0), (CAUSAL, 0), (WINDOW, 0), (WINDOW, 3), (WINDOW, 40), (WINDOW, 1000)])
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
