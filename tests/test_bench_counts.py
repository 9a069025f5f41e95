"""bench.py's FLOP convention against the allowed (query, key) pairs counted one by
one on small shapes: 4 d flops per pair for the band masks and the unmasked case;
the causal count is the metric's own convention, half the unmasked count (N^2 / 2
pairs, N / 2 fewer than the N (N + 1) / 2 allowed)."""
import numpy as np
import pytest

import bench


def _pairs(N, mask, w):
    i = np.arange(N)[:, None]
    j = np.arange(N)[None, :]
    if mask == "none":
        ok = np.ones((N, N), bool)
    elif mask == "causal":
        ok = j <= i
    elif mask == "window":
        ok = np.abs(i - j) <= w
    else:
        ok = (j <= i) & (i - j <= w)
    return int(ok.sum())


@pytest.mark.parametrize("N", [1, 2, 7, 64, 257])
@pytest.mark.parametrize("mask,w", [("none", 0), ("causal", 0), ("window", 0), ("window", 3), ("window", 300),
                                    ("causal_window", 0), ("causal_window", 5), ("causal_window", 300)])
def test_counted_flops_match_pair_counts(N, mask, w):
    B, H, d = 2, 3, 64
    got = bench.counted_flops(B, H, N, d, mask, w)
    if mask == "causal":
        assert got == 4 * B * H * d * N * N // 2
        assert 4 * B * H * d * _pairs(N, mask, w) - got == 4 * B * H * d * N // 2
    else:
        assert got == 4 * B * H * d * _pairs(N, mask, w)


def test_counted_flops_rejects_unknown_mask():
    with pytest.raises(ValueError):
        bench.counted_flops(1, 1, 8, 64, "diagonal", 0)
