"""Pins for the CPU oracle of block-sparse attention (oracle/attention_block_ref.py):
facts fixed independently of it: brute force at 50 digits, float64 torch SDPA with
a mask expanded from the layout by a Kronecker product, the reductions to the
dense oracle (all-ones layout, with and without the causal mask), the
block-diagonal layout as independent attention within each block, the empty
layout, and per-head layouts.

Every pin is ``pin_*(fwd)`` with fwd(q, k, v, scale, layout, block, causal) -> (O, LSE),
so the pins run against the oracle and against planted mutants of its source."""
from __future__ import annotations

import math

import mpmath
import numpy as np
import torch

from oracle.attention_ref import attention_forward


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _layout(H, nb, density, seed, empty_row=None):
    lay = (np.random.default_rng(seed).random((H, nb, nb)) < density).astype(np.uint8)
    if empty_row is not None:
        lay[:, empty_row, :] = 0
    return lay


def _check_empty_rows(O, L, empty):
    assert np.all(O[..., empty, :] == 0.0) and np.all(np.isneginf(L[..., empty]))


def brute_force_mp(q, k, v, scale, layout, block, causal, dps=50):
    mpmath.mp.dps = dps
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.full((B, H, N), -np.inf)
    sc = mpmath.mpf(float(np.float32(scale)))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if layout[h][i // block][j // block] and (not causal or j <= i)]
                if not keys:
                    continue
                s = {j: sc * mpmath.fsum(mpmath.mpf(float(q[b, h, i, c])) * mpmath.mpf(float(k[b, h, j, c]))
                                         for c in range(d)) for j in keys}
                e = {j: mpmath.exp(s[j]) for j in keys}
                tot = mpmath.fsum(e.values())
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(e[j] * mpmath.mpf(float(v[b, h, j, c])) for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


def pin_block_brute_force(fwd):
    cases = [(1, 2, 7, 3, 2, False, 0.5), (1, 1, 9, 4, 3, True, 0.6), (2, 1, 6, 2, 4, False, 1.0),
             (1, 2, 8, 3, 3, True, 0.4)]
    for n, (B, H, N, d, block, causal, dens) in enumerate(cases):
        nb = -(-N // block)
        lay = _layout(H, nb, dens, 600 + n, empty_row=1 if n == 0 else None)
        q, k, v = (_rand((B, H, N, d), 610 + 3 * n + t) for t in range(3))
        O, L = fwd(q, k, v, 0.7, lay, block, causal)
        Ob, Lb = brute_force_mp(q, k, v, 0.7, lay, block, causal)
        fin = np.isfinite(Lb)
        assert np.array_equal(np.isfinite(L), fin), n
        assert np.max(np.abs(O - Ob)) <= 1e-13, n
        assert np.max(np.abs(L[fin] - Lb[fin])) <= 1e-13, n


def _kron_mask(layout_h, N, block, causal):
    m = torch.kron(torch.as_tensor(layout_h != 0, dtype=torch.int64), torch.ones(block, block, dtype=torch.int64))
    m = m[:N, :N].bool()
    if causal:
        m = m & torch.ones(N, N, dtype=torch.bool).tril()
    return m


def pin_block_sdpa(fwd):
    for n, (N, block, causal, dens) in enumerate([(100, 16, False, 0.3), (130, 32, True, 0.5), (64, 64, False, 1.0),
                                                  (77, 8, True, 0.15)]):
        H, d = 2, 8
        nb = -(-N // block)
        lay = _layout(H, nb, dens, 700 + n)
        q, k, v = (_rand((1, H, N, d), 710 + 3 * n + t) for t in range(3))
        O, L = fwd(q, k, v, 0.3, lay, block, causal)
        s32 = float(np.float32(0.3))
        for h in range(H):
            m = _kron_mask(lay[h], N, block, causal)
            some = m.any(dim=1)
            tq, tk, tv = (torch.from_numpy(x[0, h]).double() for x in (q, k, v))
            Os = torch.nn.functional.scaled_dot_product_attention(tq[some], tk, tv, attn_mask=m[some], scale=s32)
            Ls = torch.logsumexp(((tq[some] @ tk.T) * s32).masked_fill(~m[some], float("-inf")), dim=-1)
            assert np.max(np.abs(O[0, h][some.numpy()] - Os.numpy())) <= 1e-12, (n, h)
            assert np.max(np.abs(L[0, h][some.numpy()] - Ls.numpy())) <= 1e-12, (n, h)
            _check_empty_rows(O[0, h], L[0, h], ~some.numpy())


def pin_block_all_ones_is_dense(fwd):
    """An all-ones layout is full attention; with the causal flag, causal attention."""
    N, d, block = 70, 8, 16
    q, k, v = (_rand((2, 2, N, d), 800 + t) for t in range(3))
    lay = np.ones((2, -(-N // block), -(-N // block)), dtype=np.uint8)
    for causal, mask in ((False, 0), (True, 1)):
        O, L = fwd(q, k, v, 1 / math.sqrt(d), lay, block, causal)
        Od, Ld = attention_forward(q, k, v, 1 / math.sqrt(d), mask, 0)
        assert np.max(np.abs(O - Od)) <= 1e-13 and np.max(np.abs(L - Ld)) <= 1e-13, causal


def pin_block_diagonal_is_independent_blocks(fwd):
    """A block-diagonal layout: each block of the sequence attends only to itself,
    i.e. dense attention run separately on every block (the last one ragged)."""
    N, d, block = 45, 4, 8
    q, k, v = (_rand((1, 1, N, d), 900 + t) for t in range(3))
    nb = -(-N // block)
    lay = np.eye(nb, dtype=np.uint8)[None]
    for causal, mask in ((False, 0), (True, 1)):
        O, L = fwd(q, k, v, 0.5, lay, block, causal)
        for s in range(0, N, block):
            e = min(N, s + block)
            Od, Ld = attention_forward(q[:, :, s:e], k[:, :, s:e], v[:, :, s:e], 0.5, mask, 0)
            assert np.max(np.abs(O[:, :, s:e] - Od)) <= 1e-13 and np.max(np.abs(L[:, :, s:e] - Ld)) <= 1e-13


def pin_block_empty_layout(fwd):
    q, k, v = (_rand((1, 2, 20, 4), 950 + t) for t in range(3))
    O, L = fwd(q, k, v, 0.5, np.zeros((2, 3, 3), dtype=np.uint8), 8, False)
    _check_empty_rows(O, L, np.ones(20, dtype=bool))


def pin_block_heads_use_their_layout(fwd):
    """Each head follows its own layout: head h alone, with layout[h], gives the same."""
    N, d, block = 40, 4, 8
    q, k, v = (_rand((1, 3, N, d), 960 + t) for t in range(3))
    lay = _layout(3, 5, 0.5, 970)
    O, L = fwd(q, k, v, 0.5, lay, block, False)
    for h in range(3):
        Oh, Lh = fwd(q[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 0.5, lay[h:h + 1], block, False)
        assert np.array_equal(O[:, h:h + 1], Oh) and np.array_equal(L[:, h:h + 1], Lh)
    assert not np.allclose(O[:, 0], fwd(q[:, 0:1], k[:, 0:1], v[:, 0:1], 0.5, lay[1:2], block, False)[0][:, 0])


ALL_BLOCK_PINS = [pin_block_brute_force, pin_block_sdpa, pin_block_all_ones_is_dense,
                  pin_block_diagonal_is_independent_blocks, pin_block_empty_layout, pin_block_heads_use_their_layout]
