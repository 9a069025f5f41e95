"""Pins for the CPU backward oracle (oracle/attention_bwd_ref.py): checks against
facts fixed by the mathematics, never against the oracle itself.

Every pin is ``pin_*(bwd)`` taking a callable with the oracle's signature, so the
same pins run against the oracle (tests/test_oracle_bwd_pins.py) and against
planted mutants of its source (tests/test_oracle_bwd_mutants.py).
"""
from __future__ import annotations

import numpy as np
import torch

from oracle.attention_ref import attention_forward

NONE, CAUSAL, WINDOW = 0, 1, 2
MASKS = [(NONE, 0), (CAUSAL, 0), (WINDOW, 1), (WINDOW, 3)]


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _loss(q, k, v, dout, scale, mask, w):
    O, _ = attention_forward(q, k, v, scale, mask, w)
    return float(np.sum(O * dout))


def pin_finite_differences(bwd):
    """Central differences of L = sum(O * dO) through the (separately pinned)
    forward oracle, every entry of dQ, dK and dV, on tiny shapes."""
    eps = 1e-6
    for mask, w in MASKS:
        B, H, N, d = 1, 2, 5, 3
        q, k, v, do = (_rand((B, H, N, d), 10 + i + 7 * mask + w) for i in range(4))
        scale = 0.7
        grads = bwd(q, k, v, do, scale, mask, w)
        for which, g in enumerate(grads):
            base = [q, k, v]
            for idx in np.ndindex(B, H, N, d):
                plus = [x.copy() for x in base]
                minus = [x.copy() for x in base]
                plus[which][idx] += eps
                minus[which][idx] -= eps
                fd = (_loss(*plus, do, scale, mask, w) - _loss(*minus, do, scale, mask, w)) / (2 * eps)
                assert abs(fd - g[idx]) <= 1e-6 * max(1.0, abs(fd)), (mask, w, which, idx, fd, g[idx])


def torch_autograd_reference(q, k, v, do, scale, mask, w):
    """float64 torch autograd through softmax(scale Q K^T + bias) V with a boolean
    mask built independently (causal j <= i, band |i - j| <= w)."""
    N = q.shape[2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    if mask == NONE:
        allowed = torch.ones(N, N, dtype=torch.bool)
    elif mask == CAUSAL:
        allowed = j <= i
    else:
        allowed = (i - j).abs() <= w
    tq, tk, tv = (torch.tensor(x, dtype=torch.float64, requires_grad=True) for x in (q, k, v))
    s = float(np.float32(scale))
    scores = (tq @ tk.transpose(-1, -2)) * s
    scores = scores.masked_fill(~allowed, float("-inf"))
    out = torch.softmax(scores, dim=-1) @ tv
    out.backward(torch.tensor(do, dtype=torch.float64))
    return tq.grad.numpy(), tk.grad.numpy(), tv.grad.numpy()


def pin_torch_autograd(bwd):
    for mask, w in MASKS + [(WINDOW, 0), (WINDOW, 40)]:
        for N in (1, 7, 33):
            q, k, v, do = (_rand((2, 2, N, 8), 100 + i + N, 1.5) for i in range(4))
            ref = torch_autograd_reference(q, k, v, do, 0.4, mask, w)
            got = bwd(q, k, v, do, 0.4, mask, w)
            for r, g in zip(ref, got):
                assert np.max(np.abs(r - g)) <= 1e-12 * max(1.0, np.max(np.abs(r))), (mask, w, N)


def pin_zero_upstream(bwd):
    q, k, v = (_rand((1, 2, 9, 4), 3 + i) for i in range(3))
    for mask, w in MASKS:
        for g in bwd(q, k, v, np.zeros_like(q), 0.5, mask, w):
            assert np.all(g == 0.0)


def pin_sum_of_key_gradients_vanishes(bwd):
    """Each softmax row's gradient sums to zero over its keys, so
    sum_j dK_j = scale sum_i q_i sum_j dS_ij = 0 for every (b, h)."""
    for mask, w in MASKS:
        q, k, v, do = (_rand((2, 1, 11, 5), 40 + i + mask + w) for i in range(4))
        _, dk, _ = bwd(q, k, v, do, 0.8, mask, w)
        assert np.max(np.abs(dk.sum(axis=2))) <= 1e-12


def pin_constant_keys(bwd):
    """All keys equal: every row's scores are constant, so P is uniform over the
    allowed keys and the scores carry no gradient to q: dQ = 0 exactly (up to
    rounding), and dV_j = sum_{i: j in A(i)} dO_i / |A(i)|."""
    N, d = 8, 4
    q, v, do = (_rand((1, 1, N, d), 60 + i) for i in range(3))
    k = np.broadcast_to(_rand((1, 1, 1, d), 64), (1, 1, N, d)).copy()
    for mask, w in MASKS:
        dq, _, dv = bwd(q, k, v, do, 0.9, mask, w)
        assert np.max(np.abs(dq)) <= 1e-12
        exp_dv = np.zeros((N, d))
        for i in range(N):
            keys = [j for j in range(N) if (mask == NONE or (mask == CAUSAL and j <= i)
                                            or (mask == WINDOW and abs(i - j) <= w))]
            for j in keys:
                exp_dv[j] += do[0, 0, i] / len(keys)
        assert np.max(np.abs(dv[0, 0] - exp_dv)) <= 1e-12


def pin_linear_in_upstream(bwd):
    q, k, v, do1, do2 = (_rand((1, 2, 10, 6), 80 + i) for i in range(5))
    for mask, w in MASKS:
        g1 = bwd(q, k, v, do1, 0.6, mask, w)
        g2 = bwd(q, k, v, do2, 0.6, mask, w)
        g12 = bwd(q, k, v, 2.0 * do1 - 3.0 * do2, 0.6, mask, w)
        for a, b, c in zip(g1, g2, g12):
            assert np.max(np.abs(c - (2.0 * a - 3.0 * b))) <= 1e-11


def pin_value_gradient_uniform(bwd):
    """Q = 0 gives uniform weights over A(i): dV_j = sum_{i: j in A(i)} dO_i / |A(i)|;
    causal: dV_j = sum_{i >= j} dO_i / (i + 1)."""
    N, d = 9, 3
    k, v, do = (_rand((1, 1, N, d), 90 + i) for i in range(3))
    q = np.zeros((1, 1, N, d))
    _, _, dv = bwd(q, k, v, do, 1.3, CAUSAL, 0)
    exp_dv = np.array([sum(do[0, 0, i] / (i + 1) for i in range(j, N)) for j in range(N)])
    assert np.max(np.abs(dv[0, 0] - exp_dv)) <= 1e-12


def pin_heads_independent(bwd):
    """Each (b, h) is its own problem: computing a head alone gives the same result."""
    q, k, v, do = (_rand((2, 3, 6, 4), 120 + i) for i in range(4))
    full = bwd(q, k, v, do, 0.5, CAUSAL, 0)
    part = bwd(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], do[1:2, 2:3], 0.5, CAUSAL, 0)
    for f, p in zip(full, part):
        assert np.max(np.abs(f[1:2, 2:3] - p)) <= 1e-14


ALL_BWD_PINS = [pin_finite_differences, pin_torch_autograd, pin_zero_upstream,
                pin_sum_of_key_gradients_vanishes, pin_constant_keys, pin_linear_in_upstream,
                pin_value_gradient_uniform, pin_heads_independent]
