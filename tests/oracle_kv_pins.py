"""Pins for the CPU oracle of attention with fewer queries than keys
(oracle/attention_kv_ref.py): brute force at 50 digits, float64 torch SDPA with a
rectangular mask built independently, and the reduction to the square oracle
(a suffix of the queries of a full sequence)."""
from __future__ import annotations

import math

import mpmath
import numpy as np
import torch

from oracle.attention_ref import attention_forward

NONE, CAUSAL, WINDOW, CAUSAL_WINDOW = 0, 1, 2, 3


def _rand(shape, seed, mult=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * mult


def _allowed(p, j, mask, w):
    if mask == NONE:
        return True
    if mask == CAUSAL:
        return j <= p
    if mask == CAUSAL_WINDOW:
        return j <= p and p - j <= w
    return abs(p - j) <= w


def brute_force_mp(q, k, v, scale, mask, w, off, dps=50):
    mpmath.mp.dps = dps
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    O = np.zeros((B, H, Nq, d))
    L = np.zeros((B, H, Nq))
    sc = mpmath.mpf(float(np.float32(scale)))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                keys = [j for j in range(Nk) if _allowed(off + i, j, mask, w)]
                s = {j: sc * mpmath.fsum(mpmath.mpf(float(q[b, h, i, c])) * mpmath.mpf(float(k[b, h, j, c]))
                                         for c in range(d)) for j in keys}
                e = {j: mpmath.exp(s[j]) for j in keys}
                tot = mpmath.fsum(e.values())
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(e[j] * mpmath.mpf(float(v[b, h, j, c])) for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


def pin_kv_brute_force(fwd_kv):
    cases = [(1, 1, 1, 7, 4, NONE, 0, 6), (1, 2, 2, 9, 3, CAUSAL, 0, 7), (1, 1, 3, 8, 4, WINDOW, 2, 2),
             (2, 1, 1, 5, 4, CAUSAL_WINDOW, 1, 4), (1, 1, 4, 4, 2, CAUSAL, 0, 0)]
    for n, (B, H, Nq, Nk, d, mask, w, off) in enumerate(cases):
        q = _rand((B, H, Nq, d), 300 + n)
        k, v = (_rand((B, H, Nk, d), 310 + 2 * n + t) for t in range(2))
        O, L = fwd_kv(q, k, v, 0.6, mask, w, off)
        Ob, Lb = brute_force_mp(q, k, v, 0.6, mask, w, off)
        assert np.max(np.abs(O - Ob)) <= 1e-13 and np.max(np.abs(L - Lb)) <= 1e-13, n


def pin_kv_sdpa(fwd_kv):
    for n, (Nq, Nk, mask, w, off) in enumerate([(1, 300, CAUSAL, 0, 299), (16, 257, NONE, 0, 100),
                                                (5, 200, WINDOW, 17, 195), (33, 120, CAUSAL_WINDOW, 40, 80)]):
        d = 16
        q = _rand((1, 2, Nq, d), 400 + n)
        k, v = (_rand((1, 2, Nk, d), 410 + 2 * n + t) for t in range(2))
        O, L = fwd_kv(q, k, v, 0.25, mask, w, off)
        p = torch.arange(Nq)[:, None] + off
        j = torch.arange(Nk)[None, :]
        allow = {NONE: torch.ones(Nq, Nk, dtype=torch.bool), CAUSAL: j <= p, WINDOW: (p - j).abs() <= w,
                 CAUSAL_WINDOW: (j <= p) & (p - j <= w)}[mask]
        tq, tk, tv = (torch.from_numpy(x).double() for x in (q, k, v))
        s32 = float(np.float32(0.25))
        Os = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allow, scale=s32)
        Ls = torch.logsumexp(((tq @ tk.transpose(-1, -2)) * s32).masked_fill(~allow, float("-inf")), dim=-1)
        assert np.max(np.abs(O - Os.numpy())) <= 1e-12 and np.max(np.abs(L - Ls.numpy())) <= 1e-12, n


def pin_kv_suffix_of_full_sequence(fwd_kv):
    """The last Nq queries of a full (square) attention, computed against all keys
    with q_offset = N - Nq, are those rows of the square result."""
    N, d = 50, 8
    q, k, v = (_rand((1, 2, N, d), 500 + t) for t in range(3))
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 6), (CAUSAL_WINDOW, 9)):
        O, L = attention_forward(q, k, v, 1 / math.sqrt(d), mask, w)
        for nq in (1, 7, N):
            Okv, Lkv = fwd_kv(q[:, :, N - nq:], k, v, 1 / math.sqrt(d), mask, w, N - nq)
            assert np.max(np.abs(Okv - O[:, :, N - nq:])) <= 1e-13
            assert np.max(np.abs(Lkv - L[:, :, N - nq:])) <= 1e-13


def pin_kv_single_key(fwd_kv):
    """Position 0 under the causal mask sees only key 0: O = v_0, LSE = scale q.k_0."""
    q = _rand((1, 1, 1, 4), 601)
    k, v = (_rand((1, 1, 9, 4), 602 + t) for t in range(2))
    O, L = fwd_kv(q, k, v, 0.5, CAUSAL, 0, 0)
    assert np.max(np.abs(O[0, 0, 0] - v[0, 0, 0])) <= 1e-15
    assert abs(L[0, 0, 0] - float(np.float32(0.5)) * float(q[0, 0, 0] @ k[0, 0, 0])) <= 1e-14


ALL_KV_PINS = [pin_kv_brute_force, pin_kv_sdpa, pin_kv_suffix_of_full_sequence, pin_kv_single_key]
