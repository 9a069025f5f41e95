"""Pins for the CPU oracle: checks against facts fixed by the pages and by the
mathematics, never against the oracle itself.

Every pin is a function ``pin_*(fwd)`` taking an attention-forward callable with
the oracle's signature, so the same pins run against the oracle
(tests/test_oracle_pins.py) and against planted mutants of its source
(tests/test_oracle_mutants.py), which must each fail at least one pin.
"""
from __future__ import annotations

import math

import mpmath
import numpy as np
import torch

NONE, CAUSAL, WINDOW, CAUSAL_WINDOW = 0, 1, 2, 3


def _rand(shape, seed, mult=1.0):
    g = np.random.default_rng(seed)
    return g.standard_normal(shape) * mult


def _allowed(i, j, mask, w):
    # Written independently of the oracle: the key set of each mask.
    if mask == NONE:
        return True
    if mask == CAUSAL:
        return j <= i
    if mask == CAUSAL_WINDOW:
        return j <= i and i - j <= w
    return abs(i - j) <= w


# --------------------------------------------------------------------------- brute force
def brute_force_mp(q, k, v, scale, mask, w, dps=50):
    """Scalar loops in mpmath at ``dps`` digits: the attention formula with masked
    keys excluded (attention as softmax(scale Q K^T) V, masked scores -inf)."""
    mpmath.mp.dps = dps
    B, H, N, d = q.shape
    O = np.zeros((B, H, N, d))
    L = np.zeros((B, H, N))
    sc = mpmath.mpf(float(np.float32(scale)))
    for b in range(B):
        for h in range(H):
            for i in range(N):
                keys = [j for j in range(N) if _allowed(i, j, mask, w)]
                s = {j: sc * mpmath.fsum(mpmath.mpf(float(q[b, h, i, c])) * mpmath.mpf(float(k[b, h, j, c]))
                                         for c in range(d)) for j in keys}
                e = {j: mpmath.exp(s[j]) for j in keys}
                tot = mpmath.fsum(e.values())
                for c in range(d):
                    O[b, h, i, c] = float(mpmath.fsum(e[j] * mpmath.mpf(float(v[b, h, j, c])) for j in keys) / tot)
                L[b, h, i] = float(mpmath.log(tot))
    return O, L


def pin_brute_force(fwd):
    cases = [(1, 1, 1, 1, NONE, 0), (1, 2, 2, 4, CAUSAL, 0), (1, 1, 3, 8, WINDOW, 1),
             (2, 1, 5, 4, WINDOW, 0), (1, 1, 16, 4, CAUSAL, 0), (1, 1, 17, 8, WINDOW, 2),
             (1, 1, 17, 1, NONE, 0), (1, 1, 5, 4, WINDOW, 5), (1, 1, 9, 4, CAUSAL_WINDOW, 2),
             (1, 1, 6, 3, CAUSAL_WINDOW, 0)]
    for n, (B, H, N, d, mask, w) in enumerate(cases):
        q, k, v = (_rand((B, H, N, d), 100 + 3 * n + t) for t in range(3))
        scale = 1.0 / math.sqrt(d)
        O, L = fwd(q, k, v, scale, mask, w)
        Ob, Lb = brute_force_mp(q, k, v, scale, mask, w)
        assert np.max(np.abs(O - Ob)) <= 1e-13, f"brute force O, case {n}"
        assert np.max(np.abs(L - Lb)) <= 1e-13, f"brute force LSE, case {n}"


# --------------------------------------------------------------------------- library routine
def sdpa_reference(q, k, v, scale, mask, w):
    """torch's scaled_dot_product_attention on the CPU in float64 (the routine the
    Blockwise Parallel Transformer page recommends), with a boolean mask built
    from the key-set definitions; LSE from torch.logsumexp."""
    N = q.shape[2]
    i = torch.arange(N)[:, None]
    j = torch.arange(N)[None, :]
    if mask == NONE:
        allow = torch.ones(N, N, dtype=torch.bool)
    elif mask == CAUSAL:
        allow = j <= i
    elif mask == CAUSAL_WINDOW:
        allow = (j <= i) & (i - j <= w)
    else:
        allow = (i - j).abs() <= w
    s32 = float(np.float32(scale))
    tq, tk, tv = (torch.from_numpy(np.ascontiguousarray(x)).double() for x in (q, k, v))
    O = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=allow, scale=s32)
    S = (tq @ tk.transpose(-1, -2)) * s32
    L = torch.logsumexp(S.masked_fill(~allow, float("-inf")), dim=-1)
    return O.numpy(), L.numpy()


def pin_sdpa(fwd):
    cases = [(1, 2, 64, 16, NONE, 0), (2, 1, 100, 32, CAUSAL, 0), (1, 2, 97, 8, WINDOW, 7),
             (1, 1, 33, 64, WINDOW, 0), (1, 1, 40, 16, WINDOW, 100), (2, 1, 77, 16, CAUSAL_WINDOW, 9),
             (1, 1, 40, 8, CAUSAL_WINDOW, 100)]
    for n, (B, H, N, d, mask, w) in enumerate(cases):
        q, k, v = (_rand((B, H, N, d), 200 + 3 * n + t) for t in range(3))
        O, L = fwd(q, k, v, 1.0 / math.sqrt(d), mask, w)
        Os, Ls = sdpa_reference(q, k, v, 1.0 / math.sqrt(d), mask, w)
        assert np.max(np.abs(O - Os)) <= 1e-12, f"sdpa O, case {n}"
        assert np.max(np.abs(L - Ls)) <= 1e-12, f"sdpa LSE, case {n}"


# --------------------------------------------------------------------------- closed forms
def pin_zero_query(fwd):
    """Q = 0: every allowed score is 0, so the weights are uniform over A(i):
    O_i is the mean of the allowed V rows and LSE_i = ln |A(i)|."""
    N, d, w = 37, 8, 4
    v = _rand((1, 1, N, d), 7)
    k = _rand((1, 1, N, d), 8)
    q = np.zeros((1, 1, N, d))
    for mask in (NONE, CAUSAL, WINDOW, CAUSAL_WINDOW):
        O, L = fwd(q, k, v, 0.3, mask, w)
        for i in range(N):
            keys = [j for j in range(N) if _allowed(i, j, mask, w)]
            assert np.max(np.abs(O[0, 0, i] - v[0, 0, keys].mean(axis=0))) <= 1e-14
            assert abs(L[0, 0, i] - math.log(len(keys))) <= 1e-14


def pin_constant_v(fwd):
    """Every V row equal to c: O_i = c for every query, whatever Q, K and mask."""
    N, d = 29, 16
    c = _rand((d,), 9)
    v = np.broadcast_to(c, (2, 1, N, d)).copy()
    q, k = _rand((2, 1, N, d), 10, 3.0), _rand((2, 1, N, d), 11)
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 3)):
        O, _ = fwd(q, k, v, 0.25, mask, w)
        assert np.max(np.abs(O - c)) <= 1e-13


def pin_dominant_score(fwd):
    """One allowed key scores above every other by a gap >= 40: O_i = v_{j*} and
    LSE_i = s_{ij*}, both within |A(i)| e^-40 max|v| (and |A(i)| e^-40)."""
    N, d = 24, 8
    rng = np.random.default_rng(12)
    q = np.zeros((1, 1, N, d))
    k = np.zeros((1, 1, N, d))
    v = rng.standard_normal((1, 1, N, d))
    # key j carries the one-hot direction (j mod d) with weight (j // d) + 1
    for j in range(N):
        k[0, 0, j, j % d] = 1.0 + j // d
    for i in range(N):
        q[0, 0, i, i % d] = 60.0
    scale = 1.0
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 9)):
        O, L = fwd(q, k, v, scale, mask, w)
        for i in range(N):
            keys = [j for j in range(N) if _allowed(i, j, mask, w)]
            s = {j: 60.0 * k[0, 0, j, i % d] for j in keys}
            best = max(keys, key=lambda j: s[j])
            gap = s[best] - max([s[j] for j in keys if j != best], default=-np.inf)
            assert gap >= 40
            bound = len(keys) * math.exp(-40)
            assert np.max(np.abs(O[0, 0, i] - v[0, 0, best])) <= bound * np.max(np.abs(v)) + 1e-15
            assert abs(L[0, 0, i] - s[best]) <= bound + 1e-13


def pin_large_scores_finite(fwd):
    """Scores in the thousands (exp would overflow without the max shift): the
    result must be finite and equal to the arg-max row, with LSE equal to the
    largest score (log-space computation, Mosaic page §5.1)."""
    N, d = 16, 4
    k = np.zeros((1, 1, N, d))
    q = np.zeros((1, 1, N, d))
    for j in range(N):
        k[0, 0, j, j % d] = 1.0 + j // d      # same-residue keys differ by 1000 after scaling
    for i in range(N):
        q[0, 0, i, i % d] = 1000.0
    v = _rand((1, 1, N, d), 14)
    for mask, w in ((NONE, 0), (CAUSAL, 0), (WINDOW, 6)):
        O, L = fwd(q, k, v, 1.0, mask, w)
        assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
        for i in range(N):
            keys = [j for j in range(N) if _allowed(i, j, mask, w) and j % d == i % d]
            best = max(keys)
            assert np.max(np.abs(O[0, 0, i] - v[0, 0, best])) <= 1e-12
            assert abs(L[0, 0, i] - 1000.0 * (1.0 + best // d)) <= 1e-9


# --------------------------------------------------------------------------- invariants
def pin_probabilities(fwd):
    """P rows sum to 1, P >= 0, and P is exactly 0 on masked keys."""
    N, d, w = 40, 8, 5
    q, k, v = (_rand((1, 2, N, d), 15 + t) for t in range(3))
    for mask in (NONE, CAUSAL, WINDOW):
        O, L, P = fwd(q, k, v, 0.5, mask, w, return_probs=True)
        assert np.all(P >= 0)
        assert np.max(np.abs(P.sum(axis=-1) - 1.0)) <= 1e-12
        for i in range(N):
            for j in range(N):
                if not _allowed(i, j, mask, w):
                    assert np.all(P[:, :, i, j] == 0.0)
        # and O is P V
        assert np.max(np.abs(O - P @ v)) <= 1e-12


def pin_special_cases(fwd):
    """w = 0 gives O = V and LSE_i = scale q_i.k_i; w >= N-1 gives the unmasked
    result; causal row 0 gives v_0; N = 1 gives O = V, LSE = scale q.k."""
    N, d = 21, 8
    q, k, v = (_rand((1, 1, N, d), 20 + t) for t in range(3))
    O, L = fwd(q, k, v, 0.7, WINDOW, 0)
    assert np.max(np.abs(O - v)) <= 1e-15
    s32 = float(np.float32(0.7))
    assert np.max(np.abs(L[0, 0] - s32 * np.einsum("nd,nd->n", q[0, 0], k[0, 0]))) <= 1e-14
    On, Ln = fwd(q, k, v, 0.7, NONE, 0)
    for w in (N - 1, N, 10 * N):
        Ow, Lw = fwd(q, k, v, 0.7, WINDOW, w)
        assert np.max(np.abs(Ow - On)) <= 1e-14 and np.max(np.abs(Lw - Ln)) <= 1e-14
    Oc, _ = fwd(q, k, v, 0.7, CAUSAL, 0)
    assert np.max(np.abs(Oc[0, 0, 0] - v[0, 0, 0])) <= 1e-15
    # the causal window: w = 0 sees only the diagonal, w >= N - 1 is plain causal
    Ocw0, Lcw0 = fwd(q, k, v, 0.7, CAUSAL_WINDOW, 0)
    assert np.max(np.abs(Ocw0 - v)) <= 1e-15 and np.max(np.abs(Lcw0 - L)) <= 1e-14
    for w in (N - 1, 5 * N):
        Ocw, _ = fwd(q, k, v, 0.7, CAUSAL_WINDOW, w)
        assert np.max(np.abs(Ocw - Oc)) <= 1e-14
    # the last causal row sees every key
    assert np.max(np.abs(Oc[0, 0, N - 1] - On[0, 0, N - 1])) <= 1e-14
    q1, k1, v1 = q[:, :, :1], k[:, :, :1], v[:, :, :1]
    for mask in (NONE, CAUSAL, WINDOW):
        O1, L1 = fwd(q1, k1, v1, 0.7, mask, 0)
        assert np.max(np.abs(O1 - v1)) <= 1e-15
        assert abs(L1[0, 0, 0] - s32 * float(q1[0, 0, 0] @ k1[0, 0, 0])) <= 1e-14


def pin_key_shift(fwd):
    """k_j += c for every j shifts row i's scores by scale q_i.c: O is unchanged
    and LSE_i grows by exactly that amount."""
    N, d, w = 33, 8, 6
    q, k, v = (_rand((1, 1, N, d), 30 + t) for t in range(3))
    c = _rand((d,), 33)
    s32 = float(np.float32(0.4))
    for mask in (NONE, CAUSAL, WINDOW):
        O, L = fwd(q, k, v, 0.4, mask, w)
        O2, L2 = fwd(q, k + c, v, 0.4, mask, w)
        assert np.max(np.abs(O2 - O)) <= 1e-12
        assert np.max(np.abs(L2[0, 0] - L[0, 0] - s32 * (q[0, 0] @ c))) <= 1e-12


def pin_structure(fwd):
    """No mask: permuting (k_j, v_j) jointly leaves O unchanged; permuting query rows
    permutes O's rows; O is linear in V; heads and batches are independent."""
    N, d = 30, 8
    q, k, v = (_rand((2, 3, N, d), 40 + t) for t in range(3))
    perm = np.random.default_rng(43).permutation(N)
    O, L = fwd(q, k, v, 0.5, NONE, 0)
    Op, Lp = fwd(q, k[:, :, perm], v[:, :, perm], 0.5, NONE, 0)
    assert np.max(np.abs(Op - O)) <= 1e-13 and np.max(np.abs(Lp - L)) <= 1e-13
    Oq, Lq = fwd(q[:, :, perm], k, v, 0.5, NONE, 0)
    assert np.max(np.abs(Oq - O[:, :, perm])) <= 1e-13
    v2 = _rand(v.shape, 44)
    for mask in (NONE, CAUSAL, WINDOW):
        Oa, _ = fwd(q, k, 2.0 * v - 3.0 * v2, 0.5, mask, 3)
        O1, _ = fwd(q, k, v, 0.5, mask, 3)
        O2, _ = fwd(q, k, v2, 0.5, mask, 3)
        assert np.max(np.abs(Oa - (2.0 * O1 - 3.0 * O2))) <= 1e-12
    # (b, h) independence: one head alone gives the same result
    Oh, Lh = fwd(q[1:2, 2:3], k[1:2, 2:3], v[1:2, 2:3], 0.5, NONE, 0)
    assert np.max(np.abs(Oh - O[1:2, 2:3])) <= 1e-14


def pin_window_band_vs_page(fwd):
    """The window band printed on the sliding-window page: an all-ones n x n matrix
    cut with tril(diagonal=w) then triu(diagonal=-w).  With V = identity-like
    one-hot rows and Q = 0, O_i is uniform over exactly the allowed keys, so the
    oracle's support must equal that band."""
    for n, w in ((8, 2), (13, 0), (13, 1), (9, 8), (6, 20)):
        band = torch.ones(n, n).tril(diagonal=w).triu(diagonal=-w).numpy() > 0
        q = np.zeros((1, 1, n, n))
        k = np.zeros((1, 1, n, n))
        v = np.eye(n)[None, None]
        O, _ = fwd(q, k, v, 1.0, WINDOW, w)
        assert np.array_equal(O[0, 0] > 0, band)


def pin_row_subset(fwd):
    """Computing a subset of rows gives those rows of the full result."""
    N, d = 50, 8
    q, k, v = (_rand((1, 2, N, d), 50 + t) for t in range(3))
    rows = np.array([0, 7, 8, 31, 49])
    for mask in (NONE, CAUSAL, WINDOW):
        O, L = fwd(q, k, v, 0.5, mask, 4)
        Os, Ls = fwd(q, k, v, 0.5, mask, 4, rows=rows)
        assert np.max(np.abs(Os - O[:, :, rows])) <= 1e-15
        assert np.max(np.abs(Ls - L[:, :, rows])) <= 1e-15


ALL_PINS = [pin_brute_force, pin_sdpa, pin_zero_query, pin_constant_v, pin_dominant_score,
            pin_large_scores_finite, pin_probabilities, pin_special_cases, pin_key_shift,
            pin_structure, pin_window_band_vs_page, pin_row_subset]
