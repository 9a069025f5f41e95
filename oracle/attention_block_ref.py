"""Plain CPU float64 oracle for block-sparse exact attention.

TEST INFRASTRUCTURE ONLY. The product path never imports this module. Only the
test-suite (``tests/``) and the CPU-baseline leg of ``bench.py`` may import or
run it. It shares no code with the HIP path.

What it computes: exact attention (the forward map of ``attention_ref``) in which
the allowed key set of query row i of head h is given by a block layout, a 0/1
matrix over (query block, key block) pairs of ``block`` x ``block`` tokens:

  A(i) = { j : layout[h, i // block, j // block] != 0 }           (causal=False)
  A(i) = { j : layout[h, i // block, j // block] != 0 and j <= i } (causal=True)
  s_ij = scale <q_i, k_j>,  O_i = sum_{j in A(i)} softmax_j(s_ij) v_j,
  LSE_i = ln sum_{j in A(i)} exp(s_ij)

The layout is shared by the batch and may differ per head.

Passages followed (page title, section):
  * Mosaic long-sequence attention page (kwkr.cn), §6: beyond about 100K tokens the
    attention matrix shows a block-sparse structure.
  * "长序列推理中的注意力机制优化策略与实践", §2.1: sparse attention lets a token attend
    only to the most relevant part of the sequence (Longformer, BigBird); §7: on
    AMD MI250X, block-sparse attention is the preferred configuration.
  * "万亿参数大模型Day-0适配实践与稀疏注意力优化", §二, item 1: an index selection
    decides which tokens take part in the attention, and the KV cache is laid out
    in blocks for the hardware's access pattern.
  * the forward definition of ``attention_ref`` (same passages as there), with the
    masked keys excluded (score -inf, probability 0).

Readings: the layout is a boolean over fixed-size square blocks (the pages name
no format); with ``causal`` the layout is intersected with j <= i; a row whose
allowed set is empty (its block row holds no allowed block) has no softmax, and
its output is taken as O = 0 and LSE = ln 0 = -inf (the value of an empty sum).
"""
from __future__ import annotations

import numpy as np


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError(f"oracle takes float arrays (bf16 must be widened to float32 first), got {a.dtype}")
    return a.astype(np.float64, copy=False)


def block_allowed(layout_h, rows, n_keys, block, causal):
    """Boolean [len(rows), n_keys]: key j allowed for query row i under one head's layout."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    allowed = np.asarray(layout_h)[i // block, j // block] != 0
    if causal:
        allowed = allowed & (j <= i)
    return allowed


def attention_forward_block_sparse(q, k, v, scale, layout, block=128, causal=False, rows=None, block_rows=256):
    """Exact block-sparse forward in float64.

    q, k, v : arrays [B, H, N, d]
    layout  : array [H, ceil(N / block), ceil(N / block)], nonzero = allowed block
    rows    : None (all rows) or a 1-D array of query rows shared by every (b, h)
    Returns (O [B, H, R, d], LSE [B, H, R])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape):
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    B, H, N, d = q.shape
    nb = -(-N // block)
    layout = np.asarray(layout)
    if layout.shape != (H, nb, nb):
        raise ValueError(f"layout must be [H, {nb}, {nb}] for N = {N} and block = {block}")
    s32 = float(np.float32(scale))
    rr_all = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rr_all.shape[0]
    out = np.zeros((B, H, R, d))
    lse = np.full((B, H, R), -np.inf)
    for b in range(B):
        for h in range(H):
            K, V = k[b, h], v[b, h]
            for r0 in range(0, R, block_rows):
                rr = rr_all[r0:r0 + block_rows]
                allowed = block_allowed(layout[h], rr, N, block, causal)
                some = allowed.any(axis=1)             # rows with at least one allowed key
                if not some.any():
                    continue
                S = s32 * (q[b, h, rr[some]] @ K.T)
                S = np.where(allowed[some], S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                l = P.sum(axis=1, keepdims=True)
                idx = np.arange(r0, r0 + len(rr))[some]
                out[b, h, idx] = (P @ V) / l
                lse[b, h, idx] = (m + np.log(l))[:, 0]
    return out, lse
