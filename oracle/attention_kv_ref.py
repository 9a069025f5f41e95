"""Plain CPU float64 oracle for attention with fewer queries than keys (decode and
chunked prefill against a key/value cache).

TEST INFRASTRUCTURE ONLY. The product path never imports this module. Only the
test-suite (``tests/``) and the CPU-baseline leg of ``bench.py`` may import or
run it. It shares no code with the HIP path.

What it computes: the forward map of ``attention_ref`` with Nq query rows and Nk
keys per (batch, head), where query row i sits at sequence position p_i = q_offset
+ i (a chunk of new tokens appended after q_offset cached ones):

  A(i)  keys allowed for position p_i: every key; j <= p_i (causal); |p_i - j| <= w
        (window); p_i - w <= j <= p_i (causal window)
  O_i   = sum_{j in A(i)} softmax_j(scale <q_i, k_j>) v_j,  LSE_i = ln sum_{j in A(i)} exp(...)

Passages followed (page title, section):
  * "长序列推理中的注意力机制优化策略与实践", §4.1: autoregressive inference keeps the
    keys and values of earlier tokens in a cache and computes attention only for
    the new tokens against it.
  * the page on the sparse-attention software stack (ruibaoantu.com), part 2: the
    prefill phase is compute-bound and the decode phase memory-bound, so the two
    paths are separated.
  * the forward definition and masks of ``attention_ref`` (same pages as there).
Reading: the new tokens occupy positions q_offset .. q_offset + Nq - 1 of the
sequence whose keys are the Nk cached ones (q_offset + Nq <= Nk), so every row has
its own position among the keys and A(i) is never empty.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import MASK_NONE, allowed_mask


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError(f"oracle takes float arrays (bf16 must be widened to float32 first), got {a.dtype}")
    return a.astype(np.float64, copy=False)


def attention_forward_kv(q, k, v, scale, mask_kind=MASK_NONE, window=0, q_offset=0, rows=None, block_rows=256):
    """Exact forward in float64 for q [B, H, Nq, d] against k, v [B, H, Nk, d].

    rows : None (all query rows) or a 1-D array of query rows shared by every (b, h).
    Returns (O [B, H, R, d], LSE [B, H, R])."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    if q.ndim != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q [B, H, Nq, d] and k, v [B, H, Nk, d] expected")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if q_offset < 0 or q_offset + Nq > Nk:
        raise ValueError("query positions q_offset .. q_offset + Nq - 1 must lie within the Nk keys")
    s32 = float(np.float32(scale))
    rr_all = np.arange(Nq, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    R = rr_all.shape[0]
    out = np.empty((B, H, R, d))
    lse = np.empty((B, H, R))
    for b in range(B):
        for h in range(H):
            K, V = k[b, h], v[b, h]
            for r0 in range(0, R, block_rows):
                rr = rr_all[r0:r0 + block_rows]
                S = s32 * (q[b, h, rr] @ K.T)
                S = np.where(allowed_mask(rr + q_offset, Nk, mask_kind, window), S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                P = np.exp(S - m)
                l = P.sum(axis=1, keepdims=True)
                out[b, h, r0:r0 + len(rr)] = (P @ V) / l
                lse[b, h, r0:r0 + len(rr)] = (m + np.log(l))[:, 0]
    return out, lse
