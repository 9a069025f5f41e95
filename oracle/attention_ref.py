"""Plain CPU float64 oracle for exact multi-head attention forward.

TEST INFRASTRUCTURE ONLY. The product path never imports this module. Only the
test-suite (``tests/``), the package smoke check (``__graft_entry__.smoke``) and
the CPU-baseline leg of ``bench.py`` may import or run it. It shares no code with
the HIP path: no kernels, no headers, no helpers, no constants.

What it computes is the plain definition of attention, written out directly.
For every batch b, head h and query row i (0-based, N queries and N keys):

  A(i)   the allowed key set
           no mask       : every key j
           causal        : j <= i                (diagonal included)
           window        : |i - j| <= w          (inclusive band, clipped at the ends)
           causal window : i - w <= j <= i       (the band's causal half: the w keys
                                                  before a token and the token itself)
  s_ij = scale * sum_c q_ic k_jc                 for j in A(i); other keys are excluded
  m_i  = max_{j in A(i)} s_ij
  p_ij = exp(s_ij - m_i)                         (0 for j outside A(i))
  l_i  = sum_j p_ij
  O_i  = (sum_j p_ij v_j) / l_i
  LSE_i = m_i + ln(l_i)

Passages followed (page title, section):
  * "Transformer多头注意力8头并行计算PyTorch实现与CUDA核函数优化", §1: attention is
    softmax(Q K^T / sqrt(d_k)) V; the 1/sqrt(d_k) factor keeps dot products from
    saturating the softmax.  Here the factor is the explicit ``scale`` argument.
  * same page, §2.2: masked scores are filled with -inf before the softmax, so a
    masked key gets probability exactly 0.
  * "长序列推理中的注意力机制优化策略与实践", §2.1: the sliding window lets a token see
    the w tokens before and after it; the band printed there (a lower-triangular
    cut at +w and an upper-triangular cut at -w of an all-ones matrix) is the
    inclusive band |i - j| <= w.  That page multiplies the scores by the 0/1 band
    instead of excluding masked keys; this oracle excludes them (-inf), as the
    previous page does.
  * "Blockwise Parallel Transformer in PyTorch", the blockwise_attention example
    and the comparison of Full / Sparse / Blockwise: every query block attends to
    all keys, so the blockwise result is the full-attention result.  The oracle
    therefore computes full attention, one block of query rows at a time.
  * Mosaic long-sequence attention page (kwkr.cn), §5.1: NaN on long sequences
    comes from exp overflow in the softmax; the cure is to work in log space.
    Hence the max subtraction and the LSE output.
  * "Blockwise Parallel Transformer in PyTorch", numerical-stability pitfall: a
    blockwise softmax needs its own normalisation (the division by l_i).

The causal mask is not on the pages; it is read as the square, top-left aligned
triangle j <= i.  Float64 throughout: inputs (bf16 or fp32) convert to float64
without loss, and ``scale`` is taken as the float32 value a caller passes across
the C ABI.
"""
from __future__ import annotations

import numpy as np

MASK_NONE = 0
MASK_CAUSAL = 1
MASK_WINDOW = 2
MASK_CAUSAL_WINDOW = 3


def allowed_mask(rows: np.ndarray, n_keys: int, mask_kind: int, window: int) -> np.ndarray:
    """Boolean matrix [len(rows), n_keys]: True where key j is in A(i) for query row i."""
    i = np.asarray(rows, dtype=np.int64)[:, None]
    j = np.arange(n_keys, dtype=np.int64)[None, :]
    if mask_kind == MASK_NONE:
        return np.ones((i.shape[0], n_keys), dtype=bool)
    if mask_kind == MASK_CAUSAL:
        return j <= i
    if mask_kind == MASK_WINDOW:
        if window < 0:
            raise ValueError("window must be >= 0")
        return np.abs(i - j) <= window
    if mask_kind == MASK_CAUSAL_WINDOW:
        if window < 0:
            raise ValueError("window must be >= 0")
        return (j <= i) & (i - j <= window)
    raise ValueError(f"unknown mask kind {mask_kind}")


def _as_f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError(f"oracle takes float arrays (bf16 must be widened to float32 first), got {a.dtype}")
    return a.astype(np.float64, copy=False)


def attention_forward(q, k, v, scale, mask_kind=MASK_NONE, window=0, rows=None,
                      block_rows=256, return_probs=False):
    """Exact attention forward in float64.

    q, k, v : arrays [B, H, N, d] (float16/float32/float64; bf16 widened to float32 by the caller)
    scale   : softmax scale; rounded to float32 first, as the C ABI receives it
    rows    : None (all rows), a 1-D array of query rows shared by every (b, h),
              or an int array [B, H, R] of rows per (b, h)
    Returns (O [B, H, R, d], LSE [B, H, R]) and, if ``return_probs``, P [B, H, R, N].
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    if q.ndim != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must share one shape [B, H, N, d]")
    B, H, N, d = q.shape
    s32 = float(np.float32(scale))

    if rows is None:
        row_sets = np.broadcast_to(np.arange(N, dtype=np.int64), (B, H, N))
    else:
        r = np.asarray(rows, dtype=np.int64)
        row_sets = np.broadcast_to(r, (B, H, r.shape[-1])) if r.ndim == 1 else r
    if row_sets.size and (row_sets.min() < 0 or row_sets.max() >= N):
        raise ValueError("row index out of range")
    R = row_sets.shape[-1]

    out = np.empty((B, H, R, d), dtype=np.float64)
    lse = np.empty((B, H, R), dtype=np.float64)
    probs = np.zeros((B, H, R, N), dtype=np.float64) if return_probs else None

    for b in range(B):
        for h in range(H):
            K = k[b, h]
            V = v[b, h]
            for r0 in range(0, R, block_rows):
                rr = row_sets[b, h, r0:r0 + block_rows]
                S = s32 * (q[b, h, rr] @ K.T)                      # scores of this row block
                S = np.where(allowed_mask(rr, N, mask_kind, window), S, -np.inf)
                m = S.max(axis=1, keepdims=True)                    # row maxima
                P = np.exp(S - m)                                   # exp(-inf) = 0 on masked keys
                l = P.sum(axis=1, keepdims=True)                    # row sums
                out[b, h, r0:r0 + len(rr)] = (P @ V) / l
                lse[b, h, r0:r0 + len(rr)] = (m + np.log(l))[:, 0]
                if return_probs:
                    probs[b, h, r0:r0 + len(rr)] = P / l
    if return_probs:
        return out, lse, probs
    return out, lse

