"""CPU float64 emulation of the blockwise (online-softmax) recurrence.

TEST INFRASTRUCTURE ONLY, like ``attention_ref``: only ``tests/`` may use it.
It never checks the GPU. Its job is to show, on the CPU, that the blockwise method
reaches the plain definition in ``attention_ref`` (up to rounding order) for any
tile shape, any ragged N and every mask, with whole tiles skipped where the mask
excludes them. With ``round_p_bf16`` it also predicts the error that rounding the
probabilities to bf16 before the P.V product adds, so GPU tolerances can be read
against it.

The method, as the pages describe it:
  * Mosaic long-sequence attention page (kwkr.cn), §2.2 and §3.2: split the queries
    into blocks; for a query block walk the keys tile by tile, stage each K/V tile
    on chip, fuse score, softmax and the product with V, and divide by the running
    sum once at the end.  The kernel sketched there keeps a sum but never updates
    its maximum; here the maximum is tracked and the old partial results are
    rescaled when it grows, which is what keeps every exp argument <= 0 (§5.1 of
    the same page: exp overflow is the source of NaN; work in log space).
  * "Blockwise Parallel Transformer in PyTorch", pitfalls: a blockwise softmax
    needs its own normalisation.

For a query block and key tiles t = t_lo .. t_hi (tiles wholly outside the mask
are never visited):
  m <- -inf, l <- 0, acc <- 0
  for each visited tile:
      S      = scale * Q_blk K_t^T, with masked entries set to -inf
      m_new  = max(m, rowmax S)
      base   = m_new, or 0 where m_new is still -inf (row saw no allowed key yet)
      alpha  = exp(m - base);  P = exp(S - base)
      l      = alpha * l + rowsum P
      acc    = alpha * acc + P V_t
      m      = m_new
  O = acc / l,  LSE = m + ln l
"""
from __future__ import annotations

import numpy as np

from .attention_ref import MASK_CAUSAL, MASK_CAUSAL_WINDOW, MASK_NONE, MASK_WINDOW, allowed_mask


def kv_tile_range(q0, q1, n_keys, block_cols, mask_kind, window):
    """Inclusive range of key tiles a query block [q0, q1) must visit: every tile
    holding at least one allowed key for some row of the block, and no other."""
    last_tile = (n_keys - 1) // block_cols
    if mask_kind == MASK_NONE:
        return 0, last_tile
    if mask_kind == MASK_CAUSAL:
        return 0, min(last_tile, (q1 - 1) // block_cols)
    if mask_kind == MASK_WINDOW:
        lo_key = max(0, q0 - window)
        hi_key = min(n_keys - 1, q1 - 1 + window)
        return lo_key // block_cols, hi_key // block_cols
    if mask_kind == MASK_CAUSAL_WINDOW:
        # the causal half of the band ("长序列推理中的注意力机制优化策略与实践", §2.1):
        # row i sees keys i - w .. i, so the block's keys run from its first row's
        # lowest key to its last row's own position
        lo_key = max(0, q0 - window)
        hi_key = min(n_keys - 1, q1 - 1)
        return lo_key // block_cols, hi_key // block_cols
    raise ValueError(f"unknown mask kind {mask_kind}")


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """Round values to bf16 the way a kernel holding them in float32 does: first to
    float32 (nearest, ties to even), then to the nearest bf16 (8 significant bits),
    ties to the neighbour whose last kept bit is 0.  Adding 0x7FFF plus the last
    kept bit to the float32 pattern and clearing the low 16 bits does exactly that,
    a carry out of the kept bits stepping into the exponent (1.99609375 -> 2.0).
    Finite inputs only (the probabilities are finite and >= 0)."""
    f = x.astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    u = (u + 0x7FFF + ((u >> 16) & 1)) & 0xFFFF0000
    return u.astype(np.uint32).view(np.float32).astype(np.float64)


def blockwise_forward(q, k, v, scale, mask_kind=MASK_NONE, window=0,
                      block_rows=64, block_cols=64, round_p_bf16=False,
                      return_visits=False):
    """Blockwise attention forward; same arguments and results as
    ``attention_ref.attention_forward`` (all rows).  With ``return_visits`` it also
    returns the number of key tiles visited per (b, h) (work count for tile skipping)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    B, H, N, d = q.shape
    s32 = float(np.float32(scale))
    out = np.empty((B, H, N, d))
    lse = np.empty((B, H, N))
    visits = 0
    for b in range(B):
        for h in range(H):
            for q0 in range(0, N, block_rows):
                q1 = min(q0 + block_rows, N)
                rows = np.arange(q0, q1)
                Qb = q[b, h, q0:q1]
                m = np.full(q1 - q0, -np.inf)
                l = np.zeros(q1 - q0)
                acc = np.zeros((q1 - q0, d))
                t_lo, t_hi = kv_tile_range(q0, q1, N, block_cols, mask_kind, window)
                for t in range(t_lo, t_hi + 1):
                    visits += 1
                    k0, k1 = t * block_cols, min((t + 1) * block_cols, N)
                    S = s32 * (Qb @ k[b, h, k0:k1].T)
                    allow = allowed_mask(rows, N, mask_kind, window)[:, k0:k1]
                    S = np.where(allow, S, -np.inf)
                    m_new = np.maximum(m, S.max(axis=1))
                    base = np.where(np.isneginf(m_new), 0.0, m_new)
                    alpha = np.exp(m - base)
                    P = np.exp(S - base[:, None])
                    l = alpha * l + P.sum(axis=1)
                    if round_p_bf16:
                        P = _round_bf16(P)
                    acc = alpha[:, None] * acc + P @ v[b, h, k0:k1]
                    m = m_new
                out[b, h, q0:q1] = acc / l[:, None]
                lse[b, h, q0:q1] = m + np.log(l)
    if return_visits:
        return out, lse, visits
    return out, lse
