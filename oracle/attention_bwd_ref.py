"""Plain CPU float64 oracle for the gradients of exact multi-head attention.

TEST INFRASTRUCTURE ONLY. The product path never imports this module. Only the
test-suite (``tests/``) and the CPU-baseline leg of ``bench.py`` may import or
run it. It shares no code with the HIP path.

What it computes: for the forward map of ``attention_ref`` (per batch b, head h,
query row i and allowed key set A(i))

  S_ij = scale <q_i, k_j>   (j in A(i); other keys excluded)
  P_ij = exp(S_ij) / sum_{j' in A(i)} exp(S_ij')
  O_i  = sum_j P_ij v_j

and an upstream gradient dO = dL/dO, the exact gradients of L with respect to q,
k and v.  They follow from the chain rule through the softmax, written out:

  dV_j  = sum_i P_ij dO_i                         (dV = P^T dO)
  dP_ij = <dO_i, v_j>                             (dP = dO V^T)
  D_i   = sum_j P_ij dP_ij  (= <dO_i, O_i>)
  dS_ij = P_ij (dP_ij - D_i)                      (softmax Jacobian; 0 on masked keys)
  dQ_i  = scale sum_j dS_ij k_j                   (dQ = scale dS K)
  dK_j  = scale sum_i dS_ij q_i                   (dK = scale dS^T Q)

Passages followed (page title, section):
  * "Transformer多头注意力8头并行计算PyTorch实现与CUDA核函数优化", §1 and §2.2: the
    forward map (softmax(Q K^T / sqrt(d_k)) V, masked scores -inf).
  * "长序列推理中的注意力机制优化策略与实践", §3.1: FlashAttention recomputes the
    attention in the backward pass instead of storing the N x N matrix; the HIP
    path does that from the saved LSE.  Here P is materialised one block of query
    rows at a time, in float64, from its definition.
  * Mosaic long-sequence attention page (kwkr.cn), §2.2: gradient checkpointing
    with the blockwise computation keeps memory O(N).

The pages do not write the gradient formulas down; they are the derivative of the
forward definition, stated above, with the masked keys excluded exactly as in the
forward.  Float64 throughout; ``scale`` is taken as the float32 value a caller
passes across the C ABI.
"""
from __future__ import annotations

import numpy as np

from .attention_ref import MASK_NONE, allowed_mask


def _f64(x) -> np.ndarray:
    a = np.asarray(x)
    if a.dtype not in (np.float16, np.float32, np.float64):
        raise TypeError(f"oracle takes float arrays (bf16 must be widened to float32 first), got {a.dtype}")
    return a.astype(np.float64, copy=False)


def attention_backward(q, k, v, dout, scale, mask_kind=MASK_NONE, window=0, block_rows=256):
    """Exact gradients (dQ, dK, dV) in float64, each [B, H, N, d].

    q, k, v, dout : arrays [B, H, N, d]
    scale         : softmax scale (rounded to float32 first)
    """
    q, k, v, dout = _f64(q), _f64(k), _f64(v), _f64(dout)
    if q.ndim != 4 or not (q.shape == k.shape == v.shape == dout.shape):
        raise ValueError("q, k, v, dout must share one shape [B, H, N, d]")
    B, H, N, d = q.shape
    s32 = float(np.float32(scale))
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for b in range(B):
        for h in range(H):
            Q, K, V, dO = q[b, h], k[b, h], v[b, h], dout[b, h]
            for r0 in range(0, N, block_rows):
                rr = np.arange(r0, min(N, r0 + block_rows))
                S = s32 * (Q[rr] @ K.T)
                S = np.where(allowed_mask(rr, N, mask_kind, window), S, -np.inf)
                m = S.max(axis=1, keepdims=True)
                E = np.exp(S - m)
                P = E / E.sum(axis=1, keepdims=True)            # softmax rows, 0 on masked keys
                dv[b, h] += P.T @ dO[rr]
                dP = dO[rr] @ V.T
                D = np.sum(P * dP, axis=1, keepdims=True)
                dS = P * (dP - D)
                dq[b, h, rr] = s32 * (dS @ K)
                dk[b, h] += s32 * (dS.T @ Q[rr])
    return dq, dk, dv
