"""Seeded synthetic inputs and checked-row selection.

Shared by the HIP-path tests, the benchmark and the oracle-side tests; it holds
none of the attention arithmetic.  Inputs are i.i.d. N(0, 1) draws in the
contiguous [B, H, N, d] layout, drawn in the order q, k, v from one seeded
generator, then rounded to the working dtype (round-to-nearest-even for bf16).
A query multiplier (x8 for the overflow stress case) is applied to the float32
draw before rounding; multiplying by a power of two commutes with the rounding.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

MASK_CODES = {"none": 0, "causal": 1, "window": 2, "causal_window": 3}


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    dtype: str          # "f32" or "bf16"
    mask: str           # "none" | "causal" | "window"
    window: int = 0
    scale: float | None = None   # None -> 1/sqrt(d)

    @property
    def mask_kind(self) -> int:
        return MASK_CODES[self.mask]

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(self.scale if self.scale is not None else 1.0 / np.sqrt(self.d)))

    @property
    def torch_dtype(self):
        return torch.float32 if self.dtype == "f32" else torch.bfloat16


# The workloads: a tiny fp32 case, a multi-head non-causal bf16 case, a
# LLaMA-7B-shaped causal case (the headline), a sliding-window case and a
# long-sequence causal case.
WORKLOADS = {
    "tiny_f32_n256": Workload("tiny_f32_n256", 1, 2, 256, 64, "f32", "none"),
    "mh_bf16_n4096_d64": Workload("mh_bf16_n4096_d64", 1, 8, 4096, 64, "bf16", "none", scale=0.125),
    "causal_bf16_b2h32_n8192_d128": Workload("causal_bf16_b2h32_n8192_d128", 2, 32, 8192, 128, "bf16", "causal"),
    "window512_bf16_h32_n32768_d128": Workload("window512_bf16_h32_n32768_d128", 1, 32, 32768, 128, "bf16",
                                               "window", window=512),
    "causal_bf16_h32_n131072_d128": Workload("causal_bf16_h32_n131072_d128", 1, 32, 131072, 128, "bf16", "causal"),
}

HEADLINE = "causal_bf16_b2h32_n8192_d128"


@dataclass(frozen=True)
class KvWorkload:
    """Nq new queries at positions Nk - Nq .. Nk - 1 against Nk cached keys (bf16)."""
    name: str
    B: int
    H: int
    Nq: int
    Nk: int
    d: int
    mask: str
    window: int = 0

    @property
    def mask_kind(self) -> int:
        return MASK_CODES[self.mask]

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))


# Decode steps (one new token per sequence) with LLaMA-7B heads: one long context,
# and a batch of eight 8K contexts.
KV_WORKLOADS = {
    "decode_bf16_h32_nk131072_d128": KvWorkload("decode_bf16_h32_nk131072_d128", 1, 32, 1, 131072, 128, "causal"),
    "decode_bf16_b8h32_nk8192_d128": KvWorkload("decode_bf16_b8h32_nk8192_d128", 8, 32, 1, 8192, 128, "causal"),
}

KV_HEADLINE = "decode_bf16_h32_nk131072_d128"


def make_qkv(B, H, N, d, dtype=torch.bfloat16, seed=0, q_mult=1.0, device="cpu"):
    """q, k, v as contiguous [B, H, N, d] tensors of ``dtype``.

    device="cpu" draws with a CPU generator (bit-reproducible everywhere);
    a CUDA device draws on that device with its own seeded generator, which is
    faster for the large workloads; the oracle then reads the copies."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = []
    for idx in range(3):
        x = torch.randn((B, H, N, d), generator=gen, dtype=torch.float32, device=device)
        if idx == 0 and q_mult != 1.0:
            x.mul_(q_mult)
        out.append(x.to(dtype).contiguous())
    return tuple(out)


def make_q_kv(B, H, Nq, Nk, d, dtype=torch.bfloat16, seed=0, q_mult=1.0, device="cpu"):
    """q [B, H, Nq, d] and k, v [B, H, Nk, d] (queries against a key/value cache),
    drawn like ``make_qkv``: one seeded generator, in the order q, k, v."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    out = []
    for idx, n in enumerate((Nq, Nk, Nk)):
        x = torch.randn((B, H, n, d), generator=gen, dtype=torch.float32, device=device)
        if idx == 0 and q_mult != 1.0:
            x.mul_(q_mult)
        out.append(x.to(dtype).contiguous())
    return tuple(out)


@dataclass(frozen=True)
class SparseWorkload:
    """A block-sparse workload: BigBird-style layout (local band, global and random
    blocks, see ``bigbird_block_layout``) over 128-token blocks, bf16."""
    name: str
    B: int
    H: int
    N: int
    d: int
    local: int
    n_global: int
    n_random: int
    causal: bool = False

    @property
    def softmax_scale(self) -> float:
        return float(np.float32(1.0 / np.sqrt(self.d)))

    def layout(self, seed=0):
        return bigbird_block_layout(self.H, -(-self.N // 128), self.local, self.n_global, self.n_random, seed)


SPARSE_WORKLOADS = {
    "bigbird_bf16_h32_n32768_d128": SparseWorkload("bigbird_bf16_h32_n32768_d128", 1, 32, 32768, 128, 1, 2, 3),
}

SPARSE_HEADLINE = "bigbird_bf16_h32_n32768_d128"


def random_block_layout(H, nb, density, seed, empty_rows=()):
    """uint8 [H, nb, nb]: each block allowed with probability ``density`` (seeded);
    the listed block rows are cleared (query blocks with no allowed key)."""
    lay = (np.random.default_rng(seed).random((H, nb, nb)) < density).astype(np.uint8)
    for r in empty_rows:
        lay[:, r, :] = 0
    return lay


def bigbird_block_layout(H, nb, local=1, n_global=2, n_random=3, seed=0):
    """uint8 [H, nb, nb] of the sparse-attention pattern the long-sequence pages cite
    (Longformer / BigBird): a band of ``local`` blocks on each side of the diagonal,
    ``n_global`` global blocks (the first key blocks for every query block, and every
    key block for the first query blocks), and ``n_random`` seeded random key blocks
    per query block, drawn per head."""
    rng = np.random.default_rng(seed)
    lay = np.zeros((H, nb, nb), dtype=np.uint8)
    for h in range(H):
        for qb in range(nb):
            lay[h, qb, max(0, qb - local):min(nb, qb + local + 1)] = 1
            lay[h, qb, :min(n_global, nb)] = 1
            if n_random:
                lay[h, qb, rng.choice(nb, size=min(n_random, nb), replace=False)] = 1
        lay[h, :min(n_global, nb), :] = 1
    return lay


def forced_rows(N, window=0):
    """Rows always checked, so tile and mask boundaries are covered whatever the
    kernel's tile sizes: both ends, power-of-two boundaries and the window edges."""
    cand = {0, 1, N - 2, N - 1, 15, 16, 31, 32, 63, 64, 127, 128, 255, 256}
    if window > 0:
        cand |= {window - 1, window, window + 1, N - 1 - window, N - window}
    return sorted(r for r in cand if 0 <= r < N)


def sample_rows(N, n_rows, seed, window=0):
    """Sorted, distinct query rows: the forced rows plus seeded draws without
    replacement, ``n_rows`` in total (all rows when n_rows >= N)."""
    if n_rows >= N:
        return np.arange(N, dtype=np.int64)
    forced = forced_rows(N, window)
    rng = np.random.default_rng(seed)
    pool = np.setdiff1d(np.arange(N, dtype=np.int64), np.asarray(forced, dtype=np.int64))
    extra = rng.choice(pool, size=max(0, n_rows - len(forced)), replace=False)
    return np.sort(np.concatenate([np.asarray(forced, dtype=np.int64), extra]))


def row_seed(workload_name, seed, b, h):
    """Deterministic per-(workload, seed, b, h) seed for row sampling."""
    acc = 1469598103934665603
    for ch in f"{workload_name}/{seed}/{b}/{h}".encode():
        acc = ((acc ^ ch) * 1099511628211) & 0xFFFFFFFFFFFFFFFF
    return acc
