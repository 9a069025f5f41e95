"""GPU parity at the largest sizes the entry points are meant for, on sampled rows:
a million-token sequence (N = 2^20, d = 128) for the forward (causal and causal
window), a decode step against a million-key cache, and a block-sparse layout of
8192 x 8192 blocks (the layout limit).  These exercise the widest index arithmetic
(per-head offsets of N d = 2^27 elements, key tiles past 2^15, the full LDS block
list)."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import bigbird_block_layout, make_q_kv, make_qkv, sample_rows
from oracle.attention_block_ref import attention_forward_block_sparse
from oracle.attention_kv_ref import attention_forward_kv
from oracle.attention_ref import attention_forward
from tests.gpu_util import REL_RMS_BF16, TOL, require_gpu, say, to_np

pytestmark = pytest.mark.gpu
N_MAX = 1 << 20


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _check(out, lse, O_ref, L_ref, rows, label):
    on, ln = to_np(out)[:, :, rows], to_np(lse)[:, :, rows]
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln)), f"{label}: non-finite output"
    d_o = float(np.abs(on - O_ref).max())
    d_l = float(np.abs(ln - L_ref).max())
    num = np.sqrt(((on - O_ref) ** 2).sum(axis=(2, 3)))
    den = np.sqrt((O_ref ** 2).sum(axis=(2, 3)))
    rel = float(np.max(num / np.maximum(den, 1e-300)))
    say(f"  {label}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e} rel_rms={rel:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"] and rel <= REL_RMS_BF16, label


@pytest.mark.parametrize("mask,window", [("causal", 0), ("causal_window", 4096)])
def test_forward_million_tokens(mask, window):
    N, d = N_MAX, 128
    label = f"forward N={N} d={d} {mask} w{window}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(1, 1, N, d, torch.bfloat16, seed=41, device="cuda")
    out, lse = attn.fwd(q, k, v, mask=mask, window=window)
    torch.cuda.synchronize()
    rows = sample_rows(N, 256, seed=42, window=window)
    scale = float(np.float32(d ** -0.5))
    O_ref, L_ref = attention_forward(to_np(q), to_np(k), to_np(v), scale, attn._lib.MASKS[mask], window, rows=rows)
    _check(out, lse, O_ref, L_ref, rows, label)


def test_decode_million_key_cache():
    B, H, Nk, d = 1, 4, N_MAX, 128
    label = f"decode Nk={Nk}"
    say(f"[gpu] {label}")
    q, k, v = make_q_kv(B, H, 1, Nk, d, torch.bfloat16, seed=43, device="cuda")
    out, lse = attn.fwd_kv(q, k, v, mask="causal")
    torch.cuda.synchronize()
    O_ref, L_ref = attention_forward_kv(to_np(q), to_np(k), to_np(v), float(np.float32(d ** -0.5)), 1, 0, Nk - 1)
    _check(out, lse, O_ref, L_ref, np.arange(1), label)


def test_block_sparse_largest_layout():
    N, d = N_MAX, 128
    nb = N // 128                                          # 8192 blocks: the layout limit
    label = f"block-sparse N={N} nb={nb}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(1, 1, N, d, torch.bfloat16, seed=44, device="cuda")
    lay = bigbird_block_layout(1, nb, local=1, n_global=1, n_random=2, seed=45)
    out, lse = attn.fwd_block_sparse(q, k, v, torch.from_numpy(lay).cuda())
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([sample_rows(N, 192, seed=46), np.arange(0, 128, 16)]))   # some global-block rows
    O_ref, L_ref = attention_forward_block_sparse(to_np(q), to_np(k), to_np(v), float(np.float32(d ** -0.5)), lay, 128,
                                                  False, rows=rows)
    _check(out, lse, O_ref, L_ref, rows, label)
