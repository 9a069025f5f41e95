"""attn_fwd_kv_noalloc (the split-KV forward whose partials live in the library's
static device array) against attn_fwd_kv with a caller workspace, through the C
ABI: two calls in a row, the second with a smaller input, each bit-identical to
the workspace entry point's result (same kernels, same plan) and within the bf16
bar of the float64 oracle; a shape over the scratch limit is rejected."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_q_kv
from oracle.attention_kv_ref import attention_forward_kv
from tests.gpu_util import TOL, require_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run_both(B, H, Nq, Nk, d, mask, window, seed):
    """Both entry points on one seeded input; returns the scratch bytes the shape uses."""
    q, k, v = make_q_kv(B, H, Nq, Nk, d, torch.bfloat16, seed=seed)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    scale = float(np.float32(d ** -0.5))
    mk = attn._lib.MASKS[mask]
    q_off = Nk - Nq
    stream = torch.cuda.current_stream().cuda_stream
    need = attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d)
    assert 0 < need <= attn._lib.ATTN_NOALLOC_SCRATCH_BYTES
    say(f"[gpu] noalloc B{B} H{H} Nq{Nq} Nk{Nk} d{d} {mask} w{window} scratch {need} bytes")
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o_ws, l_ws = torch.empty_like(qd), torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    st = attn.attn_fwd_kv(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_ws.data_ptr(), l_ws.data_ptr(), B, H, Nq,
                          Nk, d, scale, mk, window, q_off, attn.ATTN_DTYPE_BF16, ws.data_ptr(), need, stream)
    assert st == 0, attn.attn_strerror(st)
    o_na, l_na = torch.full_like(qd, 7.0), torch.full((B, H, Nq), 7.0, device="cuda")
    st = attn.attn_fwd_kv_noalloc(qd.data_ptr(), kd.data_ptr(), vd.data_ptr(), o_na.data_ptr(), l_na.data_ptr(), B,
                                  H, Nq, Nk, d, scale, mk, window, q_off, attn.ATTN_DTYPE_BF16, stream)
    assert st == 0, attn.attn_strerror(st)
    torch.cuda.synchronize()
    assert torch.equal(o_na, o_ws), "O differs from attn_fwd_kv"
    assert torch.equal(l_na, l_ws), "LSE differs from attn_fwd_kv"
    O, L = attention_forward_kv(to_np(q), to_np(k), to_np(v), scale, mk, window, q_off)
    d_o = float(np.abs(to_np(o_na) - O).max())
    d_l = float(np.abs(to_np(l_na) - L).max())
    say(f"  noalloc: bit-identical to attn_fwd_kv; max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"]
    return need


@pytest.mark.parametrize("first,second", [
    ((1, 32, 256, 20000, 128, "causal", 0), (1, 8, 100, 3000, 128, "causal", 0)),      # chunks: big, then smaller
    ((2, 16, 1, 50000, 64, "window", 700), (1, 4, 1, 4000, 64, "causal", 0)),           # decode: big, then smaller
])
def test_noalloc_matches_workspace_entry_point(first, second):
    big = _run_both(*first, seed=1)
    small = _run_both(*second, seed=2)       # reuses the array the first call left behind
    assert small < big


def test_noalloc_rejects_over_limit():
    B, H, Nq, Nk, d = 1, 255, 256, 512, 128
    assert attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d) > attn._lib.ATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((B, H, Nq, d), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, d), dtype=torch.bfloat16, device="cuda")
    o = torch.full_like(q, 3.0)
    lse = torch.zeros((B, H, Nq), device="cuda")
    st = attn.attn_fwd_kv_noalloc(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(), B, H, Nq,
                                  Nk, d, 0.1, 1, 0, Nk - Nq, attn.ATTN_DTYPE_BF16, 0)
    assert st == attn._lib.ATTN_ERR_SCRATCH_LIMIT
    torch.cuda.synchronize()
    assert torch.all(o == 3.0)
