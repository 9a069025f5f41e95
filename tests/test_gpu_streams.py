"""Calls on a stream other than torch's current one: the binding allocates its
outputs and temporaries (the split-KV workspace, the uint8 copy of a bool layout,
the gradients) on the launch stream, so memory freed when a call returns is never
handed to other work while the kernels that use it are still queued.  The launch
stream is first given a long matrix product so that the attention kernels run
well after the call returned and the current stream has allocated and written
fresh tensors; results are then checked against the float64 oracles."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import bigbird_block_layout, make_q_kv, make_qkv
from oracle.attention_block_ref import attention_forward_block_sparse
from oracle.attention_kv_ref import attention_forward_kv
from tests.gpu_util import TOL, require_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _delay(s):
    """Queue ~tens of ms of matrix products on stream s."""
    with torch.cuda.stream(s):
        a = torch.randn(4096, 4096, device="cuda")
        for _ in range(20):
            a = torch.mm(a, a) * 1e-3


def _churn():
    """Allocate and overwrite memory on the current stream (would reuse any block
    the binding freed to the current stream's pool)."""
    junk = [torch.full((1 << 22,), float(i), device="cuda") for i in range(16)]
    for t in junk:
        t.mul_(3.0)
    return junk


def _check(out, lse, O, L, label):
    d_o = float(np.abs(to_np(out) - O).max())
    d_l = float(np.abs(to_np(lse) - L).max())
    say(f"  {label}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e}")
    assert d_o <= TOL["bf16"]["o"] and d_l <= TOL["bf16"]["lse"], label


@pytest.mark.parametrize("handle", ["stream", "raw"])
def test_fwd_kv_on_side_stream(handle):
    say(f"[gpu] streams fwd_kv handle={handle}")
    q, k, v = make_q_kv(1, 4, 1, 20000, 128, torch.bfloat16, seed=3)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    assert attn.attn_fwd_kv_workspace_size(1, 4, 1, 20000, 128) > 0
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    _delay(s)
    out, lse = attn.fwd_kv(qd, kd, vd, mask="causal", stream=s if handle == "stream" else s.cuda_stream)
    junk = _churn()
    s.synchronize()
    torch.cuda.synchronize()
    O, L = attention_forward_kv(to_np(q), to_np(k), to_np(v), 128 ** -0.5, 1, 0, 19999)
    _check(out, lse, O, L, f"fwd_kv side stream ({handle})")
    del junk


def test_fwd_and_bwd_on_side_stream():
    say("[gpu] streams fwd + bwd")
    from oracle.attention_bwd_ref import attention_backward
    from oracle.attention_ref import attention_forward
    q, k, v = make_qkv(1, 2, 300, 128, torch.bfloat16, seed=4)
    qd, kd, vd = q.cuda(), k.cuda(), v.cuda()
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    _delay(s)
    out, lse = attn.fwd(qd, kd, vd, mask="causal", stream=s)
    do = torch.randn((1, 2, 300, 128), generator=torch.Generator().manual_seed(6)).to(torch.bfloat16)
    dod = do.cuda()
    torch.cuda.synchronize()
    _delay(s)
    dq, dk, dv = attn.bwd(qd, kd, vd, out, dod, lse, mask="causal", stream=s)
    junk = _churn()
    s.synchronize()
    torch.cuda.synchronize()
    O, L = attention_forward(to_np(q), to_np(k), to_np(v), 128 ** -0.5, 1, 0)
    _check(out, lse, O, L, "fwd side stream")
    refs = attention_backward(to_np(q), to_np(k), to_np(v), to_np(do), 128 ** -0.5, 1, 0)
    for name, g, r in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        err = float(np.abs(to_np(g) - r).max())
        say(f"  bwd side stream {name}: max|err|={err:.3e}")
        assert err <= 2e-2 * max(1.0, float(np.abs(r).max())), name
    del junk


def test_block_sparse_bool_layout_on_side_stream():
    say("[gpu] streams block-sparse (bool layout)")
    B, H, N, d = 1, 2, 1000, 128
    nb = -(-N // 128)
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=5)
    lay = bigbird_block_layout(H, nb, seed=1)
    s = torch.cuda.Stream()
    torch.cuda.synchronize()
    _delay(s)
    layout = torch.from_numpy(np.asarray(lay) != 0).cuda()
    out, lse = attn.fwd_block_sparse(q.cuda(), k.cuda(), v.cuda(), layout, stream=s)
    junk = _churn()
    s.synchronize()
    torch.cuda.synchronize()
    O, L = attention_forward_block_sparse(to_np(q), to_np(k), to_np(v), d ** -0.5, np.asarray(lay), 128, False)
    _check(out, lse, O, L, "block-sparse side stream")
    del junk
