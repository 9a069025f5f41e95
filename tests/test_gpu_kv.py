"""GPU parity of the split-KV forward (attn_fwd_kv): Nq queries at positions
q_offset .. q_offset + Nq - 1 against Nk cached keys, checked element by element
against the float64 oracle of oracle/attention_kv_ref.py.

Covers decode (Nq = 1) over key counts around the tile (32), the range length
(multiples of 32, >= 256) and the split count; chunks of several queries at the
start, middle and end of the cache; every mask with windows at tile edges; the
unsplit path (enough query blocks to fill the device); a negative scale; peaked
scores; workspace reuse by a second, smaller call; and the long-context decode
shapes at full size."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_q_kv
from oracle.attention_kv_ref import attention_forward_kv
from tests.gpu_util import REL_RMS_BF16, TOL, require_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def check(out, lse, O_ref, L_ref, label, rows=None):
    on, ln = to_np(out), to_np(lse)
    if rows is not None:
        on, ln = on[:, :, rows], ln[:, :, rows]
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln)), f"{label}: non-finite output"
    d_o = float(np.abs(on - O_ref).max())
    d_l = float(np.abs(ln - L_ref).max())
    num = np.sqrt(((on - O_ref) ** 2).sum(axis=(2, 3)))
    den = np.sqrt((O_ref ** 2).sum(axis=(2, 3)))
    rel = float(np.max(num / np.maximum(den, 1e-300)))
    say(f"  {label}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e} rel_rms={rel:.3e}")
    assert d_o <= TOL["bf16"]["o"], f"{label}: max|dO| {d_o}"
    assert d_l <= TOL["bf16"]["lse"], f"{label}: max|dLSE| {d_l}"
    assert rel <= REL_RMS_BF16, f"{label}: rel RMS {rel}"


def run_kv(B, H, Nq, Nk, d, mask, window=0, q_offset=None, scale=None, seed=0, q_mult=1.0, rows=None,
           gen_device="cpu", name="kv"):
    q_offset = Nk - Nq if q_offset is None else q_offset
    scale = float(np.float32(scale if scale is not None else d ** -0.5))
    ws = attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d)
    label = f"{name} B{B} H{H} Nq{Nq} Nk{Nk} d{d} {mask} w{window} off{q_offset} seed{seed} ws{ws}"
    say(f"[gpu] {label}")
    q, k, v = make_q_kv(B, H, Nq, Nk, d, torch.bfloat16, seed=seed, q_mult=q_mult, device=gen_device)
    out, lse = attn.fwd_kv(q.cuda(), k.cuda(), v.cuda(), q_offset=q_offset, mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_forward_kv(to_np(q), to_np(k), to_np(v), scale, attn._lib.MASKS[mask], window,
                                        q_offset, rows=rows)
    check(out, lse, O_ref, L_ref, label, rows)


DECODE_NK = [1, 2, 31, 32, 33, 255, 256, 257, 1000, 4097, 20000]


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("Nk", DECODE_NK)
def test_decode(d, mask, Nk):
    run_kv(1, 4, 1, Nk, d, mask, seed=Nk, name="decode")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["window", "causal_window"])
@pytest.mark.parametrize("Nk,w", [(1000, 0), (1000, 31), (1000, 32), (1000, 300), (5000, 256), (5000, 257),
                                  (5000, 4999), (20000, 1000)])
def test_decode_window(d, mask, Nk, w):
    run_kv(1, 4, 1, Nk, d, mask, window=w, seed=Nk + w, name="decode_w")


@pytest.mark.parametrize("B,H,Nk,d", [(1, 1024, 600, 64), (1, 700, 1500, 128), (2, 3, 100000, 64)])
def test_decode_many_heads_and_ranges(B, H, Nk, d):
    """Decode with more heads than one round of workgroups (one key range: the
    kernel writes O and LSE itself), with two ranges per head, and with many."""
    run_kv(B, H, 1, Nk, d, "causal", seed=H + Nk, name="decode_heads")


@pytest.mark.parametrize("mask,w", [("none", 0), ("causal", 0), ("window", 37), ("window", 300),
                                    ("causal_window", 0), ("causal_window", 100)])
@pytest.mark.parametrize("Nq,off", [(5, 0), (5, 2000), (5, 2995), (64, 1000), (129, 0), (129, 2871), (300, 700)])
def test_chunk(mask, w, Nq, off):
    run_kv(1, 3, Nq, 3000, 128, mask, window=w, q_offset=off, seed=Nq + off, name="chunk")


@pytest.mark.parametrize("d", [64, 128])
def test_chunk_d64_d128_batches(d):
    run_kv(3, 2, 17, 777, d, "causal", q_offset=400, seed=5, name="chunk_bh")


@pytest.mark.parametrize("mask", ["none", "causal", "causal_window"])
def test_unsplit_path(mask):
    # 8 query blocks x 64 heads = 512 workgroups: one key range, no workspace
    B, H, Nq, Nk = 2, 32, 1024, 2048
    assert attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, 128) == 0
    rows = np.array([0, 1, 31, 32, 127, 128, 500, 1022, 1023])
    run_kv(B, H, Nq, Nk, 128, mask, window=200, seed=9, rows=rows, name="unsplit")


def test_square_equals_offset_zero():
    # Nq = Nk with q_offset = 0 is the square problem of attn_fwd
    run_kv(1, 2, 300, 300, 64, "causal", q_offset=0, seed=3, name="square")


@pytest.mark.parametrize("scale", [-0.125, 0.0])
def test_scale_values(scale):
    run_kv(1, 2, 3, 5000, 128, "causal", scale=scale, seed=13, name="kv_scale")


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_peaked(mask):
    run_kv(1, 2, 1, 9000, 128, mask, q_mult=16.0, seed=21, name="kv_peaked")


def test_workspace_reused_by_a_smaller_call():
    """Two calls in a row through one caller workspace, the second smaller; each
    result checked against the oracle."""
    B, H, d = 1, 4, 128
    big = attn.attn_fwd_kv_workspace_size(B, H, 2, 9000, d)
    ws = torch.empty(big, dtype=torch.uint8, device="cuda")
    for Nq, Nk, seed in [(2, 9000, 31), (1, 3000, 32)]:
        assert attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d) <= big
        q, k, v = make_q_kv(B, H, Nq, Nk, d, torch.bfloat16, seed=seed)
        out, lse = attn.fwd_kv(q.cuda(), k.cuda(), v.cuda(), mask="causal", workspace=ws)
        torch.cuda.synchronize()
        O_ref, L_ref = attention_forward_kv(to_np(q), to_np(k), to_np(v), float(np.float32(d ** -0.5)), 1, 0,
                                            Nk - Nq)
        check(out, lse, O_ref, L_ref, f"reuse Nq{Nq} Nk{Nk}")


def test_short_workspace_is_rejected():
    q, k, v = make_q_kv(1, 4, 1, 9000, 128, torch.bfloat16, seed=1, device="cuda")
    need = attn.attn_fwd_kv_workspace_size(1, 4, 1, 9000, 128)
    ws = torch.empty(need - 16, dtype=torch.uint8, device="cuda")
    with pytest.raises(attn.AttnError) as e:
        attn.fwd_kv(q, k, v, workspace=ws)
    assert e.value.status == attn._lib.ATTN_ERR_WORKSPACE


@pytest.mark.parametrize("B,H,Nk", [(1, 32, 131072), (8, 32, 8192)])
def test_decode_full_size(B, H, Nk):
    """The decode workloads at their full size (LLaMA-7B heads, d = 128): every
    head's one query row checked."""
    run_kv(B, H, 1, Nk, 128, "causal", seed=Nk + B, gen_device="cuda", name="decode_full")
