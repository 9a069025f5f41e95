"""GPU parity of the block-sparse forward (attn_fwd_block_sparse) against the CPU
float64 block-sparse oracle (oracle/attention_block_ref.py), element by element.

Covers random layouts of several densities, with and without the causal flag,
ragged N around the 128-token block and the 32-key tile, both head dims, per-head
layouts over several batch entries, query blocks with no allowed key (O = 0,
LSE = -inf), the all-empty and all-ones layouts, negative and zero scales, peaked
scores, and a BigBird-style layout at N = 32768 on sampled rows."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import bigbird_block_layout, make_qkv, random_block_layout, sample_rows
from oracle.attention_block_ref import attention_forward_block_sparse
from tests.gpu_util import REL_RMS_BF16, TOL, require_gpu, say, to_np

pytestmark = pytest.mark.gpu
BLOCK = 128


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_bs(B, H, N, d, layout, causal, scale=None, seed=0, q_mult=1.0, rows=None, gen_device="cpu", name="bs"):
    scale = float(np.float32(scale if scale is not None else d ** -0.5))
    label = f"{name} B{B} H{H} N{N} d{d} causal{int(causal)} density{layout.mean():.2f} seed{seed}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=seed, q_mult=q_mult, device=gen_device)
    out, lse = attn.fwd_block_sparse(q.cuda(), k.cuda(), v.cuda(), torch.from_numpy(layout).cuda(), causal=causal,
                                     scale=scale)
    torch.cuda.synchronize()
    O_ref, L_ref = attention_forward_block_sparse(to_np(q), to_np(k), to_np(v), scale, layout, BLOCK, causal, rows=rows)
    on, ln = to_np(out), to_np(lse)
    if rows is not None:
        on, ln = on[:, :, rows], ln[:, :, rows]
    empty = np.isneginf(L_ref)
    assert np.array_equal(np.isneginf(ln), empty), f"{label}: rows without allowed keys differ"
    assert np.all(on[empty] == 0.0), f"{label}: O of an empty row is not 0"
    full = ~empty
    assert np.all(np.isfinite(on)) and np.all(np.isfinite(ln[full])), f"{label}: non-finite output"
    if not full.any():
        say(f"  {label}: every row empty")
        return
    d_o = float(np.abs(on - O_ref)[full].max())
    d_l = float(np.abs(ln[full] - L_ref[full]).max())
    num = np.sqrt(((on - O_ref) ** 2).sum(axis=(2, 3)))
    den = np.sqrt((O_ref ** 2).sum(axis=(2, 3)))
    rel = float(np.max(num / np.maximum(den, 1e-300)))
    say(f"  {label}: max|dO|={d_o:.3e} max|dLSE|={d_l:.3e} rel_rms={rel:.3e}")
    assert d_o <= TOL["bf16"]["o"], f"{label}: max|dO| {d_o}"
    assert d_l <= TOL["bf16"]["lse"], f"{label}: max|dLSE| {d_l}"
    assert rel <= REL_RMS_BF16, f"{label}: rel RMS {rel}"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("N", [1, 100, 128, 129, 300, 1000])
@pytest.mark.parametrize("density", [0.3, 1.0])
def test_random_layouts(d, causal, N, density):
    nb = -(-N // BLOCK)
    run_bs(1, 2, N, d, random_block_layout(2, nb, density, seed=N + int(10 * density)), causal, seed=N, name="random")


@pytest.mark.parametrize("causal", [False, True])
def test_empty_query_blocks(causal):
    N = 700
    lay = random_block_layout(3, 6, 0.5, seed=4, empty_rows=(0, 3))
    run_bs(1, 3, N, 128, lay, causal, seed=5, name="empty_rows")


def test_all_empty_layout():
    run_bs(1, 2, 300, 64, np.zeros((2, 3, 3), dtype=np.uint8), False, seed=6, name="all_empty")


@pytest.mark.parametrize("d", [64, 128])
def test_per_head_layouts_and_batches(d):
    run_bs(2, 4, 520, d, random_block_layout(4, 5, 0.4, seed=7), True, seed=8, name="heads")


@pytest.mark.parametrize("scale", [-0.125, 0.0])
def test_scales(scale):
    run_bs(1, 2, 400, 128, random_block_layout(2, 4, 0.6, seed=9), True, scale=scale, seed=10, name="scale")


@pytest.mark.parametrize("causal", [False, True])
def test_peaked(causal):
    run_bs(1, 2, 600, 128, random_block_layout(2, 5, 0.5, seed=11), causal, q_mult=8.0, seed=12, name="peaked")


def test_block_diagonal_and_full():
    N = 512
    run_bs(1, 2, N, 128, np.broadcast_to(np.eye(4, dtype=np.uint8), (2, 4, 4)).copy(), False, seed=13, name="diag")
    run_bs(1, 2, N, 128, np.ones((2, 4, 4), dtype=np.uint8), True, seed=14, name="full_causal")


@pytest.mark.parametrize("causal", [False, True])
def test_bigbird_long(causal):
    """BigBird-style layout at N = 32768 (256 blocks), LLaMA-7B heads, sampled rows."""
    B, H, N, d = 1, 8, 32768, 128
    lay = bigbird_block_layout(H, N // BLOCK, seed=15)
    rows = sample_rows(N, 512, seed=16)
    run_bs(B, H, N, d, lay, causal, seed=17, rows=rows, gen_device="cuda", name="bigbird")
