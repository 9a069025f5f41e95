"""GPU parity of the backward (attn_bwd) against the CPU float64 backward oracle:
every mask, both head dims, ragged lengths around the tile sizes, window widths at
tile edges, negative and large scales, peaked rows.  The GPU backward consumes the
GPU forward's own O and LSE (as a training step would); the oracle differentiates
the exact forward.  Tolerances (derived in the design notes): per tensor,
max|error| <= 2e-2 * max(1, max|reference|) and relative RMS <= 1e-2."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_qkv
from oracle.attention_bwd_ref import attention_backward
from tests.gpu_util import require_gpu, say, to_np

pytestmark = pytest.mark.gpu

TOL_MAX = 2e-2
TOL_RMS = 1e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_bwd(B, H, N, d, mask, window=0, scale=None, seed=0, q_mult=1.0, label="bwd"):
    scale = float(np.float32(scale if scale is not None else d ** -0.5))
    say(f"[gpu] {label} B{B} H{H} N{N} d{d} {mask} w{window} scale{scale:g} seed{seed} qx{q_mult}")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=seed, q_mult=q_mult)
    g = torch.Generator().manual_seed(seed + 1000)
    do = torch.randn((B, H, N, d), generator=g).to(torch.bfloat16)
    qd, kd, vd, dod = (t.cuda() for t in (q, k, v, do))
    out, lse = attn.fwd(qd, kd, vd, mask=mask, window=window, scale=scale)
    dq, dk, dv = attn.bwd(qd, kd, vd, out, dod, lse, mask=mask, window=window, scale=scale)
    torch.cuda.synchronize()
    mk = attn._lib.MASKS[mask]
    refs = attention_backward(to_np(q), to_np(k), to_np(v), to_np(do), scale, mk, window)
    stats = []
    for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
        gn = to_np(got)
        assert np.all(np.isfinite(gn)), f"{label}: non-finite {name}"
        err = np.abs(gn - ref)
        mref = float(np.max(np.abs(ref))) if ref.size else 0.0
        rms = float(np.sqrt(np.sum((gn - ref) ** 2)) / max(np.sqrt(np.sum(ref ** 2)), 1e-30))
        stats.append((name, float(err.max()), mref, rms))
        say(f"  {name}: max|err|={err.max():.3e} max|ref|={mref:.3e} relRMS={rms:.3e}")
    for name, e, mref, rms in stats:
        assert e <= TOL_MAX * max(1.0, mref), f"{label}: {name} max|err| {e} (max|ref| {mref})"
        if mref > 1e-3:
            assert rms <= TOL_RMS, f"{label}: {name} relative RMS {rms}"
    return stats


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("N", [1, 17, 63, 64, 65, 127, 128, 129, 300])
def test_bwd_ragged(d, mask, N):
    run_bwd(1, 2, N, d, mask, seed=N, label="bwd-ragged")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,w", [(300, 0), (300, 1), (300, 31), (300, 32), (300, 63), (300, 200), (300, 5000),
                                 (129, 31), (1000, 100)])
def test_bwd_window(d, N, w):
    run_bwd(1, 2, N, d, "window", window=w, seed=N + w, label="bwd-window")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("N,w", [(300, 0), (300, 1), (300, 31), (300, 63), (300, 200), (300, 5000), (1000, 128)])
def test_bwd_causal_window(d, N, w):
    run_bwd(1, 2, N, d, "causal_window", window=w, seed=N + 3 * w, label="bwd-cwindow")


@pytest.mark.parametrize("scale", [-0.125, 2.0, 1e-3])
def test_bwd_scales(scale):
    run_bwd(1, 2, 200, 128, "causal", scale=scale, seed=5, label="bwd-scale")


def test_bwd_batches_heads():
    run_bwd(2, 3, 257, 128, "causal", seed=9, label="bwd-bh")


@pytest.mark.parametrize("mask", ["none", "causal", "window", "causal_window"])
def test_bwd_peaked(mask):
    run_bwd(1, 2, 700, 128, mask, window=100, seed=3, q_mult=8.0, label="bwd-peaked")


def test_bwd_long_causal():
    run_bwd(1, 2, 2048, 128, "causal", seed=21, label="bwd-long")


def test_bwd_errors_leave_gradients_untouched():
    q, k, v = (t.cuda() for t in make_qkv(1, 1, 64, 128, torch.bfloat16, seed=1))
    out, lse = attn.fwd(q, k, v, mask="causal")
    dq = torch.full_like(q, 7.0)
    with pytest.raises(attn.AttnError):
        attn.bwd(q, k, v, out, out, lse, mask="causal", dq=dq, dk=q)      # dk aliases q
    torch.cuda.synchronize()
    assert torch.all(dq == 7.0)


def test_bwd_benchmark_shape():
    """The backward at the shape bench.py times (B2 H32 N8192 d128 causal) with the
    library's own schedule (head groups of 32: two full groups), every gradient of
    three whole heads against the float64 backward oracle: the first head, the
    first head of the second group and the last head."""
    B, H, N, d = 2, 32, 8192, 128
    scale = float(np.float32(d ** -0.5))
    say(f"[gpu] bwd-bench B{B} H{H} N{N} d{d} causal (library schedule)")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=0, device="cuda")
    g = torch.Generator(device="cuda").manual_seed(1000)
    do = torch.randn((B, H, N, d), generator=g, device="cuda").to(torch.bfloat16)
    out, lse = attn.fwd(q, k, v, mask="causal", scale=scale)
    dq, dk, dv = attn.bwd(q, k, v, out, do, lse, mask="causal", scale=scale)
    torch.cuda.synchronize()
    for b, h in ((0, 0), (1, 0), (1, 31)):
        sl = (slice(b, b + 1), slice(h, h + 1))
        refs = attention_backward(to_np(q[sl]), to_np(k[sl]), to_np(v[sl]), to_np(do[sl]), scale, 1, 0)
        for name, got, ref in zip(("dq", "dk", "dv"), (dq, dk, dv), refs):
            gn = to_np(got[sl])
            assert np.all(np.isfinite(gn)), f"head ({b},{h}): non-finite {name}"
            err = float(np.abs(gn - ref).max())
            mref = float(np.abs(ref).max())
            rms = float(np.sqrt(np.sum((gn - ref) ** 2)) / max(np.sqrt(np.sum(ref ** 2)), 1e-30))
            say(f"  head ({b},{h}) {name}: max|err|={err:.3e} max|ref|={mref:.3e} relRMS={rms:.3e}")
            assert err <= TOL_MAX * max(1.0, mref), f"head ({b},{h}): {name} max|err| {err}"
            assert rms <= TOL_RMS, f"head ({b},{h}): {name} relative RMS {rms}"
