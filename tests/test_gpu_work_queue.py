"""GPU parity of the bf16 forward's work queue (attn_set_work_queue), which serves
the 64-rows-per-wave kernels of the unmasked and causal forward (every case here
forces that tile shape and one key group): with the queue the first three quarters of every XCD's item list stay with the workgroup of the
same index and the rest, plus a few extra workgroups per XCD, claim their items
through per-XCD counters in a slot of a device array.  Which workgroup computes an
item never changes the item, so every case is checked twice: against the oracle
(outputs start as NaN, so an item nobody computed fails), and bit for bit against
the same call without the queue.  The slots rotate over 64 per device and each
launch leaves its slot at zero; the repeated cases run past one full rotation."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_qkv
from tests.gpu_util import compare, forced_key_groups, forced_rows_per_wave, oracle, require_gpu, say, to_np

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()
    yield
    assert attn.attn_set_work_queue(-1) == 0


def _fwd_nan(q, k, v, mask, window, scale):
    out = torch.full_like(q, float("nan"))
    lse = torch.full(q.shape[:3], float("nan"), dtype=torch.float32, device=q.device)
    attn.fwd(q, k, v, mask=mask, window=window, scale=scale, out=out, lse=lse)
    torch.cuda.synchronize()
    return out, lse


def _queue_vs_plain(B, H, N, d, mask, window, seed, check_oracle=True, repeats=1):
    label = f"work-queue B{B} H{H} N{N} d{d} {mask} w{window} seed{seed}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=seed)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    scale = float(np.float32(d ** -0.5))
    with forced_rows_per_wave("64"), forced_key_groups("1"):
        assert attn.attn_set_work_queue(0) == 0
        o0, l0 = _fwd_nan(qd, kd, vd, mask, window, scale)
        assert attn.attn_set_work_queue(1) == 0
        try:
            for r in range(repeats):
                o1, l1 = _fwd_nan(qd, kd, vd, mask, window, scale)
                assert torch.equal(o1.view(torch.int16), o0.view(torch.int16)), f"{label}: O differs (launch {r})"
                assert torch.equal(l1.view(torch.int32), l0.view(torch.int32)), f"{label}: LSE differs (launch {r})"
        finally:
            assert attn.attn_set_work_queue(-1) == 0
    if check_oracle:
        O_ref, L_ref, rows = oracle(to_np(q), to_np(k), to_np(v), scale, attn._lib.MASKS[mask], window)
        compare(o1, l1, O_ref, L_ref, rows, "bf16", label)


# item counts from 1 (every list but one empty, all workgroups claim) to a few per
# XCD with fixed items (7 heads x 9 blocks = 63 items: lists of 7 and 8); the window
# mask never uses the queue (its result must still match)
@pytest.mark.parametrize("B,H,N", [(1, 1, 100), (1, 3, 600), (1, 7, 2200), (2, 5, 1400), (1, 9, 4096)])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_queue_matches_oracle_and_plain(B, H, N, mask):
    _queue_vs_plain(B, H, N, 128, mask, 60, seed=B * 31 + H + N)


@pytest.mark.parametrize("mask", ["none", "causal"])
def test_queue_d64(mask):
    _queue_vs_plain(2, 6, 1800, 64, mask, 0, seed=3)


def test_queue_slot_rotation():
    # 70 launches in a row: past the 64 slots of the pool, each reused after its
    # launch reset it; every launch must match the plain call bit for bit
    _queue_vs_plain(2, 8, 2048, 128, "causal", 0, seed=11, check_oracle=False, repeats=70)


def test_queue_default_at_the_library_threshold():
    # 8192 workgroups of 256 rows: the library's own choice turns the queue on
    B, H, N, d = 4, 64, 8192, 128
    say(f"[gpu] work-queue default B{B} H{H} N{N} d{d} causal")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=21, device="cuda")
    scale = float(np.float32(d ** -0.5))
    with forced_rows_per_wave("64"):
        assert attn.attn_set_work_queue(0) == 0
        o0, l0 = _fwd_nan(q, k, v, "causal", 0, scale)
        assert attn.attn_set_work_queue(-1) == 0
        o1, l1 = _fwd_nan(q, k, v, "causal", 0, scale)
    assert torch.equal(o1.view(torch.int16), o0.view(torch.int16))
    assert torch.equal(l1.view(torch.int32), l0.view(torch.int32))
    assert not torch.isnan(o1).any() and not torch.isnan(l1).any()


def test_captured_launch_runs_without_the_queue():
    # a launch captured into a graph must not keep a queue slot for its replays: with
    # the queue forced on, the captured forward is replayed several times (eager work
    # and synchronisations between replays) and every replay matches the eager call
    B, H, N, d = 2, 8, 2048, 128
    say(f"[gpu] work-queue graph capture B{B} H{H} N{N} d{d} causal")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=31, device="cuda")
    scale = float(np.float32(d ** -0.5))
    assert attn.attn_set_work_queue(1) == 0
    assert attn.attn_set_schedule(64, -1) == 0
    try:
        o_ref, l_ref = _fwd_nan(q, k, v, "causal", 0, scale)
        out = torch.full_like(q, float("nan"))
        lse = torch.full((B, H, N), float("nan"), dtype=torch.float32, device="cuda")
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            attn.fwd(q, k, v, mask="causal", scale=scale, out=out, lse=lse)   # warm-up outside capture
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            attn.fwd(q, k, v, mask="causal", scale=scale, out=out, lse=lse)
        for r in range(4):
            out.fill_(float("nan"))
            lse.fill_(float("nan"))
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), o_ref.view(torch.int16)), f"replay {r}: O differs"
            assert torch.equal(lse.view(torch.int32), l_ref.view(torch.int32)), f"replay {r}: LSE differs"
            _fwd_nan(q, k, v, "causal", 0, scale)       # eager queued work between replays
    finally:
        assert attn.attn_set_work_queue(-1) == 0
        assert attn.attn_set_schedule(0, -1) == 0
