"""GPU parity of the key groups of the bf16 forward (no mask and causal): the waves
of a workgroup split its key tiles into 2 or 4 groups, each with its own running
maximum and sums, merged at the end.  Every tile shape (32 or 64 query rows per
wave) with every group count, forced in turn, against one oracle result per case:
ragged lengths whose tile count is not a multiple of the group count, fewer tiles
than groups, rows whose allowed keys all fall in one group (the first causal
rows), peaked scores (a group's maximum far below another's), and the library's
own choice at the full B1 H8 N4096 d64 shape."""
import numpy as np
import pytest
import torch

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_qkv, row_seed, sample_rows
from tests.gpu_util import (compare, forced_key_groups, forced_rows_per_wave, oracle, require_gpu, say,
                            to_np)

pytestmark = pytest.mark.gpu

SHAPES = [(rows, kg) for rows in ("32", "64") for kg in ("2", "4")]


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def run_groups(B, H, N, d, mask, seed, q_mult=1.0, n_rows=None, name="kgroups", shapes=SHAPES):
    scale = float(np.float32(d ** -0.5))
    label = f"{name} B{B} H{H} N{N} d{d} {mask} seed{seed} qx{q_mult}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(B, H, N, d, torch.bfloat16, seed=seed, q_mult=q_mult)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    outs = []
    for rows, kg in shapes:
        with forced_rows_per_wave(rows), forced_key_groups(kg):
            out, lse = attn.fwd(qd, kd, vd, mask=mask, scale=scale)
            torch.cuda.synchronize()
        outs.append((rows, kg, out, lse))
    if n_rows is None or n_rows >= N:
        rows_sel = None
    else:
        rows_sel = np.stack([np.stack([sample_rows(N, n_rows, row_seed(name, seed, b, h), 0) for h in range(H)])
                             for b in range(B)])
    O_ref, L_ref, rows_sel = oracle(to_np(q), to_np(k), to_np(v), scale, attn._lib.MASKS[mask], 0, rows_sel)
    for rows, kg, out, lse in outs:
        compare(out, lse, O_ref, L_ref, rows_sel, "bf16", f"{label} rows/wave={rows} key groups={kg}")


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("mask", ["none", "causal"])
@pytest.mark.parametrize("N", [1, 33, 100, 777, 1025])
def test_key_groups_ragged(d, mask, N):
    # 1, 2, 4, 25 and 33 key tiles: fewer tiles than groups, and a last step whose
    # groups past the range load the range's last tile and mask it out whole
    run_groups(2, 3, N, d, mask, seed=N + d)


@pytest.mark.parametrize("q_mult", [8.0, 32.0])
@pytest.mark.parametrize("mask", ["none", "causal"])
def test_key_groups_peaked(q_mult, mask):
    # large scores: each group raises its own reference; the merge weights 2^(m_g - M)
    # then span many orders of magnitude
    run_groups(1, 2, 700, 128, mask, seed=3, q_mult=q_mult, name="kgroups-peaked")


def test_key_groups_library_choice_full_shape():
    # B1 H8 N4096 d64 without a mask: 256 workgroups of 128 rows, so the library
    # splits the keys (32 rows per wave, 2 groups); sampled rows against the oracle
    run_groups(1, 8, 4096, 64, "none", seed=0, n_rows=256, name="kgroups-c2", shapes=[(None, None)])


def test_key_groups_deterministic():
    # the same call twice gives the same bits (no order-dependent reduction in the merge)
    q, k, v = (t.cuda() for t in make_qkv(1, 4, 3000, 64, torch.bfloat16, seed=9))
    for rows, kg in SHAPES:
        with forced_rows_per_wave(rows), forced_key_groups(kg):
            o1, l1 = attn.fwd(q, k, v, mask="causal")
            o2, l2 = attn.fwd(q, k, v, mask="causal")
            torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2), (rows, kg)


def test_band_masks_ignore_forced_key_groups():
    # the window masks always run one key group: forcing groups changes nothing
    q, k, v = (t.cuda() for t in make_qkv(1, 2, 900, 64, torch.bfloat16, seed=4))
    with forced_rows_per_wave("32"):
        base = attn.fwd(q, k, v, mask="window", window=100)
        with forced_key_groups("4"):
            forced = attn.fwd(q, k, v, mask="window", window=100)
        torch.cuda.synchronize()
    assert torch.equal(base[0], forced[0]) and torch.equal(base[1], forced[1])
