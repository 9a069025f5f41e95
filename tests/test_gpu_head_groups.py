"""GPU parity of the grouped workgroup order (heads in groups, every query or key
block of a group before the next): shapes whose (batch, head) count is not a
multiple of the group size run a partial last group.  Small sizes force small
groups through attn_set_schedule (the order never changes a result; the oracle is the
same); one long case reaches a partial group with the library's own choice
(K and V of 16 MB per head: groups of 8, 11 heads = 8 + 3)."""
import numpy as np
import pytest
import torch

from tests.gpu_util import forced_head_group, require_gpu, run_case
from tests.test_gpu_bwd import run_bwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


# (B, H): 11 heads = 8 + 3; 15 = 8 + 7; 16 = two full groups; 5 < one group
@pytest.mark.parametrize("B,H", [(1, 11), (3, 5), (2, 8), (1, 5)])
@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_forward_partial_group(B, H, mask):
    with forced_head_group(8):
        run_case(B, H, 300, 128, "bf16", mask, window=40, seed=B * 100 + H, name="hgroup")


@pytest.mark.parametrize("g", [1, 3, 16])
def test_forward_odd_group_sizes(g):
    # group sizes that are not multiples of 8 (heads of a group then spread over XCDs) still cover every block
    with forced_head_group(g):
        run_case(2, 7, 200, 64, "bf16", "causal", seed=g, name=f"hgroup{g}")


@pytest.mark.parametrize("mask", ["none", "causal", "window"])
def test_backward_partial_group(mask):
    with forced_head_group(8):
        run_bwd(1, 11, 300, 128, mask, window=40, seed=7, label="bwd-hgroup")


def test_backward_batches_partial_group():
    with forced_head_group(8):
        run_bwd(3, 5, 257, 64, "causal", seed=8, label="bwd-hgroup-bh")


def test_forward_long_natural_partial_group():
    # 16 MB of K and V per head: the library's own choice is groups of 8
    run_case(1, 11, 32768, 128, "bf16", "causal", seed=5, n_rows=48, name="hgroup-long", gen_device="cuda")


@pytest.mark.parametrize("B,H", [(1, 11), (3, 5)])
@pytest.mark.parametrize("causal", [False, True])
def test_block_sparse_lead_blocks_and_groups(B, H, causal):
    # block layouts: two leading query blocks of every head, then groups of 8 heads (partial last group)
    from exact_blockwise_attention_attn_amd.inputs import random_block_layout
    from tests.test_gpu_block_sparse import run_bs
    lay = random_block_layout(H, 8, 0.4, seed=B + H, empty_rows=(3,))
    with forced_head_group(8):
        run_bs(B, H, 1000, 128, lay, causal, seed=B * 10 + H, name="bs-hgroup")
