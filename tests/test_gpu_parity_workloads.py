"""GPU parity at the five workload shapes, in the launch configuration the
benchmark times: all rows for the two small ones, 4096 seeded rows per (b, h) for
the large ones (tile and mask boundary rows always included)."""
import pytest

from exact_blockwise_attention_attn_amd.inputs import WORKLOADS
from tests.gpu_util import require_gpu, run_case

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    require_gpu()


def _run(name, seed=0, q_mult=1.0, n_rows=None, gen_device="cpu"):
    w = WORKLOADS[name]
    return run_case(w.B, w.H, w.N, w.d, w.dtype, w.mask, window=w.window, scale=w.softmax_scale, seed=seed,
                    q_mult=q_mult, n_rows=n_rows, name=name, gen_device=gen_device,
                    rows_per_wave="auto")   # the library's own tile choice, as bench.py runs it


def test_tiny_f32_all_rows():
    _run("tiny_f32_n256")


def test_multihead_bf16_n4096_all_rows():
    _run("mh_bf16_n4096_d64")


@pytest.mark.parametrize("seed,q_mult", [(0, 1.0), (1, 8.0)])
def test_causal_b2h32_n8192(seed, q_mult):
    _run("causal_bf16_b2h32_n8192_d128", seed=seed, q_mult=q_mult, n_rows=4096)


def test_window512_n32768():
    _run("window512_bf16_h32_n32768_d128", n_rows=4096, gen_device="cuda")


def test_causal_n131072():
    _run("causal_bf16_h32_n131072_d128", n_rows=4096, gen_device="cuda")
