"""Host-only checks of the C ABI: the library loads, exports every function that
include/attn.h declares, and rejects bad arguments before touching a device.
No compute call is made (there is no GPU here)."""
import ctypes
import os
import re

import pytest

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "attn.h")


def declared_functions():
    text = open(HEADER, encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(attn_[a-z_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    assert declared_functions() == ["attn_bwd", "attn_bwd_check_args", "attn_check_args", "attn_fwd",
                                    "attn_fwd_block_sparse", "attn_fwd_block_sparse_check_args", "attn_fwd_kv",
                                    "attn_fwd_kv_check_args", "attn_fwd_kv_noalloc", "attn_fwd_kv_workspace_size",
                                    "attn_set_key_groups", "attn_set_schedule", "attn_set_work_queue", "attn_strerror", "attn_version"]


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(_lib.LIB_PATH)
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_header_enums_match_binding():
    text = open(HEADER, encoding="utf-8").read()
    for name, value in re.findall(r"\b(ATTN_[A-Z0-9_]+)\s*=\s*(-?\d+)", text):
        assert getattr(_lib, name) == int(value), name


def test_version_and_strerror():
    assert "gfx950" in attn.attn_version()
    for code in range(-11, 1):
        msg = attn.attn_strerror(code)
        assert msg and msg != "unknown status"
    assert attn.attn_strerror(-100) == "unknown status"


# A fake but aligned, non-overlapping address layout: nothing is ever dereferenced.
BASE = 1 << 40
GAP = 1 << 36


def ptrs():
    return [BASE + i * GAP for i in range(5)]


def check(**kw):
    q, k, v, o, l = ptrs()
    args = dict(q=q, k=k, v=v, out=o, lse=l, B=2, H=4, N=100, d=128, scale=0.1, mask_kind=0, window=0, dtype=1)
    args.update(kw)
    return attn.attn_check_args(args["q"], args["k"], args["v"], args["out"], args["lse"], args["B"], args["H"],
                                args["N"], args["d"], args["scale"], args["mask_kind"], args["window"], args["dtype"])


def test_valid_arguments_pass():
    assert check() == 0
    assert check(dtype=0, d=64, mask_kind=2, window=0) == 0
    assert check(mask_kind=1, scale=-0.5) == 0
    assert check(scale=0.0) == 0


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), _lib.ATTN_ERR_NULL_PTR), (dict(k=0), _lib.ATTN_ERR_NULL_PTR), (dict(v=0), _lib.ATTN_ERR_NULL_PTR),
    (dict(out=0), _lib.ATTN_ERR_NULL_PTR), (dict(lse=0), _lib.ATTN_ERR_NULL_PTR),
    (dict(B=0), _lib.ATTN_ERR_BAD_SHAPE), (dict(H=-1), _lib.ATTN_ERR_BAD_SHAPE), (dict(N=0), _lib.ATTN_ERR_BAD_SHAPE),
    (dict(N=1 << 24, d=128), _lib.ATTN_ERR_BAD_SHAPE),              # N*d = 2^31
    (dict(B=1 << 16, H=1 << 15, N=1), _lib.ATTN_ERR_BAD_SHAPE),     # B*H*N = 2^31
    (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM), (dict(d=0), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(d=256), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(mask_kind=4), _lib.ATTN_ERR_BAD_MASK), (dict(mask_kind=-1), _lib.ATTN_ERR_BAD_MASK),
    (dict(mask_kind=3, window=-1), _lib.ATTN_ERR_BAD_MASK),
    (dict(mask_kind=2, window=-1), _lib.ATTN_ERR_BAD_MASK),
    (dict(dtype=2), _lib.ATTN_ERR_BAD_DTYPE),
    (dict(scale=float("nan")), _lib.ATTN_ERR_BAD_SCALE), (dict(scale=float("inf")), _lib.ATTN_ERR_BAD_SCALE),
    (dict(q=BASE + 8), _lib.ATTN_ERR_MISALIGNED), (dict(lse=BASE + 4 * GAP + 4), _lib.ATTN_ERR_MISALIGNED),
    (dict(out=BASE), _lib.ATTN_ERR_ALIAS),                            # out == q
    (dict(out=BASE + 2 * GAP + 4096), _lib.ATTN_ERR_ALIAS),           # out inside v
    (dict(lse=BASE + 3 * GAP + 16), _lib.ATTN_ERR_ALIAS),             # lse inside out
])
def test_invalid_arguments(kw, code):
    assert check(**kw) == code


def test_window_ignored_unless_window_mask():
    assert check(mask_kind=0, window=-5) == 0
    assert check(mask_kind=1, window=-5) == 0


def test_fwd_rejects_before_launch():
    # attn_fwd runs the same checks first and returns without any device call
    q, k, v, o, l = ptrs()
    assert attn.attn_fwd(q, k, v, o, l, 1, 1, 8, 96, 0.1, 0, 0, 1, None) == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM
    assert attn.attn_fwd(0, k, v, o, l, 1, 1, 8, 64, 0.1, 0, 0, 1, None) == _lib.ATTN_ERR_NULL_PTR
    assert attn.attn_fwd(q, k, v, q, l, 1, 1, 8, 64, 0.1, 0, 0, 1, None) == _lib.ATTN_ERR_ALIAS


def test_binding_names_match_c_symbols():
    for name in declared_functions():
        assert callable(getattr(attn, name))



# ---- backward: argument checks on fake, aligned, non-overlapping addresses
def bwd_ptrs():
    return [BASE + i * GAP for i in range(9)]


def bcheck(**kw):
    q, k, v, o, do, l, dq, dk, dv = bwd_ptrs()
    a = dict(q=q, k=k, v=v, out=o, dout=do, lse=l, dq=dq, dk=dk, dv=dv, B=2, H=4, N=100, d=128, scale=0.1,
             mask_kind=1, window=0, dtype=1)
    a.update(kw)
    return attn.attn_bwd_check_args(a["q"], a["k"], a["v"], a["out"], a["dout"], a["lse"], a["dq"], a["dk"],
                                    a["dv"], a["B"], a["H"], a["N"], a["d"], a["scale"], a["mask_kind"],
                                    a["window"], a["dtype"])


def test_bwd_valid_arguments_pass():
    assert bcheck() == _lib.ATTN_OK
    assert bcheck(mask_kind=2, window=7, d=64) == _lib.ATTN_OK


@pytest.mark.parametrize("name", ["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"])
def test_bwd_null_pointer(name):
    assert bcheck(**{name: 0}) == _lib.ATTN_ERR_NULL_PTR


def test_bwd_fp32_rejected():
    assert bcheck(dtype=0) == _lib.ATTN_ERR_BAD_DTYPE


@pytest.mark.parametrize("grad", ["dq", "dk", "dv"])
@pytest.mark.parametrize("other", ["q", "k", "v", "out", "dout", "lse"])
def test_bwd_gradient_aliasing_an_input(grad, other):
    p = dict(zip(["q", "k", "v", "out", "dout", "lse", "dq", "dk", "dv"], bwd_ptrs()))
    assert bcheck(**{grad: p[other] + 64}) == _lib.ATTN_ERR_ALIAS


def test_bwd_gradients_aliasing_each_other():
    p = bwd_ptrs()
    assert bcheck(dk=p[6]) == _lib.ATTN_ERR_ALIAS
    assert bcheck(dv=p[7] + 16) == _lib.ATTN_ERR_ALIAS


def test_bwd_misaligned_and_shape():
    assert bcheck(dq=BASE + 6 * GAP + 8) == _lib.ATTN_ERR_MISALIGNED
    assert bcheck(N=0) == _lib.ATTN_ERR_BAD_SHAPE
    assert bcheck(d=96) == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM
    assert bcheck(mask_kind=2, window=-1) == _lib.ATTN_ERR_BAD_MASK


def test_bwd_rejects_before_any_launch():
    # an invalid call returns its status without touching a device (none exists here)
    q, k, v, o, do, l, dq, dk, dv = bwd_ptrs()
    st = attn.attn_bwd(q, k, v, o, do, l, dq, dk, dv, 2, 4, 100, 96, 0.1, 0, 0, 1, None)
    assert st == _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM


# ---- split-KV forward (Nq queries at positions q_offset.., Nk keys): host checks
def kv_ptrs():
    return [BASE + i * GAP for i in range(6)]


def kvcheck(**kw):
    q, k, v, o, l, ws = kv_ptrs()
    a = dict(q=q, k=k, v=v, out=o, lse=l, B=1, H=8, Nq=1, Nk=65536, d=128, scale=0.1, mask_kind=1, window=0,
             q_offset=65535, dtype=1, workspace=ws, workspace_bytes=1 << 30)
    a.update(kw)
    return attn.attn_fwd_kv_check_args(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["Nq"],
                                       a["Nk"], a["d"], a["scale"], a["mask_kind"], a["window"], a["q_offset"],
                                       a["dtype"], a["workspace"], a["workspace_bytes"])


def test_kv_workspace_size_shape():
    """Partial O and LSE in fp32: B H n_split Nq (4 d + 4) bytes, with 2 <= n_split
    <= ceil(Nk / 256) when the query blocks are too few to fill the device."""
    for B, H, Nq, Nk, d in [(1, 8, 1, 65536, 128), (4, 32, 1, 131072, 128), (1, 1, 16, 300, 64),
                            (2, 4, 5, 4096, 64)]:
        ws = attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d)
        per = B * H * Nq * (4 * d + 4)
        assert ws > 0 and ws % per == 0, (B, H, Nq, Nk, d, ws)
        assert 2 <= ws // per <= -(-Nk // 256)
    # one key range is enough once the query blocks fill the device: no workspace
    assert attn.attn_fwd_kv_workspace_size(2, 32, 8192, 8192, 128) == 0
    assert attn.attn_fwd_kv_workspace_size(1, 1, 1, 256, 128) == 0          # 256 keys: one range
    # shapes attn_fwd_kv rejects
    assert attn.attn_fwd_kv_workspace_size(1, 1, 10, 5, 128) == 0
    assert attn.attn_fwd_kv_workspace_size(0, 1, 1, 5, 128) == 0
    assert attn.attn_fwd_kv_workspace_size(1, 1, 1, 4096, 96) == 0


def test_kv_valid_arguments_pass():
    assert kvcheck() == _lib.ATTN_OK
    assert kvcheck(mask_kind=0, q_offset=0) == _lib.ATTN_OK
    assert kvcheck(mask_kind=2, window=100, d=64, Nq=64, q_offset=100) == _lib.ATTN_OK
    need = attn.attn_fwd_kv_workspace_size(1, 8, 1, 65536, 128)
    assert kvcheck(workspace_bytes=need) == _lib.ATTN_OK
    # no workspace needed: NULL is fine
    assert kvcheck(B=2, H=32, Nq=8192, Nk=8192, q_offset=0, workspace=0, workspace_bytes=0) == _lib.ATTN_OK


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), _lib.ATTN_ERR_NULL_PTR), (dict(lse=0), _lib.ATTN_ERR_NULL_PTR),
    (dict(Nq=0), _lib.ATTN_ERR_BAD_SHAPE), (dict(Nk=0), _lib.ATTN_ERR_BAD_SHAPE),
    (dict(q_offset=-1), _lib.ATTN_ERR_BAD_SHAPE), (dict(q_offset=65536), _lib.ATTN_ERR_BAD_SHAPE),
    (dict(Nq=2), _lib.ATTN_ERR_BAD_SHAPE),                                      # q_offset + Nq > Nk
    (dict(Nk=1 << 24, q_offset=0), _lib.ATTN_ERR_BAD_SHAPE),                    # Nk * d = 2^31
    (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(mask_kind=5), _lib.ATTN_ERR_BAD_MASK), (dict(mask_kind=3, window=-2), _lib.ATTN_ERR_BAD_MASK),
    (dict(scale=float("nan")), _lib.ATTN_ERR_BAD_SCALE),
    (dict(dtype=0), _lib.ATTN_ERR_BAD_DTYPE), (dict(dtype=7), _lib.ATTN_ERR_BAD_DTYPE),
    (dict(workspace=0), _lib.ATTN_ERR_WORKSPACE), (dict(workspace_bytes=100), _lib.ATTN_ERR_WORKSPACE),
    (dict(workspace=BASE + 5 * GAP + 4), _lib.ATTN_ERR_MISALIGNED),
    (dict(k=BASE + 8), _lib.ATTN_ERR_MISALIGNED),
    (dict(out=BASE + GAP + 1024), _lib.ATTN_ERR_ALIAS),                         # out inside k
    (dict(workspace=BASE + 2 * GAP + 64), _lib.ATTN_ERR_ALIAS),                 # workspace inside v
    (dict(workspace=BASE + 4 * GAP - 64), _lib.ATTN_ERR_ALIAS),                 # workspace runs into lse
    (dict(lse=BASE + 3 * GAP + 16), _lib.ATTN_ERR_ALIAS),                       # lse inside out
])
def test_kv_invalid_arguments(kw, code):
    assert kvcheck(**kw) == code


def test_kv_rejects_before_any_launch():
    q, k, v, o, l, ws = kv_ptrs()
    st = attn.attn_fwd_kv(q, k, v, o, l, 1, 8, 4, 2, 128, 0.1, 0, 0, 0, 1, ws, 1 << 30, None)
    assert st == _lib.ATTN_ERR_BAD_SHAPE
    st = attn.attn_fwd_kv(q, k, v, o, l, 1, 8, 1, 65536, 128, 0.1, 0, 0, 0, 1, 0, 0, None)
    assert st == _lib.ATTN_ERR_WORKSPACE


# ---- block-sparse forward: host checks
def bscheck(**kw):
    q, k, v, o, l, lay = [BASE + i * GAP for i in range(6)]
    a = dict(q=q, k=k, v=v, out=o, lse=l, B=2, H=4, N=1000, d=128, scale=0.1, causal=0, layout=lay, dtype=1)
    a.update(kw)
    return attn.attn_fwd_block_sparse_check_args(a["q"], a["k"], a["v"], a["out"], a["lse"], a["B"], a["H"], a["N"],
                                                 a["d"], a["scale"], a["causal"], a["layout"], a["dtype"])


def test_block_sparse_valid_arguments_pass():
    assert bscheck() == _lib.ATTN_OK
    assert bscheck(causal=1, d=64, scale=-0.5) == _lib.ATTN_OK
    assert bscheck(N=128 * 8192, B=1, H=1, d=64) == _lib.ATTN_OK          # the largest layout
    assert bscheck(layout=BASE + 5 * GAP + 1) == _lib.ATTN_OK               # bytes: no alignment needed


@pytest.mark.parametrize("kw,code", [
    (dict(layout=0), _lib.ATTN_ERR_NULL_PTR), (dict(q=0), _lib.ATTN_ERR_NULL_PTR),
    (dict(causal=2), _lib.ATTN_ERR_BAD_MASK), (dict(causal=-1), _lib.ATTN_ERR_BAD_MASK),
    (dict(dtype=0), _lib.ATTN_ERR_BAD_DTYPE),
    (dict(N=128 * 8192 + 1, B=1, H=1, d=64), _lib.ATTN_ERR_BAD_SHAPE),     # more than 8192 layout blocks
    (dict(N=0), _lib.ATTN_ERR_BAD_SHAPE), (dict(d=96), _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM),
    (dict(layout=BASE + 3 * GAP + 100), _lib.ATTN_ERR_ALIAS),             # layout inside out
    (dict(layout=BASE + 4 * GAP + 8), _lib.ATTN_ERR_ALIAS),               # layout inside lse
    (dict(out=BASE), _lib.ATTN_ERR_ALIAS),
])
def test_block_sparse_invalid_arguments(kw, code):
    assert bscheck(**kw) == code


def test_block_sparse_rejects_before_any_launch():
    q, k, v, o, l, lay = [BASE + i * GAP for i in range(6)]
    assert attn.attn_fwd_block_sparse(q, k, v, o, l, 1, 1, 100, 96, 0.1, 0, lay, 1, None) == \
        _lib.ATTN_ERR_UNSUPPORTED_HEAD_DIM
    assert attn.attn_fwd_block_sparse(q, k, v, o, l, 1, 1, 100, 64, 0.1, 0, 0, 1, None) == _lib.ATTN_ERR_NULL_PTR


def test_set_schedule_validates():
    assert attn.attn_set_schedule(0, -1) == 0
    for rpw, hg in ((32, 8), (64, 0), (0, 16)):
        assert attn.attn_set_schedule(rpw, hg) == 0
    for rpw, hg in ((16, -1), (128, -1), (-32, -1), (0, -2)):
        assert attn.attn_set_schedule(rpw, hg) == _lib.ATTN_ERR_BAD_SHAPE
    assert attn.attn_set_schedule(0, -1) == 0


def test_set_key_groups_validates():
    for kg in (1, 2, 4, -1):
        assert attn.attn_set_key_groups(kg) == 0
    for kg in (0, 3, 8, -2):
        assert attn.attn_set_key_groups(kg) == _lib.ATTN_ERR_BAD_SHAPE
    assert attn.attn_set_key_groups(-1) == 0


def test_set_work_queue_validates():
    for mode in (1, 0, -1):
        assert attn.attn_set_work_queue(mode) == 0
    for mode in (2, -2, 8):
        assert attn.attn_set_work_queue(mode) == _lib.ATTN_ERR_BAD_SHAPE
    assert attn.attn_set_work_queue(-1) == 0


def test_noalloc_rejects_over_limit_on_the_host():
    # a shape whose split-KV partials exceed the static scratch: rejected before any device call
    B, H, Nq, Nk, d = 1, 255, 256, 512, 128
    assert attn.attn_fwd_kv_workspace_size(B, H, Nq, Nk, d) > _lib.ATTN_NOALLOC_SCRATCH_BYTES
    q, k, v, o, l = ptrs()
    assert attn.attn_fwd_kv_noalloc(q, k, v, o, l, B, H, Nq, Nk, d, 0.1, 1, 0, Nk - Nq, 1, None) == \
        _lib.ATTN_ERR_SCRATCH_LIMIT
