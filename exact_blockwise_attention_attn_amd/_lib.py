"""ctypes binding of libattn.so: the C ABI of include/attn.h, one Python function
per C symbol with the same name and argument order (marshalling only), plus
``fwd``, a convenience call taking torch tensors.

Nothing here computes attention.  If the library is not built, every call raises;
there is no fallback path.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libattn.so")

ATTN_MASK_NONE, ATTN_MASK_CAUSAL, ATTN_MASK_WINDOW, ATTN_MASK_CAUSAL_WINDOW = 0, 1, 2, 3
ATTN_DTYPE_F32, ATTN_DTYPE_BF16 = 0, 1
ATTN_OK = 0
ATTN_ERR_NULL_PTR = -1
ATTN_ERR_BAD_SHAPE = -2
ATTN_ERR_UNSUPPORTED_HEAD_DIM = -3
ATTN_ERR_BAD_MASK = -4
ATTN_ERR_BAD_DTYPE = -5
ATTN_ERR_ALIAS = -6
ATTN_ERR_BAD_SCALE = -7
ATTN_ERR_MISALIGNED = -8
ATTN_ERR_HIP = -9
ATTN_ERR_WORKSPACE = -10
ATTN_ERR_SCRATCH_LIMIT = -11
ATTN_NOALLOC_SCRATCH_BYTES = 64 << 20
ATTN_BLOCK_SPARSE_BLOCK = 128
ATTN_BLOCK_SPARSE_MAX_BLOCKS = 8192

MASKS = {"none": ATTN_MASK_NONE, "causal": ATTN_MASK_CAUSAL, "window": ATTN_MASK_WINDOW,
         "causal_window": ATTN_MASK_CAUSAL_WINDOW}

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"attn error {status}: {msg}")
        self.status = status


def load():
    """Load libattn.so once; raise if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m exact_blockwise_attention_attn_amd._build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    lib.attn_fwd.restype = i
    lib.attn_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i]
    lib.attn_check_args.restype = i
    lib.attn_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
    lib.attn_bwd.restype = i
    lib.attn_bwd_check_args.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i]
    lib.attn_bwd_check_args.restype = i
    u64 = ctypes.c_ulonglong
    lib.attn_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp, u64, vp]
    lib.attn_fwd_kv.restype = i
    lib.attn_fwd_kv_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp, u64]
    lib.attn_fwd_kv_check_args.restype = i
    lib.attn_fwd_kv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
    lib.attn_fwd_kv_noalloc.restype = i
    lib.attn_fwd_kv_workspace_size.argtypes = [i, i, i, i, i]
    lib.attn_fwd_kv_workspace_size.restype = u64
    lib.attn_fwd_block_sparse.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i, vp]
    lib.attn_fwd_block_sparse.restype = i
    lib.attn_fwd_block_sparse_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
    lib.attn_fwd_block_sparse_check_args.restype = i
    lib.attn_set_schedule.argtypes = [i, i]
    lib.attn_set_schedule.restype = i
    lib.attn_set_key_groups.argtypes = [i]
    lib.attn_set_key_groups.restype = i
    lib.attn_set_work_queue.argtypes = [i]
    lib.attn_set_work_queue.restype = i
    lib.attn_strerror.argtypes = [i]
    lib.attn_strerror.restype = ctypes.c_char_p
    lib.attn_version.argtypes = []
    lib.attn_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def attn_fwd(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype, stream):
    """C ``attn_fwd``: pointers as ints, returns the status code."""
    return load().attn_fwd(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype, stream)


def attn_check_args(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype):
    """C ``attn_check_args``: host-only argument check, returns the status code."""
    return load().attn_check_args(q, k, v, out, lse, B, H, N, d, scale, mask_kind, window, dtype)


def attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, scale, mask_kind, window, dtype, stream):
    """C ``attn_bwd``: pointers as ints, returns the status code."""
    return load().attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, scale, mask_kind, window, dtype, stream)


def attn_bwd_check_args(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, scale, mask_kind, window, dtype):
    """C ``attn_bwd_check_args``: host-only argument check, returns the status code."""
    return load().attn_bwd_check_args(q, k, v, out, dout, lse, dq, dk, dv, B, H, N, d, scale, mask_kind, window,
                                      dtype)


def attn_fwd_kv(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype, workspace,
                workspace_bytes, stream):
    """C ``attn_fwd_kv``: pointers as ints, returns the status code."""
    return load().attn_fwd_kv(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype,
                              workspace, workspace_bytes, stream)


def attn_fwd_kv_noalloc(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype, stream):
    """C ``attn_fwd_kv_noalloc``: pointers as ints, returns the status code."""
    return load().attn_fwd_kv_noalloc(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype,
                                      stream)


def attn_fwd_kv_check_args(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset, dtype, workspace,
                           workspace_bytes):
    """C ``attn_fwd_kv_check_args``: host-only argument check, returns the status code."""
    return load().attn_fwd_kv_check_args(q, k, v, out, lse, B, H, Nq, Nk, d, scale, mask_kind, window, q_offset,
                                         dtype, workspace, workspace_bytes)


def attn_fwd_kv_workspace_size(B, H, Nq, Nk, d) -> int:
    """C ``attn_fwd_kv_workspace_size``: workspace bytes ``attn_fwd_kv`` needs."""
    return int(load().attn_fwd_kv_workspace_size(B, H, Nq, Nk, d))


def attn_fwd_block_sparse(q, k, v, out, lse, B, H, N, d, scale, causal, layout, dtype, stream):
    """C ``attn_fwd_block_sparse``: pointers as ints, returns the status code."""
    return load().attn_fwd_block_sparse(q, k, v, out, lse, B, H, N, d, scale, causal, layout, dtype, stream)


def attn_fwd_block_sparse_check_args(q, k, v, out, lse, B, H, N, d, scale, causal, layout, dtype):
    """C ``attn_fwd_block_sparse_check_args``: host-only argument check, returns the status code."""
    return load().attn_fwd_block_sparse_check_args(q, k, v, out, lse, B, H, N, d, scale, causal, layout, dtype)


def attn_set_schedule(rows_per_wave: int, head_group: int) -> int:
    """C ``attn_set_schedule``: force the bf16 tile shape (32 / 64 rows per wave, 0 =
    the library's choice) and head-group size (n, 0 = one group, -1 = the library's
    choice) for later calls; returns the status code."""
    return load().attn_set_schedule(rows_per_wave, head_group)


def attn_set_key_groups(key_groups: int) -> int:
    """C ``attn_set_key_groups``: force 1, 2 or 4 key groups in the bf16 forward
    with no mask or the causal mask (-1 = the library's choice) for later calls;
    returns the status code."""
    return load().attn_set_key_groups(key_groups)


def attn_set_work_queue(mode: int) -> int:
    """C ``attn_set_work_queue``: the bf16 forward's work queue (1 = on, 0 = off,
    -1 = the library's choice) for later calls; returns the status code."""
    return load().attn_set_work_queue(mode)


def attn_strerror(status: int) -> str:
    return load().attn_strerror(status).decode()


def attn_version() -> str:
    return load().attn_version().decode()


def _same_device(dev, **tensors):
    """Every named tensor must be a device tensor on ``dev`` (a host tensor's
    pointer would reach the kernels as is)."""
    for name, t in tensors.items():
        if t is None:
            continue
        if not getattr(t, "is_cuda", False) or t.device != dev:
            raise ValueError(f"{name} must be a device tensor on {dev}")


def _like(name, t, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {tuple(shape)}")


def _stream(stream, dev):
    """(torch stream object, raw hipStream_t) for ``stream``: None for torch's
    current stream on ``dev``, a torch stream, or a raw handle as an int.  The
    binding allocates its temporaries and outputs on that stream, so torch's caching
    allocator never hands their memory to other work while the kernels that use them
    are still queued there."""
    import torch

    if stream is None:
        s = torch.cuda.current_stream(dev)
    elif isinstance(stream, torch.cuda.Stream):
        s = stream
    else:
        h = int(stream)
        s = torch.cuda.default_stream(dev) if h == torch.cuda.default_stream(dev).cuda_stream \
            else torch.cuda.ExternalStream(h, device=dev)
    return s, s.cuda_stream


def fwd(q, k, v, mask="none", window=0, scale=None, out=None, lse=None, stream=None):
    """Attention forward on torch device tensors [B, H, N, d] (bf16 or fp32).

    Allocates ``out`` ([B, H, N, d], input dtype) and ``lse`` ([B, H, N], fp32)
    unless given, enqueues the kernel on ``stream`` (default: torch's current
    stream) and returns (out, lse).  Raises AttnError on any non-zero status."""
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors of one shape")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be device tensors")
    _same_device(q.device, k=k, v=v, out=out, lse=lse)
    for t in (q, k, v):
        if not t.is_contiguous():
            raise ValueError("q, k, v must be contiguous")
    B, H, N, d = q.shape
    if out is not None:
        _like("out", out, q.shape, q.dtype)
    if lse is not None:
        _like("lse", lse, (B, H, N), torch.float32)
    if scale is None:
        scale = d ** -0.5
    mk = MASKS[mask] if isinstance(mask, str) else int(mask)
    dt = ATTN_DTYPE_BF16 if q.dtype == torch.bfloat16 else ATTN_DTYPE_F32
    s, raw = _stream(stream, q.device)
    if out is not None and lse is not None and torch.cuda.current_device() == q.device.index:
        # nothing to allocate and the device is current: launch directly (the
        # launch-bound small shapes pay for every context switch)
        st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                      B, H, N, d, float(scale), mk, int(window), dt, raw)
    else:
        with torch.cuda.device(q.device), torch.cuda.stream(s):
            if out is None:
                out = torch.empty_like(q)
            if lse is None:
                lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
            st = attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                          B, H, N, d, float(scale), mk, int(window), dt, raw)
    if st != ATTN_OK:
        raise AttnError(st, attn_strerror(st))
    return out, lse


def bwd(q, k, v, out, dout, lse, mask="none", window=0, scale=None, dq=None, dk=None, dv=None, stream=None):
    """Attention backward on torch device tensors: (dq, dk, dv) for the upstream
    gradient ``dout`` of ``out``, where ``out, lse = fwd(q, k, v, mask, window,
    scale)``.  bf16 [B, H, N, d] tensors; lse fp32 [B, H, N].  Allocates the
    gradients unless given and enqueues on ``stream`` (default: torch's current
    stream).  Raises AttnError on any non-zero status."""
    import torch

    ts = (q, k, v, out, dout)
    if q.dim() != 4 or any(t.shape != q.shape for t in ts):
        raise ValueError("q, k, v, out, dout must be [B, H, N, d] tensors of one shape")
    if any(t.dtype != torch.bfloat16 for t in ts):
        raise ValueError("the backward takes bfloat16 tensors")
    if not getattr(q, "is_cuda", False):
        raise ValueError("inputs must be contiguous device tensors")
    _same_device(q.device, k=k, v=v, out=out, dout=dout, lse=lse, dq=dq, dk=dk, dv=dv)
    if not all(t.is_contiguous() for t in ts) or not lse.is_contiguous():
        raise ValueError("inputs must be contiguous device tensors")
    B, H, N, d = q.shape
    if lse.shape != (B, H, N) or lse.dtype != torch.float32:
        raise ValueError("lse must be a float32 [B, H, N] tensor")
    for name, g in (("dq", dq), ("dk", dk), ("dv", dv)):
        if g is not None:
            _like(name, g, q.shape, q.dtype)
    if scale is None:
        scale = d ** -0.5
    mk = MASKS[mask] if isinstance(mask, str) else int(mask)
    s, raw = _stream(stream, q.device)
    with torch.cuda.device(q.device), torch.cuda.stream(s):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(q) if dk is None else dk
        dv = torch.empty_like(q) if dv is None else dv
        st = attn_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(), lse.data_ptr(),
                      dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), B, H, N, d, float(scale), mk, int(window),
                      ATTN_DTYPE_BF16, raw)
    if st != ATTN_OK:
        raise AttnError(st, attn_strerror(st))
    return dq, dk, dv


def fwd_kv(q, k, v, q_offset=None, mask="none", window=0, scale=None, out=None, lse=None, workspace=None,
           stream=None):
    """Attention of Nq new queries against Nk cached keys on torch device tensors:
    q [B, H, Nq, d], k and v [B, H, Nk, d], all bf16; query row i sits at position
    ``q_offset + i`` (default ``Nk - Nq``: the queries are the last Nq tokens).
    Allocates ``out``, ``lse`` and the workspace unless given, enqueues on
    ``stream`` (default: torch's current stream) and returns (out, lse).  Raises
    AttnError on any non-zero status."""
    import torch

    if q.dim() != 4 or k.dim() != 4 or k.shape != v.shape or q.shape[:2] != k.shape[:2] or q.shape[3] != k.shape[3]:
        raise ValueError("q must be [B, H, Nq, d] and k, v [B, H, Nk, d]")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)):
        raise ValueError("attn_fwd_kv takes bfloat16 tensors")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v must be contiguous device tensors")
    _same_device(q.device, k=k, v=v, out=out, lse=lse, workspace=workspace)
    if not all(t.is_contiguous() for t in (q, k, v)):
        raise ValueError("q, k, v must be contiguous device tensors")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    if q_offset is None:
        q_offset = Nk - Nq
    if out is not None:
        _like("out", out, q.shape, q.dtype)
    if lse is not None:
        _like("lse", lse, (B, H, Nq), torch.float32)
    if workspace is not None and not workspace.is_contiguous():
        raise ValueError("workspace must be contiguous")
    need = attn_fwd_kv_workspace_size(B, H, Nq, Nk, d)
    if scale is None:
        scale = d ** -0.5
    mk = MASKS[mask] if isinstance(mask, str) else int(mask)
    s, raw = _stream(stream, q.device)
    with torch.cuda.device(q.device), torch.cuda.stream(s):
        out = torch.empty_like(q) if out is None else out
        if lse is None:
            lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        ws_ptr = workspace.data_ptr() if workspace is not None else 0
        ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
        st = attn_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, Nq, Nk, d,
                         float(scale), mk, int(window), int(q_offset), ATTN_DTYPE_BF16, ws_ptr, ws_bytes, raw)
    if st != ATTN_OK:
        raise AttnError(st, attn_strerror(st))
    return out, lse


def fwd_block_sparse(q, k, v, layout, causal=False, scale=None, out=None, lse=None, stream=None):
    """Block-sparse attention on torch device tensors: q, k, v bf16 [B, H, N, d];
    ``layout`` a uint8 (or bool) device tensor [H, nb, nb], nb = ceil(N / 128),
    nonzero = the 128 x 128 block is allowed.  Allocates ``out`` and ``lse`` unless
    given, enqueues on ``stream`` (default: torch's current stream) and returns
    (out, lse).  Raises AttnError on any non-zero status."""
    import torch

    if q.dim() != 4 or q.shape != k.shape or q.shape != v.shape:
        raise ValueError("q, k, v must be [B, H, N, d] tensors of one shape")
    if any(t.dtype != torch.bfloat16 for t in (q, k, v)):
        raise ValueError("the block-sparse forward takes bfloat16 tensors")
    if not getattr(q, "is_cuda", False):
        raise ValueError("q, k, v and layout must be contiguous device tensors")
    _same_device(q.device, k=k, v=v, layout=layout, out=out, lse=lse)
    if not all(t.is_contiguous() for t in (q, k, v, layout)):
        raise ValueError("q, k, v and layout must be contiguous device tensors")
    B, H, N, d = q.shape
    nb = -(-N // ATTN_BLOCK_SPARSE_BLOCK)
    if layout.dtype not in (torch.bool, torch.uint8) or tuple(layout.shape) != (H, nb, nb):
        raise ValueError(f"layout must be a uint8 (or bool) tensor [H, {nb}, {nb}]")
    if out is not None:
        _like("out", out, q.shape, q.dtype)
    if lse is not None:
        _like("lse", lse, (B, H, N), torch.float32)
    if scale is None:
        scale = d ** -0.5
    s, raw = _stream(stream, q.device)
    with torch.cuda.device(q.device), torch.cuda.stream(s):
        if layout.dtype == torch.bool:
            layout = layout.to(torch.uint8)     # the copy runs on the launch stream, before the kernel
        out = torch.empty_like(q) if out is None else out
        if lse is None:
            lse = torch.empty((B, H, N), dtype=torch.float32, device=q.device)
        st = attn_fwd_block_sparse(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(), B, H, N,
                                   d, float(scale), 1 if causal else 0, layout.data_ptr(), ATTN_DTYPE_BF16, raw)
    if st != ATTN_OK:
        raise AttnError(st, attn_strerror(st))
    return out, lse
