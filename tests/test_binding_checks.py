"""Host-only checks of the torch-tensor wrappers in the binding: every output,
workspace and layout must be a device tensor on q's device, and caller-supplied
outputs must have the right shape, dtype and layout.  Each case raises ValueError
before any pointer reaches the library (there is no GPU here, so device tensors
are stand-ins carrying only the attributes the checks read)."""
import pytest
import torch

from exact_blockwise_attention_attn_amd import _lib

DEV0 = torch.device("cuda", 0)
DEV1 = torch.device("cuda", 1)


class Dev:
    """A stand-in for a device tensor: shape, dtype, device and contiguity."""

    def __init__(self, shape, dtype=torch.bfloat16, device=DEV0, contiguous=True):
        self.shape = torch.Size(shape)
        self.dtype = dtype
        self.device = device
        self.is_cuda = device.type == "cuda"
        self._contig = contiguous

    def dim(self):
        return len(self.shape)

    def is_contiguous(self):
        return self._contig

    def data_ptr(self):
        raise AssertionError("a pointer was taken before the checks rejected the call")


B, H, N, d = 1, 2, 256, 64
SHAPE = (B, H, N, d)


def qkv(**over):
    t = {"q": Dev(SHAPE), "k": Dev(SHAPE), "v": Dev(SHAPE)}
    t.update(over)
    return t["q"], t["k"], t["v"]


HOST = torch.device("cpu")


@pytest.mark.parametrize("kw", [
    dict(out=Dev(SHAPE, device=HOST)), dict(out=Dev(SHAPE, device=DEV1)),
    dict(lse=Dev((B, H, N), torch.float32, device=HOST)), dict(lse=Dev((B, H, N), torch.float32, device=DEV1)),
    dict(out=Dev(SHAPE, torch.float32)), dict(out=Dev((B, H, N - 1, d))), dict(out=Dev(SHAPE, contiguous=False)),
    dict(lse=Dev((B, H, N), torch.bfloat16)), dict(lse=Dev((B, H, N - 1), torch.float32)),
])
def test_fwd_rejects_bad_outputs(kw):
    with pytest.raises(ValueError):
        _lib.fwd(*qkv(), **kw)


@pytest.mark.parametrize("which", ["k", "v"])
@pytest.mark.parametrize("dev", [HOST, DEV1])
def test_fwd_rejects_inputs_elsewhere(which, dev):
    with pytest.raises(ValueError):
        _lib.fwd(*qkv(**{which: Dev(SHAPE, device=dev)}))


def test_fwd_rejects_host_q():
    with pytest.raises(ValueError):
        _lib.fwd(*qkv(q=Dev(SHAPE, device=HOST)))


LSE = Dev((B, H, N), torch.float32)


@pytest.mark.parametrize("name", ["out", "dout", "dq", "dk", "dv"])
@pytest.mark.parametrize("dev", [HOST, DEV1])
def test_bwd_rejects_tensors_elsewhere(name, dev):
    args = dict(out=Dev(SHAPE), dout=Dev(SHAPE), lse=LSE)
    extra = {}
    if name in ("out", "dout"):
        args[name] = Dev(SHAPE, device=dev)
    else:
        extra[name] = Dev(SHAPE, device=dev)
    with pytest.raises(ValueError):
        _lib.bwd(*qkv(), args["out"], args["dout"], args["lse"], **extra)


@pytest.mark.parametrize("dev", [HOST, DEV1])
def test_bwd_rejects_lse_elsewhere(dev):
    with pytest.raises(ValueError):
        _lib.bwd(*qkv(), Dev(SHAPE), Dev(SHAPE), Dev((B, H, N), torch.float32, device=dev))


@pytest.mark.parametrize("name,bad", [("dq", Dev(SHAPE, torch.float32)), ("dk", Dev((B, H, N, 128))),
                                      ("dv", Dev(SHAPE, contiguous=False))])
def test_bwd_rejects_bad_gradients(name, bad):
    with pytest.raises(ValueError):
        _lib.bwd(*qkv(), Dev(SHAPE), Dev(SHAPE), LSE, **{name: bad})


KV = (1, 2, 1000, 128)


@pytest.mark.parametrize("kw", [
    dict(out=Dev((1, 2, 1, 128), device=HOST)), dict(lse=Dev((1, 2, 1), torch.float32, device=DEV1)),
    dict(workspace=Dev((1 << 20,), torch.uint8, device=HOST)), dict(workspace=Dev((1 << 20,), torch.uint8, device=DEV1)),
    dict(workspace=Dev((1 << 20,), torch.uint8, contiguous=False)),
    dict(out=Dev((1, 2, 1, 128), torch.float32)), dict(lse=Dev((1, 2, 2), torch.float32)),
])
def test_fwd_kv_rejects_bad_tensors(kw):
    with pytest.raises(ValueError):
        _lib.fwd_kv(Dev((1, 2, 1, 128)), Dev(KV), Dev(KV), **kw)


NB = 2   # ceil(256 / 128)


@pytest.mark.parametrize("kw", [
    dict(out=Dev(SHAPE, torch.float32)), dict(out=Dev((B, H, N + 1, d))), dict(out=Dev(SHAPE, contiguous=False)),
    dict(lse=Dev((B, H, N), torch.bfloat16)), dict(lse=Dev((B, H, 1), torch.float32)),
    dict(out=Dev(SHAPE, device=HOST)), dict(lse=Dev((B, H, N), torch.float32, device=DEV1)),
])
def test_block_sparse_rejects_bad_outputs(kw):
    with pytest.raises(ValueError):
        _lib.fwd_block_sparse(*qkv(), Dev((H, NB, NB), torch.uint8), **kw)


@pytest.mark.parametrize("layout", [Dev((H, NB, NB), torch.uint8, device=HOST), Dev((H, NB, NB), torch.bool, device=DEV1),
                                    Dev((H, NB, NB + 1), torch.uint8), Dev((H, NB, NB), torch.int32),
                                    Dev((H, NB, NB), torch.uint8, contiguous=False)])
def test_block_sparse_rejects_bad_layouts(layout):
    with pytest.raises(ValueError):
        _lib.fwd_block_sparse(*qkv(), layout)
