"""The host side of the C ABI under AddressSanitizer (CPU only, no device call).

attn_api.cpp (argument checks, workspace sizing, schedule switches, status text)
is compiled with the sanitizer on its host pass only and linked with the
library's other objects into a throw-away libattn_asan.so.  A child Python process
with the sanitizer runtime preloaded then drives every host-only entry point with
edge and random arguments: null, overlapping and misaligned pointers, zero,
negative and overflowing sizes, non-finite scales, unknown masks and dtypes,
status codes far outside the table.  None of these calls reaches a device: each
is rejected on the host, or is a pure host function.  Any sanitizer report fails
the test."""
from __future__ import annotations

import os
import shutil
import subprocess
import sys

import pytest

from exact_blockwise_attention_attn_amd import _build

CLANG = "/opt/rocm/llvm/bin/clang++"

DRIVER = r'''
import ctypes, random, sys
lib = ctypes.CDLL(sys.argv[1])
vp, i, f, u64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.c_ulonglong
lib.attn_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i]
lib.attn_bwd_check_args.argtypes = [vp] * 9 + [i, i, i, i, f, i, i, i]
lib.attn_fwd_kv_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp, u64]
lib.attn_fwd_block_sparse_check_args.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, vp, i]
lib.attn_fwd_kv_workspace_size.argtypes = [i, i, i, i, i]
lib.attn_fwd_kv_workspace_size.restype = u64
lib.attn_strerror.argtypes = [i]
lib.attn_strerror.restype = ctypes.c_char_p
lib.attn_version.restype = ctypes.c_char_p
lib.attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, f, i, i, i, vp]
lib.attn_fwd_kv_noalloc.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, f, i, i, i, i, vp]
rng = random.Random(7)
INTS = [0, 1, -1, 2, 63, 64, 127, 128, 129, 255, 4096, 8192, 65535, 1 << 20, 2**31 - 1, -2**31]
FLOATS = [0.0, 0.125, -0.125, 1e30, -1e30, float("inf"), float("-inf"), float("nan"), 1e-45]
BASE = 1 << 40
def ptr():
    c = rng.random()
    if c < 0.1:
        return None
    if c < 0.2:
        return BASE + rng.randrange(1, 16)                  # misaligned
    return BASE + 16 * rng.randrange(0, 1 << 20)            # may overlap another
def iv():
    return rng.choice(INTS) if rng.random() < 0.6 else rng.randrange(-10, 5000)
n = 0
for _ in range(4000):
    lib.attn_check_args(*[ptr() for _ in range(5)], iv(), iv(), iv(), rng.choice([64, 128, iv()]), rng.choice(FLOATS),
                        rng.randrange(-2, 6), iv(), rng.randrange(-2, 4))
    lib.attn_bwd_check_args(*[ptr() for _ in range(9)], iv(), iv(), iv(), rng.choice([64, 128, iv()]),
                            rng.choice(FLOATS), rng.randrange(-2, 6), iv(), rng.randrange(-2, 4))
    lib.attn_fwd_kv_check_args(*[ptr() for _ in range(5)], iv(), iv(), iv(), iv(), rng.choice([64, 128, iv()]),
                               rng.choice(FLOATS), rng.randrange(-2, 6), iv(), iv(), rng.randrange(-2, 4), ptr(),
                               rng.choice([0, 16, 1 << 20, 2**63]))
    lib.attn_fwd_block_sparse_check_args(*[ptr() for _ in range(5)], iv(), iv(), iv(), rng.choice([64, 128, iv()]),
                                         rng.choice(FLOATS), rng.randrange(-2, 3), ptr(), rng.randrange(-2, 4))
    lib.attn_fwd_kv_workspace_size(iv(), iv(), iv(), iv(), rng.choice([64, 128, iv()]))
    n += 5
for s in list(range(-64, 65)) + [2**31 - 1, -2**31]:
    assert lib.attn_strerror(s)
assert lib.attn_version()
for a in (-5, -1, 0, 1, 32, 33, 64, 65, 2**31 - 1):
    for b in (-2, -1, 0, 1, 8, 2**31 - 1):
        lib.attn_set_schedule(a, b)
    lib.attn_set_key_groups(a)
lib.attn_set_schedule(0, -1)
lib.attn_set_key_groups(-1)
# launch entry points whose arguments the host rejects: nothing reaches the device
assert lib.attn_fwd(None, None, None, None, None, 1, 1, 64, 64, 0.1, 0, 0, 1, None) != 0
assert lib.attn_fwd(BASE, BASE + 4096, BASE + 8192, BASE + 12288, BASE + 16384, 1, 1, 64, 96, 0.1, 0, 0, 1, None) != 0
assert lib.attn_fwd_kv_noalloc(BASE, BASE + (1 << 30), BASE + (2 << 30), BASE + (3 << 30), BASE + (4 << 30),
                               1, 255, 256, 512, 128, 0.1, 1, 0, 256, 1, None) != 0
print("calls", n)
'''


def _asan_runtime():
    if not os.path.exists(CLANG):
        return None
    r = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"], capture_output=True, text=True)
    path = r.stdout.strip()
    return path if r.returncode == 0 and os.path.isabs(path) and os.path.exists(path) else None


def test_host_abi_under_address_sanitizer(tmp_path):
    rt = _asan_runtime()
    objs = [os.path.join(_build.OBJ, os.path.splitext(s)[0] + ".o") for s in _build.SOURCES if s != "attn_api.cpp"]
    if shutil.which(_build.HIPCC) is None and not os.path.exists(_build.HIPCC):
        pytest.skip("hipcc not found")
    if rt is None:
        pytest.skip("no sanitizer runtime")
    if not all(os.path.exists(o) for o in objs):
        pytest.skip("library objects not built")
    api_o = str(tmp_path / "attn_api_asan.o")
    so = str(tmp_path / "libattn_asan.so")
    cmd = [_build.HIPCC, *_build.COMMON, "-O1", "-g", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fno-omit-frame-pointer", "-x", "hip", "-c", os.path.join(_build.CSRC, "attn_api.cpp"), "-o", api_o]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([CLANG, "-shared", "-fsanitize=address", api_o, *objs, "-L/opt/rocm/lib", "-lamdhip64",
                        "-Wl,-rpath,/opt/rocm/lib", "-o", so], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    env = dict(os.environ, LD_PRELOAD=rt, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1")
    r = subprocess.run([sys.executable, "-c", DRIVER, so], capture_output=True, text=True, env=env, timeout=600)
    assert "AddressSanitizer" not in r.stderr, r.stderr[-4000:]
    assert r.returncode == 0, r.stderr[-4000:]
    assert r.stdout.startswith("calls"), r.stdout
