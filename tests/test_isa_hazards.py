"""The score MFMAs of the bf16 kernel are inline asm, which the compiler's hazard
padding cannot see into.  Compile the kernel to gfx950 assembly with the build's
flags and check, for every instantiation, that no vector-ALU instruction writes a
source register of an asm MFMA just before it (see tests/isa_hazards.py)."""
from __future__ import annotations

import os
import re
import shutil
import subprocess
import tempfile

import pytest

from exact_blockwise_attention_attn_amd import _build
from tests import isa_hazards



def test_checker_finds_planted_hazard():
    text = "\n".join([
        "v_mov_b32_e32 v23, 0",
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[20:23], a[0:3], v[0:15]",
        ";;#ASMEND",
    ])
    n, found = isa_hazards.check(text)
    assert n == 1 and len(found) == 1


def test_checker_ignores_a_write_overwritten_by_a_load():
    # the source register was last written by an LDS load (waited for), not by the
    # earlier vector-ALU instruction; a direct-to-LDS buffer load only reads its
    # address register and does not count as a rewrite
    text = "\n".join([
        "v_lshl_add_u32 v18, v18, 8, v112",
        "buffer_load_dwordx4 v18, s[4:7], s24 offen lds",
        "ds_read_b128 v[18:21], v121",
        "s_waitcnt lgkmcnt(0)",
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[34:49], v[18:21], a[92:95], 0",
        ";;#ASMEND",
    ])
    assert isa_hazards.check(text) == (1, [])
    planted = text.replace("ds_read_b128 v[18:21], v121", "buffer_load_dwordx4 v19, s[4:7], s24 offen lds")
    n, found = isa_hazards.check(planted)
    assert n == 1 and len(found) == 1 and found[0].startswith("before")


def test_checker_finds_result_register_reused_too_early():
    # an asm MFMA whose result the compiler thinks dead: its registers handed to a
    # vector-ALU value while the MFMA still writes them
    text = "\n".join([
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[16:31], v[34:37], a[80:83], 0",
        ";;#ASMEND",
        "s_nop 1",
        "v_cvt_pk_bf16_f32 v16, v0, s0",
    ])
    n, found = isa_hazards.check(text)
    assert n == 1 and len(found) == 1 and found[0].startswith("after")


def test_checker_accepts_padded_result_and_chain():
    text = "\n".join([
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[16:31], v[34:37], a[80:83], 0",
        ";;#ASMEND",
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[16:31], v[38:41], a[84:87], v[16:31]",
        ";;#ASMEND",
        "s_nop 7",
        "s_nop 7",
        "s_nop 7",
        "v_max_f32_e32 v40, v16, v17",
    ])
    assert isa_hazards.check(text) == (2, [])


def test_checker_ignores_value_replaced_by_mfma():
    text = "\n".join([
        "v_or_b32_e32 v2, v6, v2",
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[18:21], a[80:83], 0",
        ";;#ASMEND",
        ";;#ASMSTART",
        "v_mfma_f32_32x32x16_bf16 v[0:15], v[22:25], a[64:67], v[0:15]",
        ";;#ASMEND",
    ])
    assert isa_hazards.check(text) == (2, [])


@pytest.mark.skipif(shutil.which(_build.HIPCC) is None and not os.path.exists(_build.HIPCC), reason="hipcc not found")
# the d = 128 kernels (4 masks x (rows per wave {32, 64}, plus the split-KV mode at 32)
# + the two block-layout kinds + 2 dense masks x rows per wave {32, 64} x key groups
# {2, 4} + the work-queue form of the 2 dense masks at 64 rows) and the d = 64
# split-KV and block-layout kernels live in attn_fwd_bf16.hip; the dense d = 64
# kernels (4 masks x rows per wave {32, 64}, plus the 8 key-group kernels and the 2
# work-queue kernels) in attn_fwd_bf16_d64.hip, built with its own flags
@pytest.mark.parametrize("src,count", [("attn_fwd_bf16.hip", 30), ("attn_fwd_bf16_d64.hip", 18)])
def test_bf16_kernel_asm_mfma_sources_not_written_by_valu(src, count):
    with tempfile.TemporaryDirectory() as tmp:
        out = os.path.join(tmp, "k.s")
        cmd = [_build.HIPCC, *_build.COMMON, *_build.PER_SOURCE.get(src, []),
               "-x", "hip", "-S", "--cuda-device-only", os.path.join(_build.CSRC, src), "-o", out]
        res = subprocess.run(cmd, capture_output=True, text=True)
        assert res.returncode == 0, res.stderr
        text = open(out, encoding="utf-8").read()
    names = re.findall(r"^(_ZN9attn_bf1610fwd_kernel\w+):", text, re.M)
    assert len(names) == count
    for name in names:
        body = text[text.index(name + ":"):]
        body = body[:body.index(".Lfunc_end")]      # the whole function (early exits included)
        n, found = isa_hazards.check(body)
        assert n > 0, name
        assert not found, (name, found[:3])
