"""Fixtures in tests/golden/formula_cases.json: oracle outputs on inputs given by a
closed formula (written by tests/golden/make_golden.py, which calls only the
oracle).

* CPU: the oracle still reproduces every stored value (a regression guard on the
  oracle's arithmetic; any intended change to it regenerates the file and names
  the passage that justifies it).
* GPU: both HIP paths (fp32 and bf16; every input is exact in bf16) match the
  stored values within the parity tolerances.
"""
from __future__ import annotations

import json
import os
import sys

import numpy as np
import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, os.path.join(HERE, "golden"))

from make_golden import formula_qkv  # noqa: E402
from oracle.attention_ref import attention_forward  # noqa: E402

with open(os.path.join(HERE, "golden", "formula_cases.json"), encoding="utf-8") as _f:
    CASES = json.load(_f)["cases"]
IDS = [c["name"] for c in CASES]


@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_oracle_reproduces_fixture(case):
    q, k, v = formula_qkv(case["N"], case["d"])
    O, L = attention_forward(q, k, v, case["scale"], case["mask_kind"], case["window"])
    assert np.max(np.abs(O[0, 0] - np.asarray(case["O"]))) <= 1e-13
    assert np.max(np.abs(L[0, 0] - np.asarray(case["LSE"]))) <= 1e-13


def test_formula_inputs_exact_in_bf16():
    import torch
    for case in CASES:
        for x in formula_qkv(case["N"], case["d"]):
            t = torch.from_numpy(x)
            assert torch.equal(t.to(torch.bfloat16).double(), t)


@pytest.mark.gpu
@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("case", CASES, ids=IDS)
def test_gpu_matches_fixture(case, dtype):
    import torch
    import exact_blockwise_attention_attn_amd as attn

    assert torch.cuda.is_available(), "GPU test run without a GPU"
    tdt = torch.float32 if dtype == "f32" else torch.bfloat16
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(x).to(tdt).to(dev) for x in formula_qkv(case["N"], case["d"]))
    mask = {0: "none", 1: "causal", 2: "window"}[case["mask_kind"]]
    print(f"golden {case['name']} {dtype}", flush=True)
    out, lse = attn.fwd(q, k, v, mask=mask, window=case["window"], scale=case["scale"])
    torch.cuda.synchronize()
    tol_o = 1e-5 if dtype == "f32" else 2e-2
    tol_l = 1e-5 if dtype == "f32" else 1e-3
    do = np.max(np.abs(out[0, 0].double().cpu().numpy() - np.asarray(case["O"])))
    dl = np.max(np.abs(lse[0, 0].double().cpu().numpy() - np.asarray(case["LSE"])))
    assert do <= tol_o and dl <= tol_l, (do, dl)
