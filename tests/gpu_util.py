"""Helpers for the GPU parity tests: run the HIP path through the binding, run
the CPU oracle on the same inputs (threads over heads) and compare."""
from __future__ import annotations

import concurrent.futures as cf
import os
import sys

import numpy as np
import torch
from threadpoolctl import threadpool_limits

import exact_blockwise_attention_attn_amd as attn
from exact_blockwise_attention_attn_amd.inputs import make_qkv, row_seed, sample_rows
from oracle.attention_ref import attention_forward

# Tolerances: fp32 inputs 1e-5 on O; bf16 inputs 2e-2 on O; LSE 1e-3 (1e-5 for fp32).
TOL = {"f32": dict(o=1e-5, lse=1e-5), "bf16": dict(o=2e-2, lse=1e-3)}
REL_RMS_BF16 = 1e-2        # stricter internal bar on the relative RMS error per head

WORKERS = max(1, min(16, len(os.sched_getaffinity(0))))


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def require_gpu():
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    attn.load()


def to_np(t):
    return t.detach().float().cpu().numpy()


def oracle(qn, kn, vn, scale, mask_kind, window, rows=None):
    """Oracle over all (b, h) in parallel threads; rows None, [R] or [B, H, R]."""
    B, H = qn.shape[:2]
    if rows is None:
        rows = np.broadcast_to(np.arange(qn.shape[2]), (B, H, qn.shape[2]))
    elif rows.ndim == 1:
        rows = np.broadcast_to(rows, (B, H, rows.shape[0]))
    R = rows.shape[-1]
    O = np.empty((B, H, R, qn.shape[3]))
    L = np.empty((B, H, R))

    done = [0]
    big = R * qn.shape[2] >= (1 << 26)

    def one(bh):
        b, h = divmod(bh, H)
        o, l = attention_forward(qn[b:b + 1, h:h + 1], kn[b:b + 1, h:h + 1], vn[b:b + 1, h:h + 1], scale,
                                 mask_kind, window, rows=rows[b, h])
        O[b, h] = o[0, 0]
        L[b, h] = l[0, 0]
        done[0] += 1
        if big:
            say(f"    oracle: {done[0]}/{B * H} heads")

    # one BLAS thread per worker: the workers already cover the cores
    with threadpool_limits(limits=1), cf.ThreadPoolExecutor(WORKERS) as ex:
        list(ex.map(one, range(B * H)))
    return O, L, rows


def gather_rows(x, rows):
    """x: numpy [B, H, N, ...]; rows [B, H, R] -> [B, H, R, ...]."""
    B, H = rows.shape[:2]
    return np.stack([np.stack([x[b, h, rows[b, h]] for h in range(H)]) for b in range(B)])


def compare(out, lse, O_ref, L_ref, rows, dtype, label=""):
    """Element-wise comparison on the checked rows; returns a stats dict."""
    on = gather_rows(to_np(out), rows)
    ln = gather_rows(to_np(lse), rows)
    assert np.all(np.isfinite(on)), f"{label}: non-finite O"
    assert np.all(np.isfinite(ln)), f"{label}: non-finite LSE"
    d_o = np.abs(on - O_ref)
    d_l = np.abs(ln - L_ref)
    num = np.sqrt(((on - O_ref) ** 2).sum(axis=(2, 3)))
    den = np.sqrt((O_ref ** 2).sum(axis=(2, 3)))
    rel_rms = float(np.max(num / np.maximum(den, 1e-300)))
    st = dict(max_do=float(d_o.max()), max_dlse=float(d_l.max()), rel_rms=rel_rms,
              max_o=float(np.abs(O_ref).max()), rows=int(rows.shape[-1]))
    say(f"  {label}: max|dO|={st['max_do']:.3e} max|dLSE|={st['max_dlse']:.3e} rel_rms={rel_rms:.3e} "
        f"max|O|={st['max_o']:.3e} rows/head={st['rows']}")
    tol = TOL[dtype]
    assert st["max_do"] <= tol["o"], f"{label}: max|dO| {st['max_do']} > {tol['o']}"
    assert st["max_dlse"] <= tol["lse"], f"{label}: max|dLSE| {st['max_dlse']} > {tol['lse']}"
    if dtype == "bf16":
        assert rel_rms <= REL_RMS_BF16, f"{label}: rel RMS {rel_rms}"
    return st


def run_case(B, H, N, d, dtype, mask, window=0, scale=None, seed=0, q_mult=1.0, n_rows=None,
             name="case", gen_device="cpu", rows_per_wave=None):
    """Generate seeded inputs, run the HIP path, check against the oracle."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    scale = float(np.float32(scale if scale is not None else d ** -0.5))
    mk = attn._lib.MASKS[mask]
    label = f"{name} B{B} H{H} N{N} d{d} {dtype} {mask} w{window} seed{seed} qx{q_mult}"
    say(f"[gpu] {label}")
    q, k, v = make_qkv(B, H, N, d, tdt, seed=seed, q_mult=q_mult, device=gen_device)
    qd, kd, vd = (t.cuda() for t in (q, k, v))
    # bf16: each tile shape the library can pick (32 or 64 query rows per wave, with
    # the library's key groups or one key group), forced in turn, against the one
    # oracle result
    rows = ROWS_PER_WAVE if (dtype == "bf16" and rows_per_wave is None) else (rows_per_wave,)
    groups = ("auto", "1") if (dtype == "bf16" and mask in ("none", "causal")) else (None,)
    outs = []
    for rpw in rows:
        for kg in groups:
            with forced_rows_per_wave(rpw), forced_key_groups(kg):
                out, lse = attn.fwd(qd, kd, vd, mask=mask, window=window, scale=scale)
                torch.cuda.synchronize()
            outs.append((f"{rpw or 'auto'} key groups={kg or 'auto'}", out, lse))
    qn, kn, vn = to_np(q), to_np(k), to_np(v)
    if n_rows is None or n_rows >= N:
        rows = None
    else:
        rows = np.stack([np.stack([sample_rows(N, n_rows, row_seed(name, seed, b, h), window)
                                   for h in range(H)]) for b in range(B)])
    O_ref, L_ref, rows = oracle(qn, kn, vn, scale, mk, window, rows)
    res = None
    for shape, out, lse in outs:
        res = compare(out, lse, O_ref, L_ref, rows, dtype, f"{label} rows/wave={shape}")
    return res


ROWS_PER_WAVE = ("32", "64")


_SCHED = {"rows_per_wave": 0, "head_group": -1, "key_groups": -1}   # what the library was last given


class _forced:
    """Context manager: force one schedule choice of the library (rows per wave or
    head-group size) through attn_set_schedule, restoring the previous one on exit.
    Every choice computes the same result; the tests run each against one oracle."""

    def __init__(self, key, value):
        self.key, self.value, self.old = key, value, None

    def __enter__(self):
        self.old = _SCHED[self.key]
        if self.value is not None:
            # "auto": the library's own choice (rows per wave 0, head group and key groups -1)
            _SCHED[self.key] = (0 if self.key == "rows_per_wave" else -1) if self.value == "auto" else int(self.value)
            _apply()
        return self

    def __exit__(self, *exc):
        _SCHED[self.key] = self.old
        _apply()
        return False


def _apply():
    assert attn.attn_set_schedule(_SCHED["rows_per_wave"], _SCHED["head_group"]) == 0
    assert attn.attn_set_key_groups(_SCHED["key_groups"]) == 0


def forced_rows_per_wave(rpw):
    """Force 32 or 64 query rows per wave of the bf16 forward (None: the library's choice)."""
    return _forced("rows_per_wave", rpw)


def forced_head_group(g):
    """Force the head-group size (n heads, 0 for one group; None: the library's choice)."""
    return _forced("head_group", g)


def forced_key_groups(g):
    """Force 1, 2 or 4 key groups of the bf16 forward (None: the library's choice)."""
    return _forced("key_groups", g)
