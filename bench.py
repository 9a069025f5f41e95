#!/usr/bin/env python3
"""Throughput of the exact blockwise attention forward on one MI355X.

One step = one attn_fwd call over the whole workload (default: the LLaMA-7B-shaped
causal case, B=2 H=32 N=8192 d=128 bf16), inputs already resident in HBM.
Prints one JSON line: TFLOP/s of counted FLOPs (4 B H N^2 d dense, halved for
causal, band pairs for the window), the roofline position of the kernel and the
CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline] [--pass fwd|bwd|decode|sparse]

--pass bwd times the backward (attn_bwd: dq, dk, dv from dout, O and LSE) on the
same workload instead, counted as 2.5x the forward's FLOPs (the five products of
the backward: the recomputed scores, dP, dV, dK and dQ).

--pass decode times attn_fwd_kv on a decode workload (one new query per sequence
against a key/value cache; default B=1 H=32 Nk=131072 d=128 causal).  That work is
bound by HBM bandwidth, so the figure is GB/s of the bytes the step must move (the
K and V cache read once, q read, O and LSE written) against the 8 TB/s peak.

--pass sparse times attn_fwd_block_sparse on a BigBird-style block layout (default
B=1 H=32 N=32768 d=128): TFLOP/s counted on the allowed (query, key) pairs only.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "attention fwd TFLOP/s and % of bf16 MFMA peak, d=128 N=8192 causal"
METRIC_BWD = "attention bwd TFLOP/s (2.5x forward FLOPs) and % of bf16 MFMA peak"
METRIC_DECODE = "attention decode (split-KV) GB/s of K/V cache read and % of HBM peak"
METRIC_SPARSE = "block-sparse attention fwd TFLOP/s on allowed pairs and % of bf16 MFMA peak"
# MI355X peaks: dense bf16 MFMA 2.5 PFLOP/s.  The fp32 path runs on the vector ALUs
# (fp32 FMAs and fp64 scores) with packed fp32 instructions disabled in the build, so
# its ceiling is the unpacked vector rate: 256 CUs x 4 SIMDs x 16 lanes x 2 flop x
# 2.4 GHz = 78.6 TFLOP/s (the same as the fp64 vector rate).  The 157.3 TFLOP/s fp32
# figure needs packed issue or fp32 MFMA, neither of which this path uses.
PEAK_TFLOPS = {"bf16": 2500.0, "f32": 78.6}
HBM_PEAK_GBS = 8000.0
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = "exact_blockwise_attention_attn_amd/csrc/"
# the sources each measured workload runs (and the build script, which holds their
# compiler flags): a traffic record stays valid while they are unchanged
BUILD = "exact_blockwise_attention_attn_amd/_build.py"
KERNEL_SOURCES = {
    "fwd": [CSRC + "attn_fwd_bf16.hip", CSRC + "attn_fwd_bf16_d64.hip", CSRC + "attn_tile.h", BUILD],
    "decode": [CSRC + "attn_decode_bf16.hip", CSRC + "attn_fwd_bf16.hip", BUILD],
    "bwd": [CSRC + "attn_bwd_bf16.hip", CSRC + "attn_tile.h", BUILD],
    "f32": [CSRC + "attn_fwd_f32.hip", BUILD],
}


def counted_flops(B, H, N, d, mask, window=0):
    """4 B H N^2 d for no mask, half of it for causal, 4 B H d x (pairs in the band)
    for the window |i - j| <= w and the causal window i - w <= j <= i."""
    if mask == "none":
        return 4 * B * H * N * N * d
    if mask == "causal":
        return 2 * B * H * N * N * d
    w = min(window, N - 1)
    if mask == "causal_window":
        return 4 * B * H * d * (N * (w + 1) - w * (w + 1) // 2)
    if mask != "window":
        raise ValueError(f"unknown mask {mask!r}")
    return 4 * B * H * d * (N * (2 * w + 1) - w * (w + 1))


def algorithmic_bytes(B, H, N, d, eb):
    """Read Q, K, V once, write O once and LSE once."""
    return 4 * B * H * N * d * eb + 4 * B * H * N


def roofline_bound(flops, nbytes, dtype):
    """The roof a workload sits under: its arithmetic intensity (counted flops per
    algorithmic byte) against the ridge point of the unit that does its arithmetic
    (peak flop rate / HBM peak).  Below the ridge the bound is HBM bandwidth."""
    unit = "mfma" if dtype == "bf16" else "alu"
    ridge = PEAK_TFLOPS[dtype] * 1e12 / (HBM_PEAK_GBS * 1e9)
    return (unit if flops / nbytes >= ridge else "hbm"), flops / nbytes, ridge


def _code_only(text):
    """Source text without // comments and blank lines: edits to comments leave the
    hash (and so the recorded traffic) valid, edits to code do not."""
    lines = []
    for line in text.splitlines():
        code = line.split("//", 1)[0].rstrip()
        if code:
            lines.append(code)
    return "\n".join(lines)


def kernel_source_hash(kind="fwd", read=None):
    h = hashlib.sha256()
    for rel in KERNEL_SOURCES[kind]:
        if read is None:
            with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
                text = f.read()
        else:
            text = read(rel)
        h.update(_code_only(text).encode())
    return h.hexdigest()[:16]


def measured_traffic(workload, kind="fwd"):
    """HBM bytes per step from the committed counter runs, only if they were taken
    on the current sources of the kernels the workload runs."""
    try:
        with open(TRAFFIC_FILE, encoding="utf-8") as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    ent = rec.get(workload)
    if not ent or ent.get("source_hash") != kernel_source_hash(kind):
        return None
    return ent.get("bytes_per_launch")


class cpu_threads:
    """Limit the BLAS threads of the oracle baseline to n (n <= 0: leave them)."""

    def __init__(self, n):
        self.n, self.ctx = n, None

    def __enter__(self):
        if self.n > 0:
            from threadpoolctl import threadpool_limits
            self.ctx = threadpool_limits(limits=self.n)
            self.ctx.__enter__()
        return self

    def __exit__(self, *exc):
        if self.ctx is not None:
            self.ctx.__exit__(*exc)
        return False


def cpu_baseline(wl, q, k, v, budget_s=20.0):
    """The oracle, untuned, on a bounded sample of the workload: whole heads, a
    seeded subset of query rows, growing until about ``budget_s`` of CPU time."""
    from oracle.attention_ref import attention_forward
    from exact_blockwise_attention_attn_amd.inputs import sample_rows
    try:
        from threadpoolctl import threadpool_info
        info = threadpool_info()
        threads = max([p.get("num_threads", 1) for p in info] or [1])
        blas = ",".join(sorted({p.get("internal_api", "?") for p in info})) or "?"
    except Exception:  # noqa: BLE001
        threads = 1
        blas = "?"
    rows = sample_rows(wl.N, min(wl.N, 4096), seed=12345, window=wl.window)
    mk = wl.mask_kind
    flops = 0
    heads = 0
    elapsed = 0.0
    BH = wl.B * wl.H
    while heads < BH and elapsed < budget_s:
        b, h = divmod(heads, wl.H)
        qn = q[b:b + 1, h:h + 1].float().cpu().numpy()
        kn = k[b:b + 1, h:h + 1].float().cpu().numpy()
        vn = v[b:b + 1, h:h + 1].float().cpu().numpy()
        ts = time.perf_counter()
        attention_forward(qn, kn, vn, wl.softmax_scale, mk, wl.window, rows=rows)
        elapsed += time.perf_counter() - ts
        heads += 1
        if mk == 0:
            pairs = len(rows) * wl.N
        elif mk == 1:
            pairs = int(np.sum(rows + 1))
        else:
            w = min(wl.window, wl.N - 1)
            pairs = int(np.sum(np.minimum(rows + w, wl.N - 1) - np.maximum(rows - w, 0) + 1))
        flops += 4 * wl.d * pairs
    full = counted_flops(wl.B, wl.H, wl.N, wl.d, wl.mask, wl.window)
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "extrapolated_full_workload_s": round(elapsed * full / flops, 1), "blas": blas,
            "sample": f"{heads} of {BH} (b,h) heads x {len(rows)} seeded query rows each "
                      f"(N={wl.N}, d={wl.d}, {wl.mask}), numpy float64, {elapsed:.1f} s",
            "seconds": elapsed}


def cpu_baseline_bwd(wl, q, k, v, dout, budget_s=20.0):
    """The backward oracle, untuned, on whole heads until about ``budget_s`` of CPU
    time (it has no row-subset mode: a head's gradients need every row)."""
    from oracle.attention_bwd_ref import attention_backward
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    BH = wl.B * wl.H
    per_head = counted_flops(1, 1, wl.N, wl.d, wl.mask, wl.window) * 5 // 2
    heads, elapsed = 0, 0.0
    while heads < BH and elapsed < budget_s:
        b, h = divmod(heads, wl.H)
        args = [x[b:b + 1, h:h + 1].float().cpu().numpy() for x in (q, k, v, dout)]
        ts = time.perf_counter()
        attention_backward(*args, wl.softmax_scale, wl.mask_kind, wl.window)
        elapsed += time.perf_counter() - ts
        heads += 1
    flops = per_head * heads
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "extrapolated_full_workload_s": round(elapsed * BH / heads, 1),
            "sample": f"{heads} of {BH} (b,h) heads, all rows (N={wl.N}, d={wl.d}, {wl.mask}), "
                      f"numpy float64 backward, {elapsed:.1f} s",
            "seconds": elapsed}


def kv_bytes(wl):
    """Bytes one decode step must move: K and V read once, q read, O and LSE written."""
    return 2 * wl.B * wl.H * wl.Nk * wl.d * 2 + 2 * wl.B * wl.H * wl.Nq * wl.d * 2 + 4 * wl.B * wl.H * wl.Nq


def cpu_baseline_kv(wl, q, k, v, budget_s=20.0):
    """The cache oracle, untuned, on whole heads until about ``budget_s`` of CPU time,
    reported in the decode metric's unit (bytes of the heads' K/V per second)."""
    from oracle.attention_kv_ref import attention_forward_kv
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    BH = wl.B * wl.H
    heads, elapsed = 0, 0.0
    while heads < BH and elapsed < budget_s:
        b, h = divmod(heads, wl.H)
        args = [x[b:b + 1, h:h + 1].float().cpu().numpy() for x in (q, k, v)]
        ts = time.perf_counter()
        attention_forward_kv(*args, wl.softmax_scale, wl.mask_kind, wl.window, wl.Nk - wl.Nq)
        elapsed += time.perf_counter() - ts
        heads += 1
    moved = kv_bytes(wl) * heads / BH
    return {"value": round(moved / elapsed / 1e9, 3), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "extrapolated_full_workload_s": round(elapsed * BH / heads, 3),
            "sample": f"{heads} of {BH} (b,h) heads, Nq={wl.Nq} Nk={wl.Nk} d={wl.d} {wl.mask}, numpy float64, "
                      f"{elapsed:.1f} s",
            "seconds": elapsed}


def main_decode(args, torch, attn):
    from exact_blockwise_attention_attn_amd.inputs import KV_HEADLINE, KV_WORKLOADS, make_q_kv

    name = args.workload or KV_HEADLINE
    wl = KV_WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v = make_q_kv(wl.B, wl.H, wl.Nq, wl.Nk, wl.d, torch.bfloat16, seed=args.seed, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.Nq), dtype=torch.float32, device=dev)
    need = attn.attn_fwd_kv_workspace_size(wl.B, wl.H, wl.Nq, wl.Nk, wl.d)
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device=dev)
    off = wl.Nk - wl.Nq

    def step():
        attn.fwd_kv(q, k, v, q_offset=off, mask=wl.mask, window=wl.window, scale=wl.softmax_scale, out=out,
                    lse=lse, workspace=ws)

    warm_up(step, args, torch)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    assert torch.isfinite(out).all() and torch.isfinite(lse).all(), "non-finite output"
    moved = kv_bytes(wl)
    gbs = moved / (ms * 1e-3) / 1e9
    rec = {
        "metric": METRIC_DECODE,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) q and K/V cache drawn on the device",
        "config": {"workload": name, "B": wl.B, "H": wl.H, "Nq": wl.Nq, "Nk": wl.Nk, "d": wl.d, "mask": wl.mask,
                   "q_offset": off, "workspace_bytes": need, "bytes_per_step": moved,
                   "ms_median": round(per_step[len(per_step) // 2], 5), "ms_min": round(per_step[0], 5),
                   "wall_s_timed_region": round(wall, 4),
                   "step": "split-range kernel + log-sum-exp merge kernel"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": measured_traffic(name, "decode")},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_kv(wl, q, k, v, args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


def layout_pairs(layout, N, block, causal):
    """Allowed (query, key) pairs of a block layout [H, nb, nb] (summed over heads)."""
    nb = layout.shape[1]
    sizes = np.minimum(block, N - block * np.arange(nb))           # tokens per block (last one ragged)
    total = 0
    for h in range(layout.shape[0]):
        lay = layout[h] != 0
        if not causal:
            total += int(sizes @ lay.astype(np.int64) @ sizes)
        else:
            for qb in range(nb):
                for kb in np.nonzero(lay[qb, :qb + 1])[0]:
                    if kb < qb:
                        total += int(sizes[qb] * sizes[kb])
                    else:                                       # diagonal block: j <= i
                        total += int(sizes[qb] * (sizes[qb] + 1) // 2)
    return total


def cpu_baseline_sparse(wl, layout, q, k, v, budget_s=20.0):
    """The block-sparse oracle, untuned, on whole heads x 1024 seeded query rows
    until about ``budget_s`` of CPU time, in the line's unit (allowed-pair flops)."""
    from oracle.attention_block_ref import attention_forward_block_sparse, block_allowed
    from exact_blockwise_attention_attn_amd.inputs import sample_rows
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # noqa: BLE001
        threads = 1
    rows = sample_rows(wl.N, 1024, seed=12345)
    BH = wl.B * wl.H
    heads, elapsed, flops = 0, 0.0, 0
    while heads < BH and elapsed < budget_s:
        b, h = divmod(heads, wl.H)
        args = [x[b:b + 1, h:h + 1].float().cpu().numpy() for x in (q, k, v)]
        ts = time.perf_counter()
        attention_forward_block_sparse(*args, wl.softmax_scale, layout[h:h + 1], 128, wl.causal, rows=rows)
        elapsed += time.perf_counter() - ts
        flops += 4 * wl.d * int(block_allowed(layout[h], rows, wl.N, 128, wl.causal).sum())
        heads += 1
    full = 4 * wl.d * layout_pairs(layout, wl.N, 128, wl.causal) * wl.B
    return {"value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
            "extrapolated_full_workload_s": round(elapsed * full / flops, 1),
            "sample": f"{heads} of {BH} (b,h) heads x {len(rows)} seeded query rows each (N={wl.N}, d={wl.d}, "
                      f"BigBird layout), numpy float64, {elapsed:.1f} s",
            "seconds": elapsed}


def main_sparse(args, torch, attn):
    from exact_blockwise_attention_attn_amd.inputs import SPARSE_HEADLINE, SPARSE_WORKLOADS, make_qkv

    name = args.workload or SPARSE_HEADLINE
    wl = SPARSE_WORKLOADS[name]
    dev = torch.device("cuda:0")
    q, k, v = make_qkv(wl.B, wl.H, wl.N, wl.d, torch.bfloat16, seed=args.seed, device="cuda")
    layout = wl.layout(seed=args.seed)
    lay_d = torch.from_numpy(layout).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)

    def step():
        attn.fwd_block_sparse(q, k, v, lay_d, causal=wl.causal, scale=wl.softmax_scale, out=out, lse=lse)

    warm_up(step, args, torch)
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(args.steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per_step = sorted(evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps))
    ms = evs[0].elapsed_time(evs[-1]) / args.steps
    assert torch.isfinite(out).all(), "non-finite output"
    pairs = layout_pairs(layout, wl.N, 128, wl.causal) * wl.B
    flops = 4 * wl.d * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    peak = PEAK_TFLOPS["bf16"]
    rec = {
        "metric": METRIC_SPARSE,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: seeded i.i.d. N(0,1) q, k, v drawn on the device; seeded BigBird-style block layout",
        "config": {"workload": name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "block": 128, "local": wl.local,
                   "global": wl.n_global, "random": wl.n_random, "causal": wl.causal,
                   "layout_density": round(float(layout.mean()), 4), "allowed_pairs": pairs, "flops_per_step": flops,
                   "pct_of_peak": round(100.0 * tflops / peak, 2),
                   "ms_median": round(per_step[len(per_step) // 2], 5), "ms_min": round(per_step[0], 5),
                   "wall_s_timed_region": round(wall, 4)},
        "roofline": {"bound": "mfma", "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(tflops / peak, 4), "traffic": measured_traffic(name, "fwd")},
        "cpu_baseline": None if args.no_cpu_baseline else cpu_baseline_sparse(wl, layout, q, k, v, args.cpu_budget),
    }
    print(json.dumps(rec), flush=True)


WARMUP_MIN_STEPS = 5
WARMUP_MIN_S = 0.2


def warm_up(step, args, torch):
    """Untimed warm-up: exactly --warmup steps when given; by default at least
    WARMUP_MIN_STEPS steps and at least WARMUP_MIN_S seconds of them, so that short
    steps (tens of microseconds) are timed at the clock a sustained run reaches.
    Records the count in args.warmup."""
    if args.warmup is not None:
        for _ in range(args.warmup):
            step()
        torch.cuda.synchronize()
        return
    n = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(WARMUP_MIN_STEPS):
            step()
        n += WARMUP_MIN_STEPS
        torch.cuda.synchronize()
        if time.perf_counter() - t0 >= WARMUP_MIN_S:
            break
    args.warmup = n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=None,
                    help=f"untimed warm-up steps (default: at least {WARMUP_MIN_STEPS} and {WARMUP_MIN_S} s of them)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--pass", dest="which", choices=["fwd", "bwd", "decode", "sparse"], default="fwd")
    ap.add_argument("--seed", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--cpu-threads", type=int, default=0,
                    help="BLAS threads for the oracle baseline (0: every core the process may use; 1 gives the "
                         "per-core figure)")
    ap.add_argument("--cold", action="store_true",
                    help="write a 512 MiB scratch buffer between steps so every step starts with cold L2/MALL "
                         "(steps are then timed one by one, the flush outside each)")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="instead of attention, run a plain device copy of MIB MiB per step (the reference "
                         "kernel for scaling the FETCH_SIZE / WRITE_SIZE counters)")
    ap.add_argument("--work-queue", type=int, default=-1, choices=[-1, 0, 1],
                    help="the bf16 forward's work queue (attn_set_work_queue): 1 on, 0 off, -1 the library's "
                         "choice")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: every (batch, head) is independent, so a multi-GPU run would only "
              "split the heads; run with --gpus 1", file=sys.stderr)
        sys.exit(2)

    import torch
    import exact_blockwise_attention_attn_amd as attn
    from exact_blockwise_attention_attn_amd.inputs import HEADLINE, WORKLOADS, make_qkv

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    attn.load()
    if attn.attn_set_work_queue(args.work_queue) != 0:
        raise SystemExit(f"attn_set_work_queue({args.work_queue}) failed")
    if args.which == "decode":
        main_decode(args, torch, attn)
        return
    if args.which == "sparse":
        main_sparse(args, torch, attn)
        return
    name = args.workload or HEADLINE
    wl = WORKLOADS[name]

    if args.copy_calibration:
        n = args.copy_calibration * (1 << 20) // 4
        src = torch.randn(n, device=dev)
        dst = torch.empty_like(src)
        launches = (args.warmup if args.warmup is not None else WARMUP_MIN_STEPS) + args.steps
        for _ in range(launches):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_calibration_bytes_read": n * 4, "copy_calibration_bytes_written": n * 4,
                          "launches": launches}), flush=True)
        return

    q, k, v = make_qkv(wl.B, wl.H, wl.N, wl.d, wl.torch_dtype, seed=args.seed, device="cuda")
    out = torch.empty_like(q)
    lse = torch.empty((wl.B, wl.H, wl.N), dtype=torch.float32, device=dev)
    flops = counted_flops(wl.B, wl.H, wl.N, wl.d, wl.mask, wl.window)
    if args.which == "bwd":
        if wl.dtype != "bf16":
            print("the backward takes bf16 workloads", file=sys.stderr)
            sys.exit(2)
        flops = flops * 5 // 2
    eb = 2 if wl.dtype == "bf16" else 4

    if args.which == "bwd":
        attn.fwd(q, k, v, mask=wl.mask, window=wl.window, scale=wl.softmax_scale, out=out, lse=lse)
        gen = torch.Generator(device=dev)
        gen.manual_seed(args.seed + 1000)
        dout = torch.randn(q.shape, generator=gen, device=dev).to(q.dtype)
        dq, dk, dv = torch.empty_like(q), torch.empty_like(q), torch.empty_like(q)

        def step():
            attn.bwd(q, k, v, out, dout, lse, mask=wl.mask, window=wl.window, scale=wl.softmax_scale,
                     dq=dq, dk=dk, dv=dv)
    else:
        def step():
            attn.fwd(q, k, v, mask=wl.mask, window=wl.window, scale=wl.softmax_scale, out=out, lse=lse)

    warm_up(step, args, torch)
    # the kernel runs on torch's current stream; the events are recorded on that stream,
    # one before every step and one after the last, so each step's duration is known
    stream = torch.cuda.current_stream()
    scratch = torch.empty(512 << 18, dtype=torch.float32, device=dev) if args.cold else None
    if args.cold:
        per_step = []
        for _ in range(args.steps):
            scratch.fill_(1.0)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            step()
            e1.record(stream)
            torch.cuda.synchronize()
            per_step.append(e0.elapsed_time(e1))
        gpu_ms = sum(per_step)
        wall = float("nan")
    else:
        evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        evs[0].record(stream)
        for i in range(args.steps):
            step()
            evs[i + 1].record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        gpu_ms = evs[0].elapsed_time(evs[-1])
        per_step = [evs[i].elapsed_time(evs[i + 1]) for i in range(args.steps)]
    ms_per_step = gpu_ms / args.steps
    ms_sorted = sorted(per_step)
    ms_median = ms_sorted[len(ms_sorted) // 2]
    ms_min = ms_sorted[0]
    assert torch.isfinite(out).all() and torch.isfinite(lse).all(), "non-finite output"

    tflops = flops / (ms_per_step * 1e-3) / 1e12
    peak = PEAK_TFLOPS[wl.dtype]
    if args.which == "fwd":
        traffic = measured_traffic(name, "fwd" if wl.dtype == "bf16" else "f32")
    else:
        traffic = measured_traffic(name + "/bwd", "bwd")
    alg = algorithmic_bytes(wl.B, wl.H, wl.N, wl.d, eb) if args.which == "fwd" else \
        (5 * wl.B * wl.H * wl.N * wl.d * eb + 3 * wl.B * wl.H * wl.N * wl.d * eb + 4 * wl.B * wl.H * wl.N)
    bound, intensity, ridge = roofline_bound(flops, alg, wl.dtype)
    secs = ms_per_step * 1e-3
    if bound == "hbm":
        roof = {"bound": "hbm", "achieved": round(alg / secs / 1e9, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                "frac": round(alg / secs / 1e9 / HBM_PEAK_GBS, 4), "traffic": traffic}
    else:
        roof = {"bound": bound, "achieved": round(tflops, 2), "peak": peak, "unit": "TFLOP/s",
                "frac": round(tflops / peak, 4), "traffic": traffic}
    roof.update({"algorithmic_bytes": alg, "algorithmic_gbs": round(alg / secs / 1e9, 1),
                 "traffic_gbs": round(traffic / secs / 1e9, 1) if traffic else None,
                 "flop_per_byte": round(intensity, 1), "ridge_flop_per_byte": round(ridge, 1)})
    rec = {
        "metric": METRIC if args.which == "fwd" else METRIC_BWD,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": wl.dtype,
        "data": "synthetic: seeded i.i.d. N(0,1) q, k, v drawn on the device",
        "config": {"workload": name, "B": wl.B, "H": wl.H, "N": wl.N, "d": wl.d, "mask": wl.mask,
                   "window": wl.window, "scale": wl.softmax_scale, "flops_per_step": flops,
                   "pct_of_peak": round(100.0 * tflops / peak, 2), "peak_tflops": peak,
                   "ms_median": round(ms_median, 5), "ms_min": round(ms_min, 5),
                   "tflops_at_median": round(flops / (ms_median * 1e-3) / 1e12, 2),
                   "cold_l2": bool(args.cold), "work_queue": args.work_queue, "wall_s_timed_region": round(wall, 4)},
        "roofline": roof,
        "cpu_baseline": None,
    }
    if not args.no_cpu_baseline:
        with cpu_threads(args.cpu_threads):
            if args.which == "fwd":
                rec["cpu_baseline"] = cpu_baseline(wl, q, k, v, args.cpu_budget)
            else:
                rec["cpu_baseline"] = cpu_baseline_bwd(wl, q, k, v, dout, args.cpu_budget)
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
