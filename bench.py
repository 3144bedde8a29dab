#!/usr/bin/env python3
"""Benchmark of the frame-structured block-sparse attention path on one MI355X.

One step = one pass of the whole path over one batch of synthetic input:
  plan (GPU, fsattn_plan_device) -> head bounds (GPU) -> forward (GPU), on
  one stream.
Inputs are resident in HBM before timing starts. The metric counts live-block
FLOPs only: 4 * d per live (query, key) pair (QK^T and PV), summed over
every head. The default workload is the largest single-GPU one (6 frames x
8160 tokens, 4 heads, d = 128, bf16); workloads 2 and 3 are measured in the
same run with the same protocol and reported under "workloads", as is
workload 4 (16 frames x 1024 tokens, dense, two heads that fail eligibility).

Prints ONE JSON line. The roofline object describes the dominant kernel
(the forward) from HIP events recorded around each of its launches on the
stream it runs on (median and minimum over the timed steps); `traffic` and
`mfma_busy_pct` come from the rocprofv3 summaries in profiles/ when those
were taken on the current kernel source. Bounds and producer repetitions
each follow a 512 MiB scratch write, so that their inputs are not served
from the 256 MB last-level cache. The CPU baseline times the fp64 oracle on
a bounded row sample on the host cores (rank 0, N = 1 only).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import socket
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "live-block attention TFLOP/s and % of bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 2.4 GHz x 4096 flop/clk/CU
PEAK_HBM_GBS = 8000.0
FWD_SOURCES = ["frame_block_sparse_amd/csrc/forward_bf16.hip", "frame_block_sparse_amd/csrc/forward_common.h",
               "frame_block_sparse_amd/csrc/fsattn_internal.h", "frame_block_sparse_amd/csrc/fsattn_schedule.cpp"]


def kernel_source_hash() -> str:
    h = hashlib.sha256()
    for p in FWD_SOURCES:
        with open(os.path.join(ROOT, p), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def _read_summary(name: str):
    """key: value pairs of profiles/<name>.txt (comments stripped), or None if
    absent or taken on a different kernel source."""
    path = os.path.join(ROOT, "profiles", name + ".txt")
    if not os.path.exists(path):
        return None
    kv = {}
    for line in open(path):
        line = line.split("#", 1)[0] if not line.lstrip().startswith("#") else ""
        if ":" in line:
            a, b = line.split(":", 1)
            kv[a.strip()] = b.strip()
    src = kv.get("kernel_source_sha256_16")
    if src is None:   # (the hash may sit in a comment line)
        for line in open(path):
            if "kernel_source_sha256_16:" in line:
                src = line.split("kernel_source_sha256_16:", 1)[1].split()[0]
    if src != kernel_source_hash():
        return None
    return kv


def read_traffic(workload: str):
    """HBM bytes per forward launch from profiles/forward_traffic_<workload>.txt
    (FETCH_SIZE + WRITE_SIZE, scaled by a copy-kernel calibration), or None if
    absent or taken on a different kernel source."""
    kv = _read_summary(f"forward_traffic_{workload}")
    try:
        return float(kv["hbm_bytes_per_launch"]) if kv else None
    except (KeyError, ValueError):
        return None


def read_mfma_busy(workload: str):
    """Percent of SIMD cycles the matrix unit was busy under the forward
    (SQ_VALU_MFMA_BUSY_CYCLES over 1024 SIMDs x active cycles), from
    profiles/forward_counters_<workload>.txt, or None."""
    kv = _read_summary(f"forward_counters_{workload}")
    try:
        return round(100.0 * float(kv["mfma_busy_fraction"]), 1) if kv else None
    except (KeyError, ValueError):
        return None


def partial_tile_share(w, tile: int = 128):
    """How many tile x tile blocks of the attention matrix (sequence padded to
    a multiple of `tile`) would be live and how many of those only partly
    live under this frame mask: the cost the frame-aligned blocks avoid."""
    import numpy as np
    F_, T, N = w.num_frames, w.tokens_per_frame, w.seq_len
    live = np.zeros((F_, F_), dtype=np.int64)   # live[f, g]: key frame g is visible from query frame f
    r = w.ref_frame
    nr = max(1, w.ref_count) if r >= 0 else 0     # reference frames r .. r + nr - 1
    for f in range(F_):
        live[f, max(0, f - w.window_before):min(F_ - 1, f + w.window_after) + 1] = 1
        if nr:
            live[f, r:r + nr] = 1
    if nr and w.ref_queries_global:
        live[r:r + nr, :] = 1
    pre = np.zeros((F_ + 1, F_ + 1), dtype=np.int64)
    pre[1:, 1:] = live.cumsum(0).cumsum(1)
    nt = -(-N // tile)
    lo = np.arange(nt) * tile
    hi = np.minimum(lo + tile, N) - 1            # last real token of each tile
    padded = lo + tile > N
    fa, fb = lo // T, hi // T                     # frames a tile spans
    cnt = (pre[fb[:, None] + 1, fb[None, :] + 1] - pre[fa[:, None], fb[None, :] + 1]
           - pre[fb[:, None] + 1, fa[None, :]] + pre[fa[:, None], fa[None, :]])
    span = (fb - fa + 1)[:, None] * (fb - fa + 1)[None, :]
    any_live = cnt > 0
    # every (query, key) pair live: all frame pairs live and no padding
    all_live = (cnt == span) & ~padded[:, None] & ~padded[None, :]
    n_live, n_partial = int(any_live.sum()), int((any_live & ~all_live).sum())
    return {"tile": tile, "live_tiles": n_live, "partial_tiles": n_partial,
            "partial_frac": round(n_partial / n_live, 4) if n_live else 0.0}


def mfma_reference(dev, reps: int = 5):
    """The pure-MFMA reference loop (fsattn_mfma_probe): 8 waves per CU,
    timed with events; TFLOP/s at the clock the device holds under it."""
    import torch
    import frame_block_sparse_amd as fs
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    wgs, iters = 2 * cus, 20000
    fs.mfma_probe(wgs, iters, dev)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    flops = 0
    for a, b in ev:
        a.record()
        flops = fs.mfma_probe(wgs, iters, dev)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    return {"kernel": "mfma_probe_kernel", "workgroups": wgs, "iters": iters,
            "tflops": round(flops / (ms * 1e-3) / 1e12, 2)}


def prior_art_timing(w, qd, kd, vd, fwd_ms: float, live_flops: float, reps: int = 10):
    """The prior-art comparator (fsattn_prior_art_forward: 128-token tiles,
    window and reference-frame passes, per-element predicates on partly live
    tiles, merge) on the same inputs, timed with events; the forward's
    speedup over it is what frame-aligned blocks and the single pass buy."""
    import torch
    import frame_block_sparse_amd as fs
    out = torch.empty_like(qd)
    ws = torch.empty(max(1, fs.prior_art_workspace_bytes(qd, w)), dtype=torch.uint8, device=qd.device)
    fs.prior_art_forward(qd, kd, vd, w, out=out, workspace=ws)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fs.prior_art_forward(qd, kd, vd, w, out=out, workspace=ws)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)[reps // 2]
    return {"avg_ms": round(ms, 5), "live_tflops": round(live_flops / (ms * 1e-3) / 1e12, 2),
            "forward_speedup": round(ms / fwd_ms, 3),
            "what": "128-token tiles over the padded sequence, window pass + reference-frame pass with "
                    "per-element frame predicates on partly live tiles, online softmax, fp32 (O, lse) merge"}


def mask_variant_timing(w, qd, kd, vd, reps: int = 10):
    """The forward (library default launch) on the same inputs under the mask
    variants: a global reference frame (its queries see every frame), a span
    of 2 reference frames, and a global span of 3. Live FLOPs / average
    launch time from HIP events, against the bf16 peak."""
    import dataclasses
    import torch
    import frame_block_sparse_amd as fs
    from frame_block_sparse_amd import fsattn as F
    out = []
    for rg, nr in ((1, 0), (0, 2), (1, 3)):
        if w.ref_frame < 0 or w.ref_frame + max(1, nr) > w.num_frames:
            continue
        wv = dataclasses.replace(w, ref_queries_global=rg, ref_count=nr)
        m = F.to_mask(wv)
        _, nnz = fs.plan_size(m)
        flops = 4.0 * w.head_dim * w.batch * w.heads * nnz * w.block_q * w.block_k
        dp = fs.plan_on_device(m, qd.device)
        bnd = fs.head_bounds(qd, kd, m)
        o = torch.empty_like(qd)
        for _ in range(3):
            fs.forward(qd, kd, vd, dp, bnd, out=o)
        ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for a, b in ev:
            a.record()
            fs.forward(qd, kd, vd, dp, bnd, out=o)
            b.record()
        torch.cuda.synchronize()
        avg = sum(a.elapsed_time(b) for a, b in ev) / reps
        tf = flops / (avg * 1e-3) / 1e12
        out.append({"ref_queries_global": rg, "ref_count": nr, "live_gflop": round(flops / 1e9, 2),
                    "avg_ms": round(avg, 5), "tflops": round(tf, 1), "frac": round(tf / PEAK_BF16_TFLOPS, 4),
                    "eligible_heads": int(bnd.host()["eligible"].sum())})
    return out


def flush_llc(bufs):
    """Evict the last-level cache (256 MB) before a timed launch: write one
    512 MiB scratch buffer, then read another 512 MiB one (a sum), so that
    the cache ends up holding clean lines of the second buffer and the
    timed kernel neither hits its own inputs nor pays for writing back the
    flush's data."""
    import torch
    wbuf, rbuf, sink = bufs
    wbuf.fill_(0x5A)
    torch.sum(rbuf, dim=0, out=sink)


def make_flush_buffers(dev):
    import torch
    return (torch.empty(512 << 20, dtype=torch.uint8, device=dev),
            torch.ones((512 << 20) // 4, dtype=torch.float32, device=dev),
            torch.zeros((), dtype=torch.float32, device=dev))


def producer_timing(w, dev, bounds_ms: float, flush_buf, reps: int = 20):
    """fsattn_produce at the workload's shape, from a token-major packed
    projection output [B, N, 3, H, d]: RMSNorm(gamma) and rotary embedding of
    Q and K, Q/K/V written head-major, and the bound records. Algorithmic
    bytes: Q, K, V read and written once, plus the second read of K that the
    key-norm maximum needs after the key mean (7 rows of d per token and
    head). Each repetition follows a scratch write that evicts the
    last-level cache. Reported beside the separate bounds call it replaces."""
    import numpy as np
    import torch
    import frame_block_sparse_amd as fs
    import workloads
    x = workloads.make_producer_inputs(w, seed=1)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qkv = torch.from_numpy(np.ascontiguousarray(
        np.stack((x["q"], x["k"], x["v"]), axis=2).transpose(0, 3, 2, 1, 4))).to(td).to(dev)
    views = [qkv[:, :, i].permute(0, 2, 1, 3) for i in range(3)]
    gq, gk, cs, sn = (torch.from_numpy(x[n]).to(dev) for n in ("gamma_q", "gamma_k", "cos", "sin"))
    B, H, N, d = views[0].shape
    out = tuple(torch.empty((B, H, N, d), dtype=td, device=dev) for _ in range(3))
    ws = torch.empty(max(1, fs.head_bounds_workspace_bytes(out[0], w)), dtype=torch.uint8, device=dev)
    bnd = fs.Bounds(torch.empty((B, H, d), dtype=torch.float32, device=dev),
                    torch.empty((B, H, 8), dtype=torch.float32, device=dev))
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    fs.produce(*views, w, gq, gk, 1e-6, cs, sn, out=out, workspace=ws, bounds=bnd)
    for a, b in ev:
        flush_llc(flush_buf)
        a.record()
        fs.produce(*views, w, gq, gk, 1e-6, cs, sn, out=out, workspace=ws, bounds=bnd)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    esz = 2 if w.dtype == "bf16" else 4
    nbytes = 7.0 * B * H * N * d * esz
    return {"median_ms": round(med, 5), "min_ms": round(ms[0], 5), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS,
            "frac": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "separate_bounds_ms": round(bounds_ms, 5), "llc_flushed": True,
            "what": "RMSNorm(gamma) + rotary embedding of Q, K from a token-major QKV projection output, "
                    "Q/K/V written head-major, bound records of the values written (fsattn_produce)"}


def bounds_timing(w, qd, kd, mask, flush_buf, reps: int = 50):
    """fsattn_head_bounds, each repetition after a scratch write that evicts
    the last-level cache; median and minimum of event-timed launches. The
    rate is algorithmic bytes (Q and K read once) over time; the kernels
    read K a second time (mostly from the last-level cache) after the key
    mean is known."""
    import torch
    import frame_block_sparse_amd as fs
    dev = qd.device
    ws = torch.empty(max(1, fs.head_bounds_workspace_bytes(qd, mask)), dtype=torch.uint8, device=dev)
    bnd = fs.Bounds(torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev),
                    torch.empty((w.batch, w.heads, 8), dtype=torch.float32, device=dev))
    fs.head_bounds(qd, kd, mask, workspace=ws, out=bnd)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        flush_llc(flush_buf)
        a.record()
        fs.head_bounds(qd, kd, mask, workspace=ws, out=bnd)
        b.record()
    torch.cuda.synchronize()
    ms = sorted(a.elapsed_time(b) for a, b in ev)
    med = ms[len(ms) // 2]
    esz = 2 if w.dtype == "bf16" else 4
    nbytes = 2.0 * w.batch * w.heads * w.seq_len * w.head_dim * esz
    return {"median_ms": round(med, 5), "min_ms": round(ms[0], 5), "algorithmic_bytes": nbytes,
            "GBps": round(nbytes / (med * 1e-3) / 1e9, 1), "peak_GBps": PEAK_HBM_GBS,
            "frac": round(nbytes / (med * 1e-3) / 1e9 / PEAK_HBM_GBS, 4), "llc_flushed": True,
            "launches": 4}


def sampled_error(w, q, k, v, out, per_frame: int = 16, seed: int = 7):
    """max |O_gpu - O_oracle| over sampled rows (frame edges and `per_frame`
    random rows of every frame, every (batch, head)), and max |O_gpu| over
    every element. The GPU tests compare every element; this is the
    benchmark's own check of the output it timed."""
    import numpy as np
    import oracle
    g = oracle.MaskGeometry(*w.mask_tuple())
    rng = np.random.default_rng(seed)
    rows = []
    for f in range(g.F):
        a = f * g.T
        rows += [a, a + g.T - 1] + list(a + rng.choice(g.T, min(per_frame, g.T), replace=False))
    rows = np.unique(np.array(rows))
    ref, _ = oracle.attention_live_ref(q, k, v, g, rows=rows)
    got = out[:, :, rows].float().cpu().numpy()
    return float(np.abs(got - ref).max()), float(out.float().abs().max().item()), int(len(rows))


def forward_timing(w, qd, kd, vd, dplan, bnd, flags, out, reps: int = 50, warm: int = 5):
    """Event-timed forward launches (library default launch unless flags say
    otherwise): median and minimum over `reps`."""
    import torch
    import frame_block_sparse_amd as fs
    for _ in range(warm):
        fs.forward(qd, kd, vd, dplan, bnd, flags=flags, out=out)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
    for a, b in ev:
        a.record()
        fs.forward(qd, kd, vd, dplan, bnd, flags=flags, out=out)
        b.record()
    torch.cuda.synchronize()
    return sorted(a.elapsed_time(b) for a, b in ev)


def workload_record(idx, dev, flush_buf, flags, reps: int = 50):
    """One workload measured with the headline's protocol minus the step
    loop: forward median/min over `reps` event-timed launches, flushed
    bounds, eligibility, sampled error against the oracle."""
    import torch
    import frame_block_sparse_amd as fs
    from frame_block_sparse_amd import fsattn as F
    import workloads
    w = workloads.workload(idx)
    print(f"[bench] workload {idx} {w.name}: generating inputs", file=sys.stderr, flush=True)
    q, k, v = workloads.make_inputs(w, seed=0)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(td).to(dev) for x in (q, k, v))
    od = torch.empty_like(qd)
    mask = F.to_mask(w)
    _, nnz = fs.plan_size(mask)
    live_flops = 4.0 * w.head_dim * w.batch * w.heads * nnz * w.block_q * w.block_k
    dplan = fs.plan_on_device(mask, dev)
    bnd = fs.head_bounds(qd, kd, mask)
    ms = forward_timing(w, qd, kd, vd, dplan, bnd, flags, od, reps=reps)
    med = ms[len(ms) // 2]
    err, omax, nrows = sampled_error(w, q, k, v, od)
    tf = live_flops / (med * 1e-3) / 1e12
    return {"workload": w.name, "live_gflop": round(live_flops / 1e9, 3), "t_fwd_ms_median": round(med, 5),
            "t_fwd_ms_min": round(ms[0], 5), "tflops": round(tf, 1), "pct_peak_nominal": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            "tflops_at_min": round(live_flops / (ms[0] * 1e-3) / 1e12, 1),
            "mfma_busy_pct": read_mfma_busy(w.name), "eligible_heads": int(bnd.host()["eligible"].sum()),
            "bounds": bounds_timing(w, qd, kd, mask, flush_buf), "max_abs_err": err, "max_abs_out": omax,
            "err_rows_sampled": nrows, "partial_tiles_if_128": partial_tile_share(w)}


def cpu_baseline(w, q, k, v, budget_s: float):
    """fp64 oracle on a bounded sample of query rows (every frame, every
    head), timed on the host cores. Rate in live TFLOP/s."""
    import numpy as np
    import oracle
    g = oracle.MaskGeometry(*w.mask_tuple())
    live_keys_per_row = {f: len(oracle.live_frames(g, f)) * g.T for f in range(g.F)}
    rng = np.random.default_rng(123)

    def sample(per_frame):
        rows = []
        for f in range(g.F):
            rows += list(f * g.T + rng.choice(g.T, min(per_frame, g.T), replace=False))
        return np.array(sorted(rows))

    def timed(rows):
        t0 = time.perf_counter()
        oracle.attention_ref(q, k, v, g, rows=rows)
        return time.perf_counter() - t0

    per_frame = 2
    rows = sample(per_frame)
    t = timed(rows)
    # grow the sample until it takes about the budget (per-call overheads make
    # the first small samples underestimate the rate)
    while t < 0.5 * budget_s and per_frame < g.T:
        per_frame = max(per_frame + 1, min(g.T, int(per_frame * 0.8 * budget_s / max(t, 1e-3))))
        rows = sample(per_frame)
        t = timed(rows)
    flops = sum(4 * w.head_dim * live_keys_per_row[int(r) // g.T] for r in rows) * w.batch * w.heads
    try:
        from threadpoolctl import threadpool_info
        cores = max([i.get("num_threads", 1) for i in threadpool_info()] + [1])
    except Exception:  # pragma: no cover
        cores = len(os.sched_getaffinity(0))
    return {"value": flops / t / 1e12, "unit": "TFLOP/s", "cores": int(cores), "kind": "oracle",
            "sample": f"{len(rows)} of {g.N} query rows ({per_frame} per frame), all {w.batch * w.heads} "
                      f"(batch, head) pairs, fp64 dense-masked numpy, {t:.1f} s wall",
            "seconds": round(t, 2), "host_cpus": len(os.sched_getaffinity(0))}


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", type=int, default=5,
                    help="1..5 (default 5: bf16, 6 frames x 8160 tokens, the largest single-GPU workload)")
    ap.add_argument("--extra-workloads", default="2,3,4",
                    help="comma-separated workloads also measured (forward median/min, flushed bounds, error); "
                         "empty for none")
    ap.add_argument("--waves", type=int, default=0)
    ap.add_argument("--rows", type=int, default=0)
    ap.add_argument("--kstep", type=int, default=0)
    ap.add_argument("--ring", type=int, default=0)
    ap.add_argument("--mode", default="auto", choices=["auto", "online", "fixed"])
    ap.add_argument("--cpu-baseline-seconds", type=float, default=15.0)
    ap.add_argument("--prewarm-seconds", type=float, default=1.0,
                    help="untimed forward launches before the warmup steps, so that the GPU clocks have "
                         "ramped up after the host-side input generation")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true",
                    help="only the timed steps (for profiling runs): no comparator, producer, mask variants, "
                         "extra workloads or oracle check")
    ap.add_argument("--only", choices=["bounds", "producer"], default=None,
                    help="profiling runs: only the flushed bounds (or producer) repetitions on the workload, "
                         "then a one-line JSON of that record")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a plain device-to-device copy of 512 MiB three times (the known-size "
                         "kernel that scales the FETCH_SIZE / WRITE_SIZE counters)")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py: the library runs on one GPU (the path would shard by heads with no "
              "exchange inside it; multi-GPU runs are not part of it). Use --gpus 1.", file=sys.stderr)
        sys.exit(2)

    import torch
    import frame_block_sparse_amd as fs
    from frame_block_sparse_amd import fsattn as F
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    if args.calibrate_copy:
        nbytes = 512 << 20
        src = torch.ones(nbytes // 4, dtype=torch.float32, device=dev)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": nbytes, "launches": 3}), flush=True)
        return
    fs.lib()
    w = workloads.workload(args.workload)
    print(f"[bench] workload {args.workload} {w.name}: generating inputs", file=sys.stderr, flush=True)
    flush_buf = make_flush_buffers(dev)
    if args.only == "producer":
        print(json.dumps({"workload": w.name, "producer": producer_timing(w, dev, 0.0, flush_buf)}), flush=True)
        return
    q, k, v = workloads.make_inputs(w, seed=0)
    td = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    qd, kd, vd = (torch.from_numpy(x).to(td).to(dev) for x in (q, k, v))
    mask = F.to_mask(w)
    if args.only == "bounds":
        print(json.dumps({"workload": w.name, "bounds": bounds_timing(w, qd, kd, mask, flush_buf)}), flush=True)
        return
    od = torch.empty_like(qd)
    nqb, nnz = fs.plan_size(mask)
    flags = fs.make_flags(args.mode, waves=args.waves, rows_per_wave=args.rows, key_step=args.kstep, ring=args.ring)
    waves, rows_pw, kstep, wgs, lds = fs.launch_info(tuple(qd.shape), fs.BF16 if w.dtype == "bf16" else fs.F32,
                                                     mask, flags)
    live_flops = 4.0 * w.head_dim * w.batch * w.heads * nnz * w.block_q * w.block_k
    # the plan is written on the GPU (fsattn_plan_device) into one reused
    # device buffer; the host plan (fsattn_plan) is the same array, checked
    # element for element by the GPU parity tests
    dplan = fs.plan_on_device(mask, dev)
    ws = torch.empty(max(1, fs.head_bounds_workspace_bytes(qd, mask)), dtype=torch.uint8, device=dev)
    bnd = fs.Bounds(torch.empty((w.batch, w.heads, w.head_dim), dtype=torch.float32, device=dev),
                    torch.empty((w.batch, w.heads, 8), dtype=torch.float32, device=dev))
    total = args.warmup + args.steps
    # Timed steps carry only the two events around the forward (each event
    # record costs the stream a few microseconds); the plan and bounds
    # launches are timed with events in a separate, untimed loop.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(total)]

    def step(i):
        fs.plan_on_device(mask, out=dplan)
        fs.head_bounds(qd, kd, mask, workspace=ws, out=bnd)
        ev[i][0].record()
        fs.forward(qd, kd, vd, dplan, bnd, flags=flags, out=od)
        ev[i][1].record()

    print(f"[bench] prewarm {args.prewarm_seconds} s, warmup {args.warmup}", file=sys.stderr, flush=True)
    step(0)
    torch.cuda.synchronize()
    t_pre = time.perf_counter()
    while time.perf_counter() - t_pre < args.prewarm_seconds:
        fs.forward(qd, kd, vd, dplan, bnd, flags=flags, out=od)
        torch.cuda.synchronize()
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    print(f"[bench] timing {args.steps} steps", file=sys.stderr, flush=True)
    t0 = time.perf_counter()
    for i in range(args.warmup, total):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    ms_step = elapsed * 1e3 / args.steps
    fwd_ms = sorted(ev[i][0].elapsed_time(ev[i][1]) for i in range(args.warmup, total))
    fwd_avg = sum(fwd_ms) / len(fwd_ms)
    fwd_med = fwd_ms[len(fwd_ms) // 2]
    # plan launch times (untimed loop, events around each)
    aux = [tuple(torch.cuda.Event(enable_timing=True) for _ in range(2)) for _ in range(args.steps)]
    for a, b in aux:
        a.record()
        fs.plan_on_device(mask, out=dplan)
        b.record()
    torch.cuda.synchronize()
    plan_ms = sorted(a.elapsed_time(b) for a, b in aux)
    value = live_flops / (ms_step * 1e-3) / 1e12
    achieved = live_flops / (fwd_avg * 1e-3) / 1e12
    elig = bnd.host()["eligible"]
    esz = 2 if w.dtype == "bf16" else 4

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "pct_of_bf16_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "prewarm_s": args.prewarm_seconds,
        "host": socket.gethostname(),
        "device_uuid": str(getattr(torch.cuda.get_device_properties(dev), "uuid", "")),
        "config": {
            "workload": w.name, "batch": w.batch, "heads": w.heads, "seq_len": w.seq_len,
            "head_dim": w.head_dim, "frames": w.num_frames, "tokens_per_frame": w.tokens_per_frame,
            "window": [w.window_before, w.window_after], "ref_frame": w.ref_frame,
            "block_q": w.block_q, "block_k": w.block_k, "live_gflop": round(live_flops / 1e9, 3),
            "mode": args.mode, "eligible_heads": int(elig.sum()),
            "launch": {"waves": waves, "rows_per_wave": rows_pw, "key_step": kstep, "workgroups": wgs,
                       "lds_bytes": lds},
        },
        "roofline": {
            "kernel": "fwd_bf16_kernel" if w.dtype == "bf16" else "fwd_f32_kernel",
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(achieved / PEAK_BF16_TFLOPS, 4), "traffic": read_traffic(w.name),
            "avg_launch_ms": round(fwd_avg, 5), "t_fwd_ms_median": round(fwd_med, 5),
            "t_fwd_ms_min": round(fwd_ms[0], 5),
            "frac_at_median": round(live_flops / (fwd_med * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "frac_at_min": round(live_flops / (fwd_ms[0] * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 4),
            "algorithmic_flop_per_launch": live_flops, "mfma_busy_pct": read_mfma_busy(w.name),
        },
        "plan": {"median_ms": round(plan_ms[len(plan_ms) // 2], 5), "nnz": nnz},
    }
    if not args.no_extras:
        print("[bench] bounds (flushed), reference MFMA loop, comparator, producer, variants", file=sys.stderr,
              flush=True)
        bounds = bounds_timing(w, qd, kd, mask, flush_buf)
        result["bounds"] = bounds
        if w.dtype == "bf16":
            ref_mfma = mfma_reference(dev)
            result["roofline"]["measured_mfma_peak"] = ref_mfma
            result["roofline"]["frac_of_measured_peak"] = round(achieved / ref_mfma["tflops"], 4)
            result["prior_art"] = prior_art_timing(w, qd, kd, vd, fwd_avg, live_flops)
            result["mask_variants"] = mask_variant_timing(w, qd, kd, vd)
        result["producer"] = producer_timing(w, dev, bounds["median_ms"], flush_buf)
        result["partial_tiles_if_128"] = partial_tile_share(w)
        print("[bench] output check against the oracle (sampled rows)", file=sys.stderr, flush=True)
        err, omax, nrows = sampled_error(w, q, k, v, od)
        result["max_abs_err"] = err
        result["max_abs_out"] = omax
        result["err_rows_sampled"] = nrows
        extra = [int(x) for x in args.extra_workloads.split(",") if x.strip()]
        extra = [x for x in extra if x != args.workload]
        if extra:
            result["workloads"] = [workload_record(x, dev, flush_buf, flags) for x in extra]
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle, bounded sample)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_baseline_seconds)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
