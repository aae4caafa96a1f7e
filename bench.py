#!/usr/bin/env python3
"""Throughput of the causal LLA forward on one MI355X.

One step = one full forward (all three phases: moment scan, CG, output scan)
over one batch of the synthetic workload, inputs resident in HBM. Prints one
JSON line: queries/s (one query = one (batch, head, position) row solved),
TFLOP/s of the algorithmic FLOP count, the dominant kernel's roofline
fraction, and the float64 CPU oracle timed on a bounded sample of the same
workload on this host's cores.

Algorithmic FLOPs per causal pair (i, j <= i), d = head dim: 4d for the
moment scan (q.k and w k), 6d per CG iteration (q.k, p.k and U k), 6d for the
output scan (q.k, rho.k and a v). F = d * sum_i (i+1) (10 + 6 T_i), with T_i
the CG iterations query i took.

--backward times lla_backward_ex instead (its own JSON line and FLOP count,
see backward_flops); --decode, --given-rho and --memory-curve time the other
entry points.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK = {  # MI355X published dense peaks
    "mfma_fp16": 2500.0,   # TFLOP/s, fp16/bf16 matrix
    "valu_fp32": 157.3,    # TFLOP/s, fp32 vector
    "hbm": 8000.0,         # GB/s
}


def algorithmic_flops(n: int, d: int, iters: np.ndarray) -> float:
    """iters: [B, H, n] CG iterations per query."""
    pairs = np.arange(1, n + 1, dtype=np.float64)
    return float(d * np.sum(pairs[None, None, :] * (10.0 + 6.0 * iters.astype(np.float64))))


def min_flops(n: int, d: int, iters: np.ndarray) -> float:
    """The count without re-forming the scores in every CG sweep: per causal
    pair 8d (one score product, the moment, rho and output products) plus 4d per
    iteration (p.k and U k), F_min = d sum_i (i+1)(8 + 4 T_i)."""
    pairs = np.arange(1, n + 1, dtype=np.float64)
    return float(d * np.sum(pairs[None, None, :] * (8.0 + 4.0 * iters.astype(np.float64))))


def cg_flops(n: int, d: int, iters: np.ndarray) -> float:
    """The conjugate-gradient share of algorithmic_flops: 6d per causal pair per
    iteration (q.k, p.k and U k)."""
    pairs = np.arange(1, n + 1, dtype=np.float64)
    return float(d * np.sum(pairs[None, None, :] * 6.0 * iters.astype(np.float64)))


def measured_traffic(path: str):
    """HBM bytes (calibrated FETCH_SIZE + WRITE_SIZE) of one launch of the
    conjugate-gradient kernel, from a rocprofv3 summary, or None when the summary
    is missing or was taken on another version of the kernel source."""
    import hashlib
    if not os.path.exists(path):
        return None
    src = os.path.join(ROOT, "local_linear_attention_flashlla_amd", "csrc", "lla_mfma.hip")
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    found_sha, value = None, None
    with open(path) as f:
        for line in f:
            if line.startswith("lla_mfma.hip sha256:"):
                found_sha = line.split(":", 1)[1].strip()
            elif line.startswith("bytes_per_launch cg_kernel:"):
                value = float(line.split(":", 1)[1])
    return value if found_sha == sha else None


def calibration_kernels(torch, dev, mib: int):
    """Kernels whose HBM traffic is known, run once each (after the timed
    region) so that byte counters taken in the same run can be scaled: a fill
    of N MiB (writes N), dst = src + 1 (reads N, writes N), a sum (reads N)."""
    n = (mib << 20) // 4
    src = torch.empty(n, dtype=torch.float32, device=dev)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    src.fill_(1.0)
    torch.cuda.synchronize()
    torch.add(src, 1.0, out=dst)
    torch.cuda.synchronize()
    src.sum()
    torch.cuda.synchronize()
    del src, dst


def _oracle_sample_job(args):
    q, k, v, lam, rows = args
    from threadpoolctl import threadpool_limits
    from oracle import lla_oracle as O
    with threadpool_limits(1):
        t0 = time.perf_counter()
        O.oracle_head(q, k, v, lam, rows=rows)
        return time.perf_counter() - t0, len(rows)


def cpu_baseline(wl, target_rows: int, seed: int = 0):
    """Time the float64 oracle (Cholesky per row, as written) on a seeded
    uniform sample of (b, h, i) rows of the workload, one worker per core."""
    from concurrent.futures import ProcessPoolExecutor
    cores = max(1, min(16, len(os.sched_getaffinity(0))))
    rng = np.random.default_rng(seed)
    B, H, n = wl.B, wl.H, wl.n
    flat = rng.choice(B * H * n, size=min(target_rows, B * H * n), replace=False)
    by_head = {}
    for f in flat:
        bh, i = divmod(int(f), n)
        by_head.setdefault(bh, []).append(i)
    jobs = []
    for bh, rows in by_head.items():
        b, h = divmod(bh, H)
        rows = sorted(rows)
        # split long row lists so every worker gets a share
        for c in range(0, len(rows), 64):
            part = rows[c:c + 64]
            kmax = part[-1] + 1
            jobs.append((wl.q[b, h, :kmax], wl.k[b, h, :kmax], wl.v[b, h, :kmax], wl.lam, part))
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=cores) as ex:
        res = list(ex.map(_oracle_sample_job, jobs))
    wall = time.perf_counter() - t0
    cpu_s = sum(r[0] for r in res)
    nrows = sum(r[1] for r in res)
    # rows are drawn uniformly, so rows / rate estimates the whole workload's
    # time without bias (a row's cost grows with its prefix length)
    full_s = B * H * n * wall / nrows
    return {
        "value": nrows / wall, "unit": "queries/s", "cores": cores, "kind": "oracle",
        "sample": (f"{nrows} rows drawn uniformly (seed {seed}) from the {B}x{H}x{n} rows of "
                   f"the workload; float64 Cholesky per row; {cpu_s:.1f} CPU-s over "
                   f"{wall:.1f} s wall"),
        "full_config_s": full_s,
        "full_config_note": (f"extrapolated, not run: all {B * H * n} rows at the sampled rate "
                             f"on {cores} cores"),
    }


def memory_curve(torch, lla, dev, ns=(1024, 2048, 4096, 8192, 16384), B=1, H=16, d=128):
    """Peak device memory of one forward at the long-sequence shape (B=1, H=16,
    d=128, bf16) for n = 1k .. 16k, on two paths: the blocked matrix-core
    forward and the naive one (pairwise differences z_ij and moment matrices
    Sigma_i materialised; lla_forward_naive). Inputs, output and workspace are
    all allocated here through torch (the library allocates nothing when it
    is handed a workspace). Working memory linear in n shows as a constant
    peak per row; the naive path's grows with n. A naive size whose workspace
    does not fit in the device's free memory is reported from the size query
    alone, not run. Each point also carries the time of that one forward."""
    free_total = torch.cuda.mem_get_info(dev)
    curves = {}
    for path in ("blocked", "naive"):
        rows = []
        for n in ns:
            io = 3 * B * H * n * d * 2 + B * H * n * d * 4
            if path == "naive":
                ws_bytes = lla.naive_workspace_bytes(B, H, n, d, "bf16")
            else:
                ws_bytes = lla.workspace_bytes(B, H, n, d, "bf16", lla.LLA_KERNEL_MFMA)
            torch.cuda.synchronize(dev)
            torch.cuda.empty_cache()
            if ws_bytes == 0 or ws_bytes + io > 0.9 * torch.cuda.mem_get_info(dev)[0]:
                rows.append({"n": n, "run": False, "workspace_bytes": int(ws_bytes),
                             "inputs_outputs_bytes": int(io),
                             "note": "workspace does not fit in free device memory"})
                continue
            base = torch.cuda.memory_allocated(dev)
            gen = torch.Generator(device=dev)
            gen.manual_seed(n)
            qkv = []
            for _ in range(3):
                x = torch.randn((B, H, n, d), device=dev, generator=gen, dtype=torch.float32)
                qkv.append(x.to(torch.bfloat16))
                del x
            q, k, v = qkv
            q /= q.float().norm(dim=-1, keepdim=True).to(torch.bfloat16)
            k /= k.float().norm(dim=-1, keepdim=True).to(torch.bfloat16)
            torch.cuda.synchronize(dev)
            torch.cuda.reset_peak_memory_stats(dev)
            ws = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
            out = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
            t0 = time.perf_counter()
            if path == "naive":
                lla.forward(q, k, v, 1.0, 0, 0.0, out=out, workspace=ws, naive=True)
            else:
                lla.forward(q, k, v, 1.0, 2, 0.0, out=out, workspace=ws, kernel=lla.LLA_KERNEL_MFMA)
            torch.cuda.synchronize(dev)
            ms = (time.perf_counter() - t0) * 1e3
            peak = torch.cuda.max_memory_allocated(dev) - base
            rows.append({"n": n, "run": True, "peak_bytes": int(peak), "workspace_bytes": int(ws_bytes),
                         "inputs_outputs_bytes": int(io),
                         "peak_bytes_per_row": peak / (B * H * n),
                         "workspace_bytes_per_row": ws_bytes / (B * H * n),
                         "forward_ms": ms})
            print(f"[memory] {path} n={n} peak {peak / 2**30:.3f} GiB ({ms:.1f} ms)",
                  file=sys.stderr, flush=True)
            del q, k, v, ws, out, qkv
        curves[path] = rows
    return {"metric": "peak device memory of one forward vs n", "unit": "bytes",
            "config": {"workload": "long-sequence shape", "B": B, "H": H, "d": d,
                       "dtype": "bf16",
                       "blocked": "matrix-core forward, 2 CG steps",
                       "naive": "lla_forward_naive (exact solve)"},
            "device_memory_bytes": int(free_total[1]),
            "data": "synthetic", "curves": curves}


def bench_given_rho(args, torch, lla, wl, q, k, v, out, ws, kernel, kernel_used):
    """Throughput of the output given rho (here the forward's own rho for
    this workload, computed untimed). On the matrix cores it is one sweep over
    the keys and values with a running score reference: 6d FLOPs per causal
    pair (scores, k.rho and the weighted value sum, 2d each), and that kernel
    is the timed one. The vector path runs the forward's moment and output
    scans in its fused kernel: 10d per pair (4d + 6d)."""
    B, H, n, d = wl.B, wl.H, wl.n, wl.d
    rho = torch.empty((B, H, n, d), dtype=torch.float32, device=q.device)
    lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, workspace=ws,
                kernel=kernel, rho=rho)
    torch.cuda.synchronize()

    def step(events=None):
        lla.forward(q, k, v, wl.lam, 0, 0.0, out=out, workspace=ws, kernel=kernel, events=events,
                    rho_in=rho)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events=ev[i])
    torch.cuda.synchronize()
    ms_step = (time.perf_counter() - t0) * 1e3 / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    pairs = B * H * n * (n + 1) / 2.0
    mfma = kernel_used == lla.LLA_KERNEL_MFMA
    flops = (6.0 if mfma else 10.0) * d * pairs
    achieved = flops / (kern_ms * 1e-3) / 1e12
    peak = PEAK["mfma_fp16"] if mfma else PEAK["valu_fp32"]
    rec = {
        "metric": "LLA output given rho: queries/s + TFLOP/s, 1 MI355X",
        "value": B * H * n / (ms_step * 1e-3), "unit": "queries/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": ms_step,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "fp16" if mfma else "f32", "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "n": n, "d": d, "lambda": wl.lam,
                   "kernel": "mfma" if mfma else "valu", "rho": "the forward's own rho"},
        "tflops": flops / (ms_step * 1e-3) / 1e12, "flops_per_step": flops,
        "main_kernel_ms": kern_ms,
        "main_kernel": "one-sweep output for a supplied rho" if mfma else "fused kernel",
        "roofline": {"bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None},
    }
    print(json.dumps(rec), flush=True)
    return 0


def bench_decode(args, torch, lla, dev):
    """Decode throughput: one new query per (batch, head) against n-key caches
    of the workload's shape (the workload's generator for one batch element,
    tiled over --decode-batch). Queries/s = heads answered per second. One
    query per head against n keys is bound by reading the cache: the floor is
    K and V read once. bf16 caches (the workloads here) take one pass over K
    and V (moments, Gram matrix and cross moment together), then a small
    solve per head; the roofline line is that pass against HBM with its
    algorithmic bytes, K and V read once. fp32 caches take the five-kernel
    path that reads K three times and V once; there the line is its Gram
    kernel with K read once. The whole call's rate against K + V read once is
    reported beside it, and the main kernel's matrix-core rate as
    information."""
    from local_linear_attention_flashlla_amd.workloads import make_workload
    wl = make_workload(args.workload, B=1)
    B = args.decode_batch if args.decode_batch > 0 else {"standard": 4, "long": 1, "recall": 8}.get(
        args.workload, 1)
    H, n, d = wl.H, wl.n, wl.d
    if wl.dtype == "f32":
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    else:
        up = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(dev).view(torch.bfloat16)
    k1, v1 = up(wl.k_dev), up(wl.v_dev)
    q1 = up(wl.q_dev[:, :, n - 1])
    k = k1.expand(B, H, n, d).contiguous()
    v = v1.expand(B, H, n, d).contiguous()
    q = q1.expand(B, H, d).contiguous()
    out = torch.empty((B, H, d), dtype=torch.float32, device=dev)
    ws = torch.empty(max(lla.decode_workspace_bytes(B, H, n, d, wl.dtype), 16), dtype=torch.uint8,
                     device=dev)
    iters = torch.empty((B, H), dtype=torch.int32, device=dev)
    lla.decode(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, workspace=ws,
               cg_iters=iters)
    torch.cuda.synchronize()

    def step(events=None):
        lla.decode(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, workspace=ws,
                   events=events)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    steps = max(args.steps, 20)
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(steps)]
    t0 = time.perf_counter()
    for i in range(steps):
        step(events=ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / steps
    gram_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    esz = 2 if wl.dtype == "bf16" else 4
    cache = B * H * n * d * esz
    one_pass = wl.dtype == "bf16"
    if one_pass:
        # per key: G (d^2 multiply-adds), the cross moment (d^2) and the score
        # (d): 2 (2 d^2 + d) FLOPs; the pass reads K and V once
        main_flops = 2.0 * B * H * n * (2 * d * d + d)
        main_bytes = 2 * cache
        main_name, read_bytes, mdtype = "single pass over K and V", 2 * cache, "bf16"
    else:
        # G = sum_j u_j u_j^T is symmetric: its d (d + 1) / 2 distinct entries
        # take d (d + 1) FLOPs per key (a multiply and an add each), n d (d + 1)
        # per head; the kernel forms only the blocks on or above the diagonal
        main_flops = 1.0 * B * H * n * d * (d + 1)
        main_bytes = cache
        main_name, read_bytes, mdtype = "Gram kernel", 4 * cache, "fp16"
    rec = {
        "metric": "LLA decode queries/s (one new query per head), 1 MI355X",
        "value": B * H / (ms * 1e-3), "unit": "queries/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        # bf16 caches: bf16 x bf16 products into fp32 (w k and w v in two bf16
        # terms), CG in fp32; fp32 caches: the Gram kernel's fp16 x fp16
        # products (two fp16 terms), the rest fp32
        "vs_baseline": None, "dtype": mdtype, "data": "synthetic",
        "config": {"workload": f"decode over the {wl.name} caches", "B": B, "H": H, "n": n, "d": d,
                   "input_dtype": wl.dtype,
                   "lambda": wl.lam, "cg_max_iters": wl.cg_max_iters, "cg_rel_tol": wl.cg_rel_tol},
        "cg_iters_mean": float(iters.float().mean().item()),
        "cache_bytes_k_plus_v": 2 * cache,
        "cache_bytes_read_by_the_kernels": read_bytes,
        "whole_call_vs_hbm": {"bytes": 2 * cache, "GBps": 2 * cache / (ms * 1e-3) / 1e9,
                              "frac": 2 * cache / (ms * 1e-3) / 1e9 / PEAK["hbm"]},
        "main_kernel": main_name, "main_kernel_ms": gram_ms,
        "main_kernel_mfma": {"TFLOPs": main_flops / (gram_ms * 1e-3) / 1e12,
                             "frac": main_flops / (gram_ms * 1e-3) / 1e12 / PEAK["mfma_fp16"]},
        "roofline": {"bound": "hbm", "achieved": main_bytes / (gram_ms * 1e-3) / 1e9,
                     "peak": PEAK["hbm"], "unit": "GB/s",
                     "frac": main_bytes / (gram_ms * 1e-3) / 1e9 / PEAK["hbm"],
                     "traffic": None},
    }
    print(json.dumps(rec), flush=True)
    return 0


def backward_flops(n: int, d: int, iters: np.ndarray) -> float:
    """Algorithmic FLOPs of one backward: per causal pair 4d for the moment
    scan it repeats (q.k, w k), 6d for the sweep that forms the adjoint
    right-hand side (q.k, g.v, U k), 6d per adjoint CG iteration (q.k, p.k,
    U k), 10d for the dq sweep (q.k, rho_c.k, y.k, g.v, dL/ds k) and 16d for
    the dk/dv sweep (the same four score products, then dL/ds q, w A y,
    w e rho_c, w A g): d (36 + 6 T_i) per pair, T_i the adjoint iterations of
    query i. Operands carried as two terms count once."""
    pairs = np.arange(1, n + 1, dtype=np.float64)
    return float(d * np.sum(pairs[None, None, :] * (36.0 + 6.0 * iters.astype(np.float64))))


def bench_backward(args, torch, lla, wl, q, k, v, dev):
    """Throughput of lla_backward_ex on the workload: one step = one full
    backward (dq, dk, dv of sum(dout * out)) given the forward's out and rho_c,
    all inputs resident. Queries/s = rows whose gradient contributions are
    formed per second. The roofline line is the adjoint CG kernel (the
    forward's CG kernel on the adjoint right-hand side); on the fp32 vector
    path (--kernel valu, or fp32 inputs) it is the one fused backward kernel."""
    from local_linear_attention_flashlla_amd.workloads import make_cotangent
    B, H, n, d = wl.B, wl.H, wl.n, wl.d
    shape = (B, H, n, d)
    mfma = args.kernel == "mfma" or (
        args.kernel == "auto" and lla.backward_workspace_bytes(B, H, n, d, wl.dtype) > 0)
    kern = lla.LLA_KERNEL_MFMA if mfma else lla.LLA_KERNEL_VALU
    out = torch.empty(shape, dtype=torch.float32, device=dev)
    rho_c = torch.empty(shape, dtype=torch.float32, device=dev)
    fws = torch.empty(max(lla.workspace_bytes(B, H, n, d, wl.dtype, kern), 16),
                      dtype=torch.uint8, device=dev)
    lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, rho_c=rho_c,
                workspace=fws, kernel=kern)
    dout = torch.from_numpy(make_cotangent(B, H, n, d, seed=1)).to(dev)
    dq, dk, dv = (torch.empty(shape, dtype=torch.float32, device=dev) for _ in range(3))
    bws = torch.empty(max(lla.backward_workspace_bytes(B, H, n, d, wl.dtype) if mfma else 0, 16),
                      dtype=torch.uint8, device=dev)
    iters = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    lla.backward(q, k, v, out, dout, rho_c, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, dq=dq, dk=dk,
                 dv=dv, adj_iters=iters, workspace=bws, kernel=kern,
                 flags=lla.LLA_FLAG_SPLIT_U if args.split_u else 0)
    torch.cuda.synchronize()
    iters_np = iters.cpu().numpy()
    flops = backward_flops(n, d, iters_np)
    flops_cg = cg_flops(n, d, iters_np)

    def step(events=None):
        lla.backward(q, k, v, out, dout, rho_c, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, dq=dq, dk=dk,
                     dv=dv, workspace=bws, events=events, kernel=kern,
                     flags=lla.LLA_FLAG_SPLIT_U if args.split_u else 0)

    def fwd():
        lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, rho_c=rho_c,
                    workspace=fws, kernel=kern)

    for _ in range(args.warmup):
        step()
        fwd()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events=ev[i])
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    cg_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    t0 = time.perf_counter()
    for _ in range(args.steps):
        fwd()
    torch.cuda.synchronize()
    fwd_ms = (time.perf_counter() - t0) * 1e3 / args.steps
    # matrix cores: the adjoint CG kernel; vector path: the fused kernel (all of it)
    achieved = (flops_cg if mfma else flops) / (cg_ms * 1e-3) / 1e12
    peak = PEAK["mfma_fp16"] if mfma else PEAK["valu_fp32"]
    rec = {
        "metric": "LLA backward queries/s + TFLOP/s (% MFMA peak) at n=4096,d=128, 1 MI355X",
        "value": B * H * n / (ms * 1e-3), "unit": "queries/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": ms, "higher_is_better": True, "scaling": "weak",
        # matrix cores: score-side products fp16 x fp16 (operands in one or
        # two terms), the dk/dv products bf16 x bf16, all into fp32
        "vs_baseline": None, "dtype": "fp16" if mfma else "f32", "data": "synthetic",
        "config": {"workload": f"backward of the {wl.name} forward", "B": B, "H": H, "n": n, "d": d,
                   "lambda": wl.lam, "cg_max_iters": wl.cg_max_iters, "cg_rel_tol": wl.cg_rel_tol,
                   "input_dtype": wl.dtype, "accumulate": "f32",
                   "kernel": "mfma" if mfma else "valu",
                   "dk_dv_products": "bf16" if mfma else "f32", "split_u": bool(args.split_u)},
        "tflops": flops / (ms * 1e-3) / 1e12, "flops_per_step": flops,
        "adj_iters_mean": float(iters_np.mean()),
        "forward_ms_same_run": fwd_ms,
        "main_kernel": "adjoint conjugate-gradient kernel" if mfma else "fused backward kernel",
        "main_kernel_ms": cg_ms, "main_kernel_flops": flops_cg if mfma else flops,
        "roofline": {"bound": "mfma" if mfma else "alu", "achieved": achieved, "peak": peak,
                     "unit": "TFLOP/s", "frac": achieved / peak, "traffic": None},
    }
    print(json.dumps(rec), flush=True)
    return 0


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--workload", default="standard",
                    choices=["tiny", "piecewise", "standard", "long", "recall"])
    ap.add_argument("--kernel", default="auto", choices=["auto", "valu", "mfma"])
    ap.add_argument("--split-u", action="store_true")
    ap.add_argument("--cpu-rows", type=int, default=8192,
                    help="rows in the CPU-oracle sample (0 = skip)")
    ap.add_argument("--traffic", default=None,
                    help="byte-counter summary to read the main kernel's HBM bytes per launch "
                         "from (default: the one under profiles/ for this workload)")
    ap.add_argument("--calib-mb", type=int, default=0,
                    help="after timing, run three kernels of known traffic on buffers of this "
                         "many MiB, references for the hardware byte counters: a fill (writes "
                         "N MiB), an elementwise copy dst = src + 1 (reads N, writes N) and a "
                         "sum (reads N)")
    ap.add_argument("--given-rho", action="store_true",
                    help="time lla_output_given_rho (moment and output scans, the CG solve "
                         "replaced by a supplied rho) instead of the full forward")
    ap.add_argument("--decode", action="store_true",
                    help="time lla_decode_ex: one new query per head against the workload's "
                         "key and value caches (its last row)")
    ap.add_argument("--decode-batch", type=int, default=0,
                    help="with --decode: batch size B (default: the workload's)")
    ap.add_argument("--backward", action="store_true",
                    help="time lla_backward_ex (dq, dk, dv given the forward's out and rho_c) "
                         "instead of the forward")
    ap.add_argument("--memory-curve", action="store_true",
                    help="instead of timing, print the peak device memory of one forward at "
                         "n = 1k .. 16k (B=1, H=16, d=128), blocked and naive, as one JSON line")
    args = ap.parse_args(argv)

    if args.gpus != 1:
        print(f"bench.py: this build measures one GPU only (asked for --gpus {args.gpus}); "
              "the forward shards by (batch, head) with no communication, so the "
              "whole-job rate is the per-GPU rate times the GPU count.", file=sys.stderr)
        return 2

    import torch
    import local_linear_attention_flashlla_amd as lla
    from local_linear_attention_flashlla_amd.workloads import make_workload
    if not os.path.exists(lla._lib.LIB_PATH):
        from local_linear_attention_flashlla_amd import build as _b
        _b.build()
    if not lla._lib.is_current():
        print(f"bench.py: {lla._lib.LIB_PATH} was built from other sources than this tree's; "
              "rebuild it (python -m local_linear_attention_flashlla_amd.build)", file=sys.stderr)
        return 3
    assert torch.cuda.is_available(), "bench.py needs a HIP device"
    dev = torch.device("cuda:0")
    if args.memory_curve:
        print(json.dumps(memory_curve(torch, lla, dev)), flush=True)
        return 0

    if args.decode:
        return bench_decode(args, torch, lla, dev)

    wl = make_workload(args.workload)
    if wl.dtype == "f32":
        q, k, v = (torch.from_numpy(a).to(dev) for a in (wl.q_dev, wl.k_dev, wl.v_dev))
    else:
        q, k, v = (torch.from_numpy(a.view(np.int16)).to(dev).view(torch.bfloat16)
                   for a in (wl.q_dev, wl.k_dev, wl.v_dev))
    kernel = {"auto": lla.LLA_KERNEL_AUTO, "valu": lla.LLA_KERNEL_VALU,
              "mfma": lla.LLA_KERNEL_MFMA}[args.kernel]
    flags = lla.LLA_FLAG_SPLIT_U if args.split_u else 0
    B, H, n, d = wl.B, wl.H, wl.n, wl.d
    out = torch.empty((B, H, n, d), dtype=torch.float32, device=dev)
    ws_bytes = lla.workspace_bytes(B, H, n, d, wl.dtype, kernel)
    ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)
    kernel_used = kernel
    if kernel == lla.LLA_KERNEL_AUTO:
        kernel_used = lla.LLA_KERNEL_MFMA if ws_bytes > 0 else lla.LLA_KERNEL_VALU

    def step(events=None):
        lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, workspace=ws,
                    kernel=kernel, flags=flags, events=events)

    if args.given_rho:
        return bench_given_rho(args, torch, lla, wl, q, k, v, out, ws, kernel, kernel_used)
    if args.backward:
        return bench_backward(args, torch, lla, wl, q, k, v, dev)

    # iteration counts for the algorithmic FLOP count (untimed)
    iters = torch.empty((B, H, n), dtype=torch.int32, device=dev)
    lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, out=out, workspace=ws,
                kernel=kernel, flags=flags, cg_iters=iters)
    torch.cuda.synchronize()
    iters_np = iters.cpu().numpy()
    flops = algorithmic_flops(n, d, iters_np)
    flops_cg = cg_flops(n, d, iters_np)
    flops_nom = algorithmic_flops(n, d, np.full_like(iters_np, wl.cg_max_iters))
    flops_min = min_flops(n, d, iters_np)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    # (and events around each whole step, on the stream the library launches on)
    sev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(args.steps)]
    t0 = time.perf_counter()
    for i in range(args.steps):
        sev[i][0].record()
        step(events=ev[i])
        sev[i][1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall * 1e3 / args.steps
    kern_ms = float(np.mean([a.elapsed_time(b) for a, b in ev]))
    step_ev = np.array([a.elapsed_time(b) for a, b in sev])

    queries = B * H * n
    value = queries / (ms_step * 1e-3)
    tflops = flops / (ms_step * 1e-3) / 1e12
    if kernel_used == lla.LLA_KERNEL_MFMA:
        bound, peak, unit = "mfma", PEAK["mfma_fp16"], "TFLOP/s"
    else:
        bound, peak, unit = "alu", PEAK["valu_fp32"], "TFLOP/s"
    # the timed kernel: the CG kernel on the matrix-core path (the dominant one),
    # the single fused kernel on the vector path
    achieved = (flops_cg if kernel_used == lla.LLA_KERNEL_MFMA else flops) / (kern_ms * 1e-3) / 1e12
    traffic = measured_traffic(args.traffic or os.path.join(
        ROOT, "profiles", f"lla_cg_kernel_{wl.name}_hbm_bytes.txt")) \
        if kernel_used == lla.LLA_KERNEL_MFMA and not args.split_u else None

    if args.calib_mb > 0:
        calibration_kernels(torch, dev, args.calib_mb)

    cpu = None
    if args.cpu_rows > 0:
        cpu = cpu_baseline(wl, args.cpu_rows)

    rec = {
        "metric": "LLA fwd queries/s + TFLOP/s (% MFMA peak) at n=4096,d=128, 1 MI355X",
        "value": value,
        "unit": "queries/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        # the arithmetic type: bf16 inputs convert exactly to fp16, and the
        # matrix cores multiply fp16 x fp16 into fp32; the fp32 path is fp32
        "dtype": ("fp16" if kernel_used == lla.LLA_KERNEL_MFMA else "f32"),
        "data": "synthetic",
        "config": {"workload": wl.name, "B": B, "H": H, "n": n, "d": d,
                   "lambda": wl.lam, "cg_max_iters": wl.cg_max_iters,
                   "cg_rel_tol": wl.cg_rel_tol,
                   "input_dtype": wl.dtype, "accumulate": "f32",
                   "kernel": {lla.LLA_KERNEL_MFMA: "mfma", lla.LLA_KERNEL_VALU: "valu"}[kernel_used],
                   "split_u": bool(args.split_u)},
        "tflops": tflops,
        "flops_per_step": flops,
        "flops_nominal": flops_nom,
        "flops_min": flops_min,
        "step_ms_events": {"median": float(np.median(step_ev)), "min": float(step_ev.min())},
        "cg_iters_mean": float(iters_np.mean()),
        "cg_iters_max": int(iters_np.max()),
        "main_kernel_ms": kern_ms,
        "main_kernel": ("conjugate-gradient kernel (phase 2 of 3)" if kernel_used == lla.LLA_KERNEL_MFMA
                        else "fused three-phase kernel"),
        "main_kernel_flops": flops_cg if kernel_used == lla.LLA_KERNEL_MFMA else flops,
        "roofline": {"bound": bound, "achieved": achieved, "peak": peak, "unit": unit,
                     "frac": achieved / peak, "traffic": traffic},
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)
    return 0


if __name__ == "__main__":
    sys.exit(main())
