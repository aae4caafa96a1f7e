"""Shared test helpers: library loading, device upload, and oracle rows.

GPU results are always compared with the float64 oracle on the same seeded
inputs; the oracle never sees a GPU value except the one it is compared with.
"""
from __future__ import annotations

import os
import sys
from concurrent.futures import ProcessPoolExecutor

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

from oracle import lla_oracle as O  # noqa: E402


def ensure_built():
    from local_linear_attention_flashlla_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    return _lib.load()


def to_device(wl, device="cuda"):
    import torch
    if wl.dtype == "f32":
        cast = lambda a: torch.from_numpy(np.ascontiguousarray(a)).to(device)
    else:
        cast = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).to(device).view(torch.bfloat16)
    return cast(wl.q_dev), cast(wl.k_dev), cast(wl.v_dev)


def row_errors(b_gpu, b_ref):
    """Per-row relative error ||b_gpu - b_ref|| / max(||b_ref||, 1e-6 rms)."""
    b_gpu = np.asarray(b_gpu, dtype=np.float64)
    b_ref = np.asarray(b_ref, dtype=np.float64)
    nref = np.linalg.norm(b_ref, axis=-1)
    rms = np.sqrt(np.mean(nref ** 2)) if nref.size else 1.0
    return np.linalg.norm(b_gpu - b_ref, axis=-1) / np.maximum(nref, 1e-6 * rms)


def _oracle_job(args):
    q, k, v, lam, rows, solver, T, tol = args
    out = O.oracle_head(q, k, v, lam, rows=rows, solver=solver, cg_max_iters=T, cg_rel_tol=tol)
    return out


def oracle_rows(wl, heads_rows, solver="cholesky", T=0, tol=0.0, lam=None, workers=None):
    """heads_rows: list of ((b, h), rows). Returns a list of oracle_head dicts."""
    lam = wl.lam if lam is None else lam
    jobs = []
    for (b, h), rows in heads_rows:
        rows = list(rows)
        kmax = max(rows) + 1
        jobs.append((wl.q[b, h, :kmax], wl.k[b, h, :kmax], wl.v[b, h, :kmax], lam, rows,
                     solver, T, tol))
    workers = workers or min(len(jobs), max(1, min(16, len(os.sched_getaffinity(0)))))
    if workers <= 1 or len(jobs) == 1:
        return [_oracle_job(j) for j in jobs]
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_oracle_job, jobs))
