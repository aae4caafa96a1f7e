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
from oracle import lla_oracle_bwd as OB  # noqa: E402


GOLDEN = os.path.join(ROOT, "tests", "golden")


def load_golden(name):
    """Parse a fixture under tests/golden: 'key: v1 v2 ...' lines of integers
    or fractions p/q, '#' comments. Returns {key: float64 array}."""
    from fractions import Fraction
    out = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                key, vals = line.split(":", 1)
                out[key.strip()] = np.array([float(Fraction(x)) for x in vals.split()])
    return out


def pad(x, d):
    """x zero-padded to length d."""
    y = np.zeros(d)
    y[:len(x)] = x
    return y


def worked_example_inputs(g, d):
    """q, k, v ([n, d] float64, zero-padded) of the equal-scores worked example."""
    n = sum(1 for key in g if key.startswith("k"))
    q = np.stack([pad(g["q"], d)] * n)
    k = np.stack([pad(g[f"k{j}"], d) for j in range(n)])
    v = np.stack([pad(g[f"v{j}"], d) for j in range(n)])
    return q, k, v


def ensure_built():
    """The library, checked to be built from the sources in this tree. Without
    a GPU (the host build check) a missing or stale library is rebuilt; on a
    GPU machine a stale one is an error, so tests never pass on old code."""
    from local_linear_attention_flashlla_amd import _lib, build
    if not os.path.exists(_lib.LIB_PATH):
        build.build()
    lib = _lib.load()
    if not _lib.is_current(lib):
        import torch
        if torch.cuda.is_available():
            raise RuntimeError(f"{_lib.LIB_PATH} was built from other sources than this tree's: "
                               "rebuild it (python -m local_linear_attention_flashlla_amd.build)")
        build.build()
        lib = _lib.load(_lib.LIB_PATH)
        _lib._lib = lib
        assert _lib.is_current(lib)
    return lib


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


def oracle_given_rho(wl, heads_rows, rho, lam=None):
    """Eq. (8) rows for a supplied rho (float64 copy of what the GPU read):
    rho is [B, H, n, d]; returns a list of [len(rows), d] arrays."""
    lam = wl.lam if lam is None else lam
    res = []
    for (b, h), rows in heads_rows:
        out = []
        for i in rows:
            q_i, K, V = wl.q[b, h, i], wl.k[b, h, :i + 1], wl.v[b, h, :i + 1]
            _, _, w = O.causal_weights(q_i, K, 1.0 / np.sqrt(wl.d))
            Z, omega, mu, _ = O.pairwise_moments(q_i, K, w, lam)
            bi, _, _ = O.intercept_from_rho(w, Z, V, omega, mu, np.asarray(rho[b, h, i], np.float64))
            out.append(bi)
        res.append(np.array(out))
    return res


def mfma_solver(flags, T, tol):
    """The oracle's float64 counterpart of the matrix-core CG under the rule of
    include/lla.h: preconditioned with LLA_FLAG_PRECOND, plain with
    LLA_FLAG_NO_PRECOND, otherwise preconditioned iff cg_rel_tol > 0."""
    from local_linear_attention_flashlla_amd import _lib
    if T > 0 and ((flags & _lib.LLA_FLAG_PRECOND) or
                  (not flags & _lib.LLA_FLAG_NO_PRECOND and tol > 0)):
        return "pcg_centred"
    return "cg_centred"


def check_parity(wl, out, heads_rows, tol, T=None, cg_tol=None, lam=None, label="",
                 factor=3.0, solver="cg_centred"):
    """Compare GPU rows with the float64 oracle.

    e_gpu = row error of the GPU output against the exact (Cholesky) oracle;
    e_cg  = row error of the oracle's own float64 CG run (same system, same
            iteration cap and stop rule) against the same exact answer.
    Every row must satisfy e_gpu <= tol + factor * e_cg. Where the configured
    CG budget reaches the exact answer in float64 (e_cg ~ 0) this is the plain
    tolerance. Where it does not (the CG budget, not the arithmetic, limits
    those rows: no arithmetic can match the exact answer there), the GPU must
    stay as close as an unconverged CG iterate of another precision does. The
    numpy model of the kernel's rounding (tests/kernel_model.py) lands within
    1.33 times the float64 iterate's error on every truncated row of the
    standard recipe's fixed 16 steps (n = 300, and sampled rows at full size);
    the factor 3 is over twice that.
    Returns a dict of statistics (also printed)."""
    T = wl.cg_max_iters if T is None else T
    cg_tol = wl.cg_rel_tol if cg_tol is None else cg_tol
    exact = oracle_rows(wl, heads_rows, lam=lam)
    cg = oracle_rows(wl, heads_rows, solver=solver, T=T, tol=cg_tol, lam=lam)
    e_gpu, e_cg, idx = [], [], []
    for ((b, h), rows), ex, c in zip(heads_rows, exact, cg):
        rows = list(rows)
        e_gpu.append(row_errors(out[b, h, rows], ex["b"]))
        e_cg.append(row_errors(c["b"], ex["b"]))
        idx.append(np.asarray(rows))
    e_gpu = np.concatenate(e_gpu)
    e_cg = np.concatenate(e_cg)
    idx = np.concatenate(idx)
    # errors by position: prefixes shorter than d (the fit nearly interpolates),
    # between d and 2d, and longer
    for name, sel in (("i<d", idx < wl.d), ("d<=i<2d", (idx >= wl.d) & (idx < 2 * wl.d)),
                      ("i>=2d", idx >= 2 * wl.d)):
        if sel.any():
            print(f"[bucket] {label} {name}: rows={int(sel.sum())} gpu max={e_gpu[sel].max():.3e} "
                  f"p50={np.median(e_gpu[sel]):.2e} | float64-CG max={e_cg[sel].max():.3e} | "
                  f"gpu - float64-CG max={np.max(e_gpu[sel] - e_cg[sel]):.3e}", flush=True)
    bound = tol + factor * e_cg
    conv = e_cg <= 1e-3          # rows where float64 CG clearly reached the answer
    trunc = e_cg > tol / 2       # rows the CG budget leaves far from it
    stats = {
        "rows": int(e_gpu.size), "max": float(e_gpu.max()), "p50": float(np.median(e_gpu)),
        "p99": float(np.quantile(e_gpu, 0.99)),
        "strict_frac": float((e_gpu <= tol).mean()),
        "converged_rows": int(conv.sum()),
        "converged_max": float(e_gpu[conv].max()) if conv.any() else 0.0,
        "truncation_rows": int(trunc.sum()),
        "cg64_max": float(e_cg.max()),
        "worst_ratio": float((e_gpu / bound).max()),
    }
    print(f"[parity] {label} rows={stats['rows']} max={stats['max']:.3e} p50={stats['p50']:.2e} "
          f"p99={stats['p99']:.2e} within {tol}: {stats['strict_frac'] * 100:.2f}% | rows with "
          f"float64-CG err <= 1e-3: {stats['converged_rows']}, max {stats['converged_max']:.3e} | "
          f"float64-CG err max {stats['cg64_max']:.2e}, rows > tol/2: {stats['truncation_rows']} | "
          f"worst e_gpu/(tol+{factor}e_cg) {stats['worst_ratio']:.2f}", flush=True)
    assert stats["worst_ratio"] <= 1.0, (
        f"{label}: {int((e_gpu > bound).sum())} rows exceed tol + {factor} x float64-CG error "
        f"(worst ratio {stats['worst_ratio']:.2f})")
    assert stats["converged_max"] <= tol, f"{label}: a converged row exceeds {tol}"
    return stats


def _grad_job(args):
    q, k, v, g, lam, rows, form, solver, T, tol, jst = args
    return OB.backward_head(q, k, v, g, lam, form=form, solver=solver, cg_max_iters=T,
                            cg_rel_tol=tol, rows=rows, jstar=jst)


def oracle_grads(wl, g, heads_rows, form="pages", solver="cholesky", T=0, tol=0.0, lam=None,
                 jstar=None):
    """Float64 gradients (dq, dk, dv) of sum(g * out) per head: heads_rows is a
    list of ((b, h), rows); with rows a subset, dk and dv hold those rows'
    share only (complete for keys at or after the first listed row when the
    rows run to the end of the head). ``jstar``: optional {(b, h): [n] array}
    of maximising keys. Runs heads in a process pool."""
    lam = wl.lam if lam is None else lam
    jobs = []
    for (b, h), rows in heads_rows:
        rows = list(rows)
        m = max(rows) + 1
        jst = None if jstar is None else np.asarray(jstar[(b, h)])[:m]
        jobs.append((wl.q[b, h, :m], wl.k[b, h, :m], wl.v[b, h, :m], np.asarray(g[b, h, :m], np.float64),
                     lam, rows, form, solver, T, tol, jst))
    workers = min(len(jobs), max(1, min(16, len(os.sched_getaffinity(0)))))
    if workers <= 1:
        return [_grad_job(j) for j in jobs]
    with ProcessPoolExecutor(max_workers=workers) as ex:
        return list(ex.map(_grad_job, jobs))
