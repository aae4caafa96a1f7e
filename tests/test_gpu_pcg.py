"""GPU parity of the preconditioned CG (include/lla.h: prefix-Gram
preconditioner per group of 32 queries, rows below 256 with their whole
prefix through a rank-r correction; the default whenever an early-stopping
tolerance is set) against the float64 oracle.

  * the PCG iterate itself after T = 1, 2, 4 steps against the oracle's
    float64 PCG iterate (tolerance 4e-3: three times the most the numpy model
    of the kernel's rounding, tests/kernel_model.py, gives on the same inputs,
    1.27e-3 over both cases and all three T; the model lands on the GPU's
    figures to three digits, e.g. 2.76e-4 at T = 1 and 1.03e-3 at T = 2 on
    the d = 64 case);
  * the recall recipe (lambda = 1e-3, clustered keys, tol 1e-4, at most 64
    steps) on the default path: every row within 2e-2 of the exact
    (Cholesky) answer, with no allowance for CG truncation, at n = 300 and at
    the full size through lla_forward_bf16; and far fewer steps than plain CG;
  * the two flags that override the default.
"""
import ctypes

import numpy as np
import pytest

from tests._support import (check_parity, ensure_built, oracle_rows, row_errors, to_device)
from local_linear_attention_flashlla_amd.workloads import make_random, make_workload
from oracle import lla_oracle as O
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
MFMA = lla.LLA_KERNEL_MFMA
ITER_TOL = {1: 4e-3, 2: 4e-3, 4: 4e-3}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def all_rows(wl):
    return [((b, h), range(wl.n)) for b in range(wl.B) for h in range(wl.H)]


def buckets(idx, e, d, label):
    """Print the row errors by position: i < d, d <= i < 2d, the rest."""
    for name, sel in (("i<d", idx < d), ("d<=i<2d", (idx >= d) & (idx < 2 * d)), ("i>=2d", idx >= 2 * d)):
        if sel.any():
            print(f"[bucket] {label} {name}: rows={int(sel.sum())} max={e[sel].max():.3e} "
                  f"p50={np.median(e[sel]):.2e}", flush=True)


CASES = {
    "standard-300": lambda: make_workload("standard", B=1, H=2, n=300),
    "random-d64-260": lambda: make_random(1, 2, 260, 64, "bf16", seed=5, qk_scale=2.0),
}


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("case", sorted(CASES))
def test_pcg_iterate_after_T_steps(torch, case, T):
    wl = CASES[case]()
    print(f"\n[case] pcg iterate {case} T={T} flags=PRECOND", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n, wl.d)
    rho_c = torch.empty(shape, device="cuda")
    iters = torch.empty(shape[:3], dtype=torch.int32, device="cuda")
    lla.forward(q, k, v, wl.lam, T, 0.0, rho_c=rho_c, cg_iters=iters, kernel=MFMA,
                flags=lla.LLA_FLAG_PRECOND)
    torch.cuda.synchronize()
    got = rho_c.cpu().numpy().astype(np.float64)
    it = iters.cpu().numpy()
    c = 1.0 / np.sqrt(wl.d)
    worst = 0.0
    for h in range(wl.H):
        qh, kh = wl.q[0, h], wl.k[0, h]
        ref = []
        for i in range(wl.n):
            _, _, w = O.causal_weights(qh[i], kh[:i + 1], c)
            _, _, _, mu, Sc = O.centred_moments(qh[i], kh[:i + 1], w, wl.lam)
            x, _, _ = O.cg_solve(Sc, mu, T, 0.0, precond=O.prefix_preconditioner(kh[:i + 1], wl.lam))
            ref.append(x)
        e = row_errors(got[0, h], np.array(ref))
        worst = max(worst, float(e.max()))
        assert np.all(it[0, h, T:] == T)
    print(f"[iterate] {case} T={T}: max row error of rho_c against the float64 PCG iterate "
          f"{worst:.2e} (bar {ITER_TOL[T]:.1e})", flush=True)
    assert worst <= ITER_TOL[T]


def _recall_rows_within_bar(torch, wl, out, heads_rows, label):
    ex = oracle_rows(wl, heads_rows)
    e, idx = [], []
    for ((b, h), rows), x in zip(heads_rows, ex):
        e.append(row_errors(out[b, h, list(rows)], x["b"]))
        idx.append(np.asarray(list(rows)))
    e, idx = np.concatenate(e), np.concatenate(idx)
    buckets(idx, e, wl.d, label)
    print(f"[parity] {label}: rows={e.size} max={e.max():.3e} p50={np.median(e):.2e} "
          f"p99={np.quantile(e, 0.99):.2e} (bar {BF16_TOL}, no truncation allowance)", flush=True)
    assert e.max() <= BF16_TOL
    return e


def test_recall_default_path_matches_exact_answer(torch):
    wl = make_workload("recall", B=1, H=2, n=300)
    print("\n[case] recall-300 default flags and NO_PRECOND", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n)
    it_pc = torch.empty(shape, dtype=torch.int32, device="cuda")
    it_cg = torch.empty(shape, dtype=torch.int32, device="cuda")
    out = lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, cg_iters=it_pc, kernel=MFMA)
    lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, cg_iters=it_cg, kernel=MFMA,
                flags=lla.LLA_FLAG_NO_PRECOND)
    torch.cuda.synchronize()
    _recall_rows_within_bar(torch, wl, out.cpu().numpy().astype(np.float64), all_rows(wl),
                            "recall-300 default (preconditioned)")
    a, b = it_pc.cpu().numpy(), it_cg.cpu().numpy()
    print(f"[cg] recall-300 steps: preconditioned mean {a.mean():.1f} max {a.max()}; plain mean "
          f"{b.mean():.1f} max {b.max()}", flush=True)
    assert a.mean() < 0.6 * b.mean()


def test_recall_full_size_through_the_plain_entry_point(torch):
    """The whole recall workload (B=8, H=16, n=2048) through lla_forward_bf16
    with its own CG settings and nothing else: sampled rows of three heads
    against the exact answer."""
    wl = make_workload("recall")
    print(f"\n[case] recall full size via lla_forward_bf16 B={wl.B} H={wl.H} n={wl.n}", flush=True)
    lib = ensure_built()
    q, k, v = to_device(wl)
    out = torch.empty((wl.B, wl.H, wl.n, wl.d), dtype=torch.float32, device="cuda")
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    st = lib.lla_forward_bf16(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), wl.B, wl.H,
                              wl.n, wl.d, ctypes.c_float(wl.lam), wl.cg_max_iters,
                              ctypes.c_float(wl.cg_rel_tol), stream)
    assert st == 0, lla._lib.last_error()
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    heads_rows = [((b, h), O.sample_rows(wl.n, seed=17 * b + h, n_first=300))
                  for b, h in [(0, 0), (5, 9), (7, 15)]]
    _recall_rows_within_bar(torch, wl, got, heads_rows, "recall full size, lla_forward_bf16")


def test_precond_flag_on_a_fixed_budget(torch):
    wl = make_workload("standard", B=1, H=2, n=300)
    print("\n[case] standard-300 T=16 tol=0 flags=PRECOND", flush=True)
    q, k, v = to_device(wl)
    out = lla.forward(q, k, v, wl.lam, 16, 0.0, kernel=MFMA, flags=lla.LLA_FLAG_PRECOND)
    torch.cuda.synchronize()
    st = check_parity(wl, out.cpu().numpy().astype(np.float64), all_rows(wl), BF16_TOL, T=16,
                      cg_tol=0.0, label="standard-300 preconditioned, 16 steps", solver="pcg_centred")
    assert st["max"] <= BF16_TOL


def test_no_precond_flag_with_a_tolerance(torch):
    wl = make_workload("long", B=1, H=2, n=300)
    print("\n[case] long-300 tol=1e-4 flags=NO_PRECOND", flush=True)
    q, k, v = to_device(wl)
    out = lla.forward(q, k, v, wl.lam, wl.cg_max_iters, wl.cg_rel_tol, kernel=MFMA,
                      flags=lla.LLA_FLAG_NO_PRECOND)
    torch.cuda.synchronize()
    check_parity(wl, out.cpu().numpy().astype(np.float64), all_rows(wl), BF16_TOL,
                 label="long-300 plain CG", solver="cg_centred")
