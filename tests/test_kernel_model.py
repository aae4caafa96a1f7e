"""The numpy model of the kernel's rounding (tests/kernel_model.py) with its
rounding turned off must run the oracle's own float64 recurrences: plain CG
on the centred system and the preconditioned CG with the prefix-Gram
preconditioner. That pins the model, so its rounded runs measure rounding
and nothing else."""
import numpy as np
import pytest

from oracle import lla_oracle as O
from tests import kernel_model as KM
from tests._support import row_errors
from local_linear_attention_flashlla_amd.workloads import make_workload


@pytest.mark.parametrize("name,T,tol,n", [("standard", 16, 0.0, 160), ("recall", 64, 1e-4, 40)])
def test_exact_model_runs_the_oracle_cg(name, T, tol, n):
    # (recall only on its first rows: beyond them plain CG is so ill-conditioned
    # that two float64 implementations differing only in rounding order part
    # ways within 64 steps)
    wl = make_workload(name, B=1, H=1, n=n)
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    rows = list(range(0, n, 7))
    ref = O.oracle_head(q, k, v, wl.lam, rows=rows, solver="cg_centred", cg_max_iters=T, cg_rel_tol=tol)
    m = KM.model_head(q, k, v, wl.lam, T, tol, rows=rows, exact=True)
    assert np.array_equal(m["iters"], ref["cg_iters"])
    assert row_errors(m["b"], ref["b"]).max() < 1e-8


@pytest.mark.parametrize("name,T,tol", [("standard", 16, 0.0), ("recall", 64, 1e-4)])
def test_exact_model_runs_the_oracle_pcg(name, T, tol):
    wl = make_workload(name, B=1, H=1, n=300)
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    rows = list(range(0, 300, 11))
    for i in rows:
        assert KM.group_prefix(i) == O.prefix_group_length(i)
    ref = O.oracle_head(q, k, v, wl.lam, rows=rows, solver="pcg_centred", cg_max_iters=T, cg_rel_tol=tol)

    def exact_M(i):
        P = O.prefix_preconditioner(k[:i + 1], wl.lam)
        return None if P is None else np.linalg.inv(P)
    m = KM.model_head(q, k, v, wl.lam, T, tol, rows=rows, exact=True, precond=exact_M)
    if tol == 0.0:
        assert np.array_equal(m["iters"], ref["cg_iters"])
        assert row_errors(m["b"], ref["b"]).max() < 1e-7
    else:
        # with a tolerance, rounding-order differences may move the step at
        # which a residual crosses it by one; both have then converged
        assert np.abs(m["iters"] - ref["cg_iters"]).max() <= 1
        assert row_errors(m["b"], ref["b"]).max() < 1e-4


@pytest.mark.parametrize("name,T,tol", [("standard", 16, 0.0), ("recall", 64, 1e-4)])
def test_exact_model_of_the_kernels_preconditioning_runs_the_oracle_pcg(name, T, tol):
    """With rounding off, the model's preconditioning as the kernel applies it
    (rows below 256: the group's matrix and the masked rank-r correction by the
    group's own keys; beyond: the group matrix) is the oracle's PCG."""
    wl = make_workload(name, B=1, H=1, n=300)
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    rows = list(range(0, 300, 7))
    ref = O.oracle_head(q, k, v, wl.lam, rows=rows, solver="pcg_centred", cg_max_iters=T, cg_rel_tol=tol)
    m = KM.model_head(q, k, v, wl.lam, T, tol, rows=rows, exact=True, precond=KM.preconditioners(k, wl.lam))
    if tol == 0.0:
        assert np.array_equal(m["iters"], ref["cg_iters"])
        assert row_errors(m["b"], ref["b"]).max() < 1e-7
    else:
        assert np.abs(m["iters"] - ref["cg_iters"]).max() <= 1
        assert row_errors(m["b"], ref["b"]).max() < 1e-4
