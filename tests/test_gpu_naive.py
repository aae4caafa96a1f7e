"""GPU parity of the naive forward (lla_forward_naive: pairwise differences
and moment matrices materialised, exact Cholesky solves, fp32) against the
float64 oracle's exact answer, on every row: there is no CG here, so no
truncation allowance either. Bars: 1e-3 for fp32 inputs and 2e-2 for bf16
inputs, the forward's own. Also the optional outputs (omega, the pages' rho,
the row max) and the zeroed CG counters."""
import numpy as np
import pytest

from tests._support import ensure_built, oracle_rows, row_errors, to_device
from local_linear_attention_flashlla_amd.workloads import make_random, make_workload
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}

CASES = {
    "tiny": lambda: make_workload("tiny"),
    "piecewise-400": lambda: make_workload("piecewise", n=400),
    "standard-300": lambda: make_workload("standard", B=1, H=2, n=300),
    "recall-300": lambda: make_workload("recall", B=1, H=2, n=300),
    "random-d32-ragged": lambda: make_random(2, 1, 77, 32, "f32", seed=4),
}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def all_rows(wl):
    return [((b, h), range(wl.n)) for b in range(wl.B) for h in range(wl.H)]


@pytest.mark.parametrize("case", sorted(CASES))
def test_naive_forward_matches_the_exact_answer(torch, case):
    wl = CASES[case]()
    print(f"\n[case] naive {case} B={wl.B} H={wl.H} n={wl.n} d={wl.d} dtype={wl.dtype} "
          f"lambda={wl.lam:g}", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n)
    omega = torch.empty(shape, device="cuda")
    rowmax = torch.empty(shape, device="cuda")
    rho = torch.empty(shape + (wl.d,), device="cuda")
    iters = torch.full(shape, 7, dtype=torch.int32, device="cuda")
    out = lla.forward(q, k, v, wl.lam, 5, 0.5, omega=omega, rowmax=rowmax, rho=rho,
                      cg_iters=iters, naive=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    ex = oracle_rows(wl, all_rows(wl))
    e, e_om, e_rm, e_rho = [], [], [], []
    for ((b, h), _), x in zip(all_rows(wl), ex):
        e.append(row_errors(got[b, h], x["b"]))
        e_om.append(np.abs(omega[b, h].cpu().numpy() - x["omega"]) / x["omega"])
        e_rm.append(np.abs(rowmax[b, h].cpu().numpy() - x["m"]))
        e_rho.append(row_errors(rho[b, h].cpu().numpy(), x["rho"]))
    e, e_om, e_rm, e_rho = (np.concatenate(t) for t in (e, e_om, e_rm, e_rho))
    tol = TOL[wl.dtype]
    print(f"[parity] naive {case}: rows={e.size} max={e.max():.3e} p50={np.median(e):.2e} "
          f"(bar {tol}); omega rel max {e_om.max():.1e}; rowmax abs max {e_rm.max():.1e}; "
          f"rho row max {e_rho.max():.1e}", flush=True)
    assert e.max() <= tol
    assert e_om.max() <= 1e-4 and e_rm.max() <= 1e-4
    assert np.all(iters.cpu().numpy() == 0)
    if wl.dtype == "f32":
        assert e_rho.max() <= 1e-3


def test_naive_forward_on_sampled_rows_of_a_longer_sequence(torch):
    """The headline shape's head layout (d = 128, bf16) at n = 1024, where
    the workspace holds 512 MiB of pairwise differences per head: every 7th
    row of two heads against the oracle."""
    wl = make_workload("standard", B=1, H=2, n=1024)
    print(f"\n[case] naive standard-1024 H={wl.H}", flush=True)
    q, k, v = to_device(wl)
    out = lla.forward(q, k, v, wl.lam, 0, 0.0, naive=True)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    rows = list(range(0, 1024, 7))
    ex = oracle_rows(wl, [((0, h), rows) for h in range(wl.H)])
    e = np.concatenate([row_errors(got[0, h, rows], x["b"]) for h, x in enumerate(ex)])
    print(f"[parity] naive standard-1024 sampled rows={e.size} max={e.max():.3e}", flush=True)
    assert e.max() <= TOL["bf16"]
