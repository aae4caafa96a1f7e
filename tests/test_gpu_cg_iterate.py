"""GPU pin of the conjugate-gradient iterate itself: rho_c after exactly T
steps (tolerance 0) against the float64 CG iterate on the same centred system
("Local Linear Attention: reading notes", section 2.2: matrix-free CG on
Sigma_i rho_i = mu_i, here on the equivalent system centred at the weighted
key mean), and for T = 1 against the closed form of one CG step,
rho = (mu.mu / mu.Sigma mu) mu.

Tolerance. The numpy model of the kernel's rounding (tests/kernel_model.py)
lands within 3.1e-4 (max row relative error) of the float64 iterate on these
inputs for T = 1, 2, 4; that deviation is the fp16 rounding of the CG
direction (2^-12 relative). The bar is 1e-3, about three times the model's.
"""
import numpy as np
import pytest

from tests._support import ensure_built, row_errors, to_device
from local_linear_attention_flashlla_amd.workloads import make_random, make_workload
from oracle import lla_oracle as O
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

ITER_TOL = 1e-3


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def _oracle_iterates(wl, b, h, T):
    """float64 CG iterate after T steps and the one-step closed form, per row."""
    q, k = wl.q[b, h], wl.k[b, h]
    c = 1.0 / np.sqrt(wl.d)
    xs, one = [], []
    for i in range(wl.n):
        _, _, w = O.causal_weights(q[i], k[:i + 1], c)
        _, _, _, mu, Sc = O.centred_moments(q[i], k[:i + 1], w, wl.lam)
        x, _, _ = O.cg_solve(Sc, mu, T, 0.0)
        xs.append(x)
        one.append((mu @ mu) / (mu @ Sc @ mu) * mu)
    return np.array(xs), np.array(one)


CASES = {
    "standard-300": lambda: make_workload("standard", B=1, H=2, n=300),
    "random-d64-260": lambda: make_random(1, 2, 260, 64, "bf16", seed=5, qk_scale=2.0),
}


@pytest.mark.parametrize("T", [1, 2, 4])
@pytest.mark.parametrize("case", sorted(CASES))
def test_cg_iterate_after_T_steps(torch, case, T):
    wl = CASES[case]()
    print(f"\n[case] cg iterate {case} T={T} kernel=mfma", flush=True)
    q, k, v = to_device(wl)
    shape = (wl.B, wl.H, wl.n, wl.d)
    rho_c = torch.empty(shape, device="cuda")
    iters = torch.empty(shape[:3], dtype=torch.int32, device="cuda")
    lla.forward(q, k, v, wl.lam, T, 0.0, rho_c=rho_c, cg_iters=iters, kernel=lla.LLA_KERNEL_MFMA)
    torch.cuda.synchronize()
    got = rho_c.cpu().numpy().astype(np.float64)
    it = iters.cpu().numpy()
    assert it.max() <= T
    worst = 0.0
    for h in range(wl.H):
        x, one = _oracle_iterates(wl, 0, h, T)
        e = row_errors(got[0, h], x)
        worst = max(worst, float(e.max()))
        if T == 1:
            e1 = row_errors(got[0, h], one)
            print(f"[iterate] {case} head {h} T=1 vs closed form: max {e1.max():.2e}", flush=True)
            assert e1.max() <= ITER_TOL
        # tolerance 0 runs all T steps; rows with at most T keys (whose exact
        # arithmetic Krylov space is exhausted sooner) may stop at r = 0
        assert np.all(it[0, h, T:] == T)
    print(f"[iterate] {case} T={T}: max row error of rho_c against the float64 iterate {worst:.2e}",
          flush=True)
    assert worst <= ITER_TOL
