"""GPU parity on inputs of widely varying magnitude (include/lla.h: on the
matrix-core path the keys and the values of a head each take one power-of-two
scale, from the head's largest key row and largest value row, and are then
held in fp16; queries enter as q log2(e) / (sqrt(d) s)).

  * rows whose norms spread over 2^20 inside one head (q, k and v rows each
    scaled by their own 2^u, u ~ U(-20, 0)): the small rows fall into fp16's
    subnormal range after scaling; the numpy model of the kernel's rounding
    (tests/kernel_model.py) puts the worst row at 1.5e-3 of the exact answer;
  * a whole head at 2^-60 (ridge at 2^-120, the same fit), values at 2^100,
    and queries at 2^-30 against keys at 2^30 (ridge at 2^60): bf16 ranges
    far outside fp16's, which the scales must absorb (model: 3.9e-4 to
    8.2e-4);
  * the fp32 vector path on the spread inputs in fp32.

Every row is held to the forward's bar (tests/_support.check_parity: the
bf16 or fp32 tolerance, plus three times the float64 CG iterate's own
distance from the exact answer where 16 steps leave it short).
"""
import numpy as np
import pytest

from tests._support import check_parity, ensure_built, to_device
from local_linear_attention_flashlla_amd.workloads import make_scaled
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
F32_TOL = 1e-3

CASES = {
    "spread-2^20": dict(span_log2=20.0),
    "head-at-2^-60": dict(log2_q=-60, log2_k=-60, log2_v=-60, lam=2.0 ** -120),
    "values-at-2^100": dict(log2_v=100),
    "q-2^-30-k-2^30": dict(log2_q=-30, log2_k=30, lam=2.0 ** 60),
}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def all_rows(wl):
    return [((b, h), range(wl.n)) for b in range(wl.B) for h in range(wl.H)]


def norm_span(x):
    r = np.linalg.norm(x, axis=-1)
    return float(np.log2(r.max() / r.min()))


@pytest.mark.parametrize("case", sorted(CASES))
def test_matrix_core_path_over_magnitudes(torch, case):
    wl = make_scaled(1, 2, 300, 128, "bf16", seed=11, **CASES[case])
    print(f"\n[case] {case} n={wl.n} d={wl.d} lambda={wl.lam:.3g}; log2 row-norm span "
          f"q {norm_span(wl.q):.1f} k {norm_span(wl.k):.1f} v {norm_span(wl.v):.1f}", flush=True)
    q, k, v = to_device(wl)
    out = lla.forward(q, k, v, wl.lam, 16, 0.0, kernel=lla.LLA_KERNEL_MFMA)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    check_parity(wl, got, all_rows(wl), BF16_TOL, T=16, cg_tol=0.0, lam=wl.lam,
                 label=f"{case} matrix cores")


def test_vector_path_over_magnitudes(torch):
    wl = make_scaled(1, 2, 300, 64, "f32", seed=12, span_log2=20.0)
    print(f"\n[case] spread-2^20 fp32 vector path n={wl.n} d={wl.d}", flush=True)
    q, k, v = to_device(wl)
    out = lla.forward(q, k, v, wl.lam, 16, 0.0, kernel=lla.LLA_KERNEL_VALU)
    torch.cuda.synchronize()
    got = out.cpu().numpy().astype(np.float64)
    assert np.isfinite(got).all()
    check_parity(wl, got, all_rows(wl), F32_TOL, T=16, cg_tol=0.0, lam=wl.lam,
                 label="spread-2^20 vector path")
