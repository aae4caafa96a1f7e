"""Both kernels on the hand-derived worked example in tests/golden (every
weight exactly 1, exact fractions from the LLA paper's Eqs. (6)-(8)): the
output, omega, the pages' rho and the row max of every row against the
fixture's values, with the head dimension zero-padded to the kernel's size.
The expected values come from the fixture alone."""
import numpy as np
import pytest

from tests._support import ensure_built, load_golden, pad, worked_example_inputs
from local_linear_attention_flashlla_amd.workloads import f64_to_bf16_bits
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


@pytest.mark.parametrize("kernel,dtype,d,tol", [
    (lla.LLA_KERNEL_VALU, "f32", 16, 1e-5),
    (lla.LLA_KERNEL_VALU, "bf16", 32, 1e-5),
    (lla.LLA_KERNEL_MFMA, "bf16", 64, 2e-2),
    (lla.LLA_KERNEL_MFMA, "bf16", 128, 2e-2),
])
def test_worked_example(torch, kernel, dtype, d, tol):
    g = load_golden("equal_scores_worked_example.txt")
    q, k, v = worked_example_inputs(g, d)
    n = q.shape[0]
    print(f"\n[case] worked example kernel={kernel} dtype={dtype} d={d}", flush=True)

    def up(a):
        a = a.reshape(1, 1, n, d)
        if dtype == "f32":
            return torch.from_numpy(a.astype(np.float32)).cuda()
        return torch.from_numpy(f64_to_bf16_bits(a).view(np.int16)).cuda().view(torch.bfloat16)

    shp = (1, 1, n)
    omega, rowmax = torch.empty(shp, device="cuda"), torch.empty(shp, device="cuda")
    rho = torch.empty(shp + (d,), device="cuda")
    out = lla.forward(up(q), up(k), up(v), float(g["lambda"][0]), 16, 0.0, omega=omega, rho=rho,
                      rowmax=rowmax, kernel=kernel)
    torch.cuda.synchronize()
    out, omega, rho, rowmax = (t.cpu().numpy().astype(np.float64)[0, 0] for t in (out, omega, rho, rowmax))
    worst = 0.0
    for i in range(n):
        b_ref, rho_ref = pad(g[f"b{i}"], d), pad(g[f"rho{i}"], d)
        e_b = np.linalg.norm(out[i] - b_ref) / np.linalg.norm(b_ref)
        e_rho = np.linalg.norm(rho[i] - rho_ref) / np.linalg.norm(rho_ref)
        worst = max(worst, e_b, e_rho)
        assert e_b <= tol, f"row {i}: output off by {e_b:.2e}"
        assert e_rho <= tol, f"row {i}: rho off by {e_rho:.2e}"
        assert abs(omega[i] - g[f"omega{i}"][0]) <= 1e-6 * g[f"omega{i}"][0]
        # the matrix-core path scores with the query rounded to fp16 once
        # (scaled to log2 units): relative error up to 2^-11 of the score,
        # the same for every key of a row, so the weights stay exactly 1
        m_ref = g["score"][0] / np.sqrt(d)
        m_tol = 2.0 ** -10 * m_ref if kernel == lla.LLA_KERNEL_MFMA else 1e-6
        assert abs(rowmax[i] - m_ref) <= m_tol, f"row {i}: row max {rowmax[i]} vs {m_ref}"
    print(f"[golden] kernel={kernel} d={d}: worst relative error of b and rho {worst:.2e}", flush=True)
