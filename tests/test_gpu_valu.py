"""GPU parity of the fp32 vector-ALU kernel against the float64 oracle.

Every case prints what names it before it runs, so that a failing run can be
traced from its log alone.
"""
import numpy as np
import pytest

from tests._support import (check_parity, ensure_built, oracle_given_rho, oracle_rows,
                            row_errors, to_device)
from local_linear_attention_flashlla_amd.workloads import make_workload, make_random
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

F32_TOL = 1e-3    # fp32 inputs
BF16_TOL = 2e-2   # bf16 inputs, fp32 accumulation


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def run(torch, wl, kernel=lla.LLA_KERNEL_VALU, T=None, tol=None, lam=None, extras=False):
    print(f"\n[case] {wl.name} B={wl.B} H={wl.H} n={wl.n} d={wl.d} dtype={wl.dtype} "
          f"kernel={kernel} T={T} tol={tol} lam={lam}", flush=True)
    q, k, v = to_device(wl)
    T = wl.cg_max_iters if T is None else T
    tol = wl.cg_rel_tol if tol is None else tol
    lam = wl.lam if lam is None else lam
    res = {}
    kw = {}
    if extras:
        shp = (wl.B, wl.H, wl.n)
        kw = dict(omega=torch.empty(shp, device="cuda"), rowmax=torch.empty(shp, device="cuda"),
                  rho=torch.empty(shp + (wl.d,), device="cuda"),
                  cg_iters=torch.empty(shp, dtype=torch.int32, device="cuda"),
                  cg_resid=torch.empty(shp, device="cuda"))
    out = lla.forward(q, k, v, lam, T, tol, kernel=kernel, **kw)
    torch.cuda.synchronize()
    res["out"] = out.cpu().numpy().astype(np.float64)
    for key, t in kw.items():
        res[key] = t.cpu().numpy()
    return res


def compare(wl, res, tol_rel, heads_rows, T, tol, lam=None, label=""):
    ref = oracle_rows(wl, heads_rows, lam=lam)
    errs = []
    for ((b, h), rows), r in zip(heads_rows, ref):
        errs.append(row_errors(res["out"][b, h, list(rows)], r["b"]))
    e = np.concatenate(errs)
    print(f"[parity] {label} rows={e.size} max={e.max():.3e} p50={np.median(e):.2e} "
          f"p99={np.quantile(e, 0.99):.2e}", flush=True)
    assert e.max() <= tol_rel, f"max row error {e.max():.3e} > {tol_rel}"
    return ref, e


def all_rows(wl):
    return [((b, h), range(wl.n)) for b in range(wl.B) for h in range(wl.H)]


def given_rho_cases(torch, wl, kernel, tol_rel, label):
    """Eq. (8) for supplied rho against the oracle's Eq. (8) with the same rho:
    the exact rho (then also the exact output), rho = 0 (softmax) and a rho
    halfway to zero with noise (any rho; the denominator stays away from 0)."""
    hr = all_rows(wl)
    lam = wl.lam
    ex = oracle_rows(wl, hr, lam=lam)
    shape = (wl.B, wl.H, wl.n, wl.d)
    rho_exact = np.zeros(shape, np.float32)
    for ((b, h), _), x in zip(hr, ex):
        rho_exact[b, h] = x["rho"]
    rng = np.random.default_rng(11)
    noise = rng.standard_normal(shape) * np.abs(rho_exact).mean(axis=-1, keepdims=True)
    cases = {"exact": rho_exact, "zero": np.zeros(shape, np.float32),
             "other": (0.5 * rho_exact + 0.1 * noise).astype(np.float32)}
    q, k, v = to_device(wl)
    for name, rho in cases.items():
        print(f"\n[case] given rho ({name}) {label} kernel={kernel}", flush=True)
        rho_t = torch.from_numpy(rho).cuda()
        rho_o = torch.empty(shape, device="cuda")
        it_o = torch.full(shape[:3], -1, dtype=torch.int32, device="cuda")
        out = lla.forward(q, k, v, lam, 16, 0.0, kernel=kernel, rho_in=rho_t, rho=rho_o,
                          cg_iters=it_o)
        torch.cuda.synchronize()
        got = out.cpu().numpy().astype(np.float64)
        ref = oracle_given_rho(wl, hr, rho.astype(np.float64), lam)
        e = np.concatenate([row_errors(got[b, h], r) for ((b, h), _), r in zip(hr, ref)])
        print(f"[parity] given rho ({name}) {label} rows={e.size} max={e.max():.3e} "
              f"p50={np.median(e):.2e}", flush=True)
        assert e.max() <= tol_rel
        if name == "exact":
            ee = np.concatenate([row_errors(got[b, h], x["b"]) for ((b, h), _), x in zip(hr, ex)])
            assert ee.max() <= tol_rel
        # rho comes back (up to the rounding of a factor 1 / (1 + (q - q).rho)),
        # and no CG step is taken
        np.testing.assert_allclose(rho_o.cpu().numpy(), rho, rtol=1e-6, atol=0)
        assert np.all(it_o.cpu().numpy() == 0)


def test_tiny_all_rows_and_optional_outputs(torch):
    wl = make_workload("tiny")
    res = run(torch, wl, extras=True)
    ref, _ = compare(wl, res, F32_TOL, all_rows(wl), wl.cg_max_iters, wl.cg_rel_tol, label="tiny")
    r = ref[0]
    np.testing.assert_allclose(res["omega"][0, 0], r["omega"], rtol=2e-5)
    np.testing.assert_allclose(res["rowmax"][0, 0], r["m"], rtol=0, atol=2e-5)
    # the pages' rho_i from the centred CG solution
    rho_err = row_errors(res["rho"][0, 0], r["rho"])
    print(f"[rho] max rel {rho_err.max():.2e}", flush=True)
    assert rho_err.max() < 1e-2
    it = res["cg_iters"][0, 0]
    assert it.min() >= 1 and it.max() <= wl.cg_max_iters
    assert np.all(res["cg_resid"][0, 0] >= 0) and np.all(res["cg_resid"][0, 0] < 1e-3)


def test_piecewise_all_rows(torch):
    wl = make_workload("piecewise")
    res = run(torch, wl)
    compare(wl, res, F32_TOL, all_rows(wl), wl.cg_max_iters, wl.cg_rel_tol, label="piecewise")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_no_cg_is_causal_softmax(torch, dtype):
    """cg_max_iters = 0 leaves rho = 0: the output is the local-constant
    (softmax) estimate with the same kernel weights."""
    wl = make_random(2, 2, 150, 64, dtype, seed=5, qk_scale=3.0)
    res = run(torch, wl, T=0, tol=0.0, lam=1.0)
    hr = [((b, h), range(wl.n)) for b in range(2) for h in range(2)]
    ref = oracle_rows(wl, hr, solver="zero", lam=1.0)
    e = np.concatenate([row_errors(res["out"][b, h], r["b"]) for ((b, h), _), r in zip(hr, ref)])
    print(f"[softmax] {dtype} max={e.max():.2e}", flush=True)
    assert e.max() < 1e-5


@pytest.mark.parametrize("d", [16, 32, 64, 128])
@pytest.mark.parametrize("n", [1, 2, 31, 33, 77])
def test_ragged_sizes_f32(torch, n, d):
    wl = make_random(1, 2, n, d, "f32", seed=100 + n + d, qk_scale=1.0)
    res = run(torch, wl, T=2 * d, tol=1e-7, lam=0.5)
    hr = [((0, h), range(n)) for h in range(2)]
    ref = oracle_rows(wl, hr, lam=0.5)
    e = np.concatenate([row_errors(res["out"][0, h], r["b"]) for ((_, h), _), r in zip(hr, ref)])
    print(f"[ragged] n={n} d={d} max={e.max():.2e}", flush=True)
    assert e.max() <= F32_TOL
    # the first row is the first value exactly (a single key fits the line)
    np.testing.assert_allclose(res["out"][0, 0, 0], wl.v[0, 0, 0], rtol=1e-6, atol=1e-6)


# The forward serves 32, 16, 8 or (d <= 64) 4 query rows per workgroup (8, 16,
# 32 or 64 lanes per row: the fewest that give each of the device's compute
# units two workgroups; 256 on this device) and keeps a block's weights in LDS
# when n is short enough (n <= 496, 992, 1984, 3968 for 32, 16, 8, 4 rows).
# One shape per layout and form of the sweeps, against the oracle on sampled
# rows of two heads.
LAYOUTS = [
    (1, 64, 256, 16, "32 rows, weights cached"),
    (2, 8, 512, 32, "16 rows, cached"),
    (1, 4, 2048, 64, "16 rows, recomputed"),
    (1, 2, 1001, 128, "8 rows, cached, ragged tail"),
    (1, 1, 4096, 16, "8 rows, recomputed"),
    (1, 1, 1023, 64, "4 rows, cached, ragged tail"),
    (1, 1, 4000, 32, "4 rows, recomputed"),
]


@pytest.mark.parametrize("B,H,n,d,layout", LAYOUTS, ids=[x[-1] for x in LAYOUTS])
def test_lane_layouts_f32(torch, B, H, n, d, layout):
    wl = make_random(B, H, n, d, "f32", seed=300 + n + d, qk_scale=2.0)
    res = run(torch, wl, T=2 * d, tol=1e-7, lam=0.5)
    rng = np.random.default_rng(n + d)
    rows = sorted(set(range(40)) | set(range(n - 40, n)) | set(rng.integers(0, n, 40).tolist()))
    heads = [(0, 0), (B - 1, H - 1)]
    hr = [(bh, rows) for bh in heads]
    compare(wl, res, F32_TOL, hr, 2 * d, 1e-7, lam=0.5, label=f"valu layout {layout} n={n} d={d}")


@pytest.mark.parametrize("name", ["standard", "long", "recall"])
def test_bf16_recipes_small_valu(torch, name):
    """The bf16 workloads' recipes at a size the oracle checks row by row."""
    wl = make_workload(name, B=1, H=2, n=300)
    res = run(torch, wl)
    check_parity(wl, res["out"], all_rows(wl), BF16_TOL, label=f"valu {name}-300")


def test_large_lambda_is_softmax(torch):
    wl = make_random(1, 1, 200, 32, "f32", seed=9)
    res = run(torch, wl, T=8, tol=0.0, lam=1e8)
    ref = oracle_rows(wl, [((0, 0), range(200))], solver="zero", lam=1.0)
    e = row_errors(res["out"][0, 0], ref[0]["b"])
    assert e.max() < 1e-4


def test_converging_budget_recall(torch):
    wl = make_workload("recall", B=1, H=2, n=300)
    res = run(torch, wl, T=400, tol=1e-7)
    st = check_parity(wl, res["out"], all_rows(wl), BF16_TOL, T=400, cg_tol=1e-7,
                      label="valu recall-300 T=400")
    assert st["truncation_rows"] == 0 and st["max"] <= BF16_TOL


def test_deterministic(torch):
    wl = make_workload("piecewise")
    a = run(torch, wl)["out"]
    b = run(torch, wl)["out"]
    assert np.array_equal(a, b)


def test_output_given_rho_f32(torch):
    wl = make_workload("tiny")
    given_rho_cases(torch, wl, lla.LLA_KERNEL_VALU, F32_TOL, "valu tiny")


def test_output_given_rho_bf16(torch):
    wl = make_random(1, 2, 150, 128, "bf16", seed=13, qk_scale=4.0)
    given_rho_cases(torch, wl, lla.LLA_KERNEL_VALU, BF16_TOL, "valu bf16 d=128")
