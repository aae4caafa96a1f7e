"""GPU parity of the fp16 matrix-core kernel (bf16 inputs) against the
float64 oracle, from ragged toy sizes to the full-size workloads (sampled
rows), in the same launch configuration bench.py times."""
import numpy as np
import pytest

from tests._support import (check_parity, ensure_built, mfma_solver, oracle_given_rho,
                            oracle_rows, row_errors, to_device)
from local_linear_attention_flashlla_amd.workloads import make_workload, make_random
from oracle import lla_oracle as O
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

BF16_TOL = 2e-2
MFMA = lla.LLA_KERNEL_MFMA


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def run(torch, wl, kernel=MFMA, T=None, tol=None, lam=None, extras=False, flags=0):
    print(f"\n[case] {wl.name} B={wl.B} H={wl.H} n={wl.n} d={wl.d} dtype={wl.dtype} "
          f"kernel={kernel} T={T} tol={tol} lam={lam} flags={flags}", flush=True)
    q, k, v = to_device(wl)
    T = wl.cg_max_iters if T is None else T
    tol = wl.cg_rel_tol if tol is None else tol
    lam = wl.lam if lam is None else lam
    kw = {}
    if extras:
        shp = (wl.B, wl.H, wl.n)
        kw = dict(omega=torch.empty(shp, device="cuda"), rowmax=torch.empty(shp, device="cuda"),
                  rho=torch.empty(shp + (wl.d,), device="cuda"),
                  cg_iters=torch.empty(shp, dtype=torch.int32, device="cuda"),
                  cg_resid=torch.empty(shp, device="cuda"))
    out = lla.forward(q, k, v, lam, T, tol, kernel=kernel, flags=flags, **kw)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy().astype(np.float64)}
    for key, t in kw.items():
        res[key] = t.cpu().numpy()
    return res


def all_rows(wl):
    return [((b, h), range(wl.n)) for b in range(wl.B) for h in range(wl.H)]


def given_rho_cases(torch, wl, kernel, tol_rel, label, lam=None):
    """Eq. (8) for supplied rho against the oracle's Eq. (8) with the same rho:
    the exact rho (then also the exact output), rho = 0 (softmax) and a rho
    halfway to zero with noise (any rho; the denominator stays away from 0).
    omega and the row max, which the one-sweep kernel forms against its own
    running reference, against the oracle's."""
    hr = all_rows(wl)
    lam = wl.lam if lam is None else lam
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
        om_o = torch.empty(shape[:3], device="cuda")
        rm_o = torch.empty(shape[:3], device="cuda")
        out = lla.forward(q, k, v, lam, 16, 0.0, kernel=kernel, rho_in=rho_t, rho=rho_o,
                          cg_iters=it_o, omega=om_o, rowmax=rm_o)
        # without omega and the row max (on the matrix cores a variant that
        # tracks neither): the same raises of the reference, the same output
        out_plain = lla.forward(q, k, v, lam, 16, 0.0, kernel=kernel, rho_in=rho_t)
        torch.cuda.synchronize()
        assert torch.equal(out, out_plain)
        for ((b, h), _), x in zip(hr, ex):
            np.testing.assert_allclose(rm_o[b, h].cpu().numpy(), x["m"], rtol=1e-3, atol=1e-3)
            np.testing.assert_allclose(om_o[b, h].cpu().numpy(), x["omega"], rtol=5e-3)
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


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 2, 31, 32, 33, 127, 128, 129, 300])
def test_ragged_sizes(torch, n, d):
    wl = make_random(1, 2, n, d, "bf16", seed=200 + n + d, qk_scale=2.0)
    res = run(torch, wl, T=d, tol=1e-5, lam=1.0)
    check_parity(wl, res["out"], all_rows(wl), BF16_TOL, T=d, cg_tol=1e-5, lam=1.0,
                 label=f"ragged n={n} d={d}", solver=mfma_solver(0, d, 1e-5))
    # one key: the line through it is flat, the output is that value
    np.testing.assert_allclose(res["out"][0, :, 0], wl.v[0, :, 0], rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("d", [64, 128])
def test_no_cg_is_causal_softmax(torch, d):
    wl = make_random(2, 2, 200, d, "bf16", seed=7, qk_scale=4.0)
    res = run(torch, wl, T=0, tol=0.0, lam=1.0)
    hr = all_rows(wl)
    ref = oracle_rows(wl, hr, solver="zero", lam=1.0)
    e = np.concatenate([row_errors(res["out"][b, h], r["b"]) for ((b, h), _), r in zip(hr, ref)])
    print(f"[softmax] d={d} max={e.max():.2e}", flush=True)
    assert e.max() < 2e-3


@pytest.mark.parametrize("d", [64, 128])
def test_rising_scores_move_the_moment_reference(torch, d):
    # Key norms grow 10-20 fold along the sequence, so many rows' max score lies
    # far above the first tile's: the moment phase must raise its reference
    # weight (and rescale its sums) on the way. omega, the row max and the
    # output are checked against the exact oracle.
    wl = make_random(1, 2, 512, d, "bf16", seed=40 + d, qk_scale=8.0, key_ramp={64: 9.0, 128: 19.0}[d])
    lam = 1e3
    s = np.einsum("bhid,bhjd->bhij", wl.q, wl.k) / np.sqrt(d)
    causal = np.tril(np.ones((wl.n, wl.n), dtype=bool))
    s = np.where(causal, s, -np.inf)
    climb = (s.max(-1) - s[..., :32].max(-1)) / np.log(2)
    print(f"[rising] rows whose max lies > 15 binades above the first tile's: "
          f"{np.mean(climb > 15):.2f}", flush=True)
    assert np.mean(climb > 15) > 0.3
    res = run(torch, wl, T=16, tol=0.0, lam=lam, extras=True)
    hr = all_rows(wl)
    ex = oracle_rows(wl, hr, lam=lam)
    for (bh, _), x in zip(hr, ex):
        b, h = bh
        np.testing.assert_allclose(res["rowmax"][b, h], x["m"], rtol=1e-3, atol=1e-3)
        np.testing.assert_allclose(res["omega"][b, h], x["omega"], rtol=5e-3)
    check_parity(wl, res["out"], hr, BF16_TOL, T=16, cg_tol=0.0, lam=lam,
                 label=f"rising scores d={d}")


def test_large_lambda_is_softmax(torch):
    wl = make_random(1, 2, 300, 128, "bf16", seed=8, qk_scale=4.0)
    res = run(torch, wl, T=16, tol=0.0, lam=1e7)
    ref = oracle_rows(wl, all_rows(wl), solver="zero", lam=1.0)
    e = np.concatenate([row_errors(res["out"][0, h], r["b"]) for h, r in zip(range(2), ref)])
    assert e.max() < 2e-3


def test_optional_outputs(torch):
    wl = make_workload("standard", B=1, H=2, n=260)
    res = run(torch, wl, extras=True)
    hr = all_rows(wl)
    cg = oracle_rows(wl, hr, solver="cg_centred", T=wl.cg_max_iters, tol=wl.cg_rel_tol)
    ex = oracle_rows(wl, hr)
    for (bh, _), c, x in zip(hr, cg, ex):
        b, h = bh
        np.testing.assert_allclose(res["omega"][b, h], x["omega"], rtol=2e-3)
        np.testing.assert_allclose(res["rowmax"][b, h], x["m"], rtol=0, atol=1e-4)
        # tol 0 runs the full count except where the residual is exactly zero or
        # the step breaks down (row 0, whose system is lambda I, is one such row)
        it = res["cg_iters"][b, h]
        assert it.max() <= wl.cg_max_iters and np.mean(it[1:] == wl.cg_max_iters) > 0.99
        rho_err = row_errors(res["rho"][b, h], x["rho"])
        print(f"[rho] head {h} max rel {rho_err.max():.2e} p50 {np.median(rho_err):.2e}", flush=True)
        # rho itself is the ill-conditioned quantity; compare loosely with the
        # exact solve, rows where float64 CG is close
        close = row_errors(c["rho"], x["rho"]) < 1e-3
        assert np.median(rho_err[close]) < 5e-2
    assert np.all(res["cg_resid"] >= 0)


# Every workload runs with the library's defaults: the long and recall
# recipes stop early (tolerance 1e-4), so their CG is preconditioned; the
# standard recipe runs exactly 16 plain CG steps.
FLAGS = {"standard": 0, "long": 0, "recall": 0}


@pytest.mark.parametrize("name", ["standard", "long", "recall"])
def test_small_recipes(torch, name):
    wl = make_workload(name, B=1, H=2, n=300)
    a = run(torch, wl, flags=FLAGS[name])
    check_parity(wl, a["out"], all_rows(wl), BF16_TOL, label=f"mfma {name}-300",
                 solver=mfma_solver(FLAGS[name], wl.cg_max_iters, wl.cg_rel_tol))


def test_split_u_on_well_conditioned_workload(torch):
    wl = make_workload("standard", B=1, H=2, n=300)
    a = run(torch, wl, flags=lla.LLA_FLAG_SPLIT_U)
    check_parity(wl, a["out"], all_rows(wl), BF16_TOL, label="mfma split-U standard-300")


@pytest.mark.parametrize("name,T,tol", [("recall", 400, 1e-7), ("standard", 64, 0.0)])
def test_converging_budget_matches_exact_answer(torch, name, T, tol):
    """With a CG budget under which float64 CG reaches the exact answer on every
    row, the kernel must match the exact (Cholesky) oracle on every row: the
    arithmetic is not what limits parity at the configured budgets."""
    wl = make_workload(name, B=1, H=2, n=300)
    res = run(torch, wl, T=T, tol=tol, flags=FLAGS[name])
    st = check_parity(wl, res["out"], all_rows(wl), BF16_TOL, T=T, cg_tol=tol,
                      label=f"mfma {name}-300 T={T}", solver=mfma_solver(FLAGS[name], T, tol))
    assert st["truncation_rows"] == 0 and st["max"] <= BF16_TOL


def test_deterministic(torch):
    wl = make_workload("standard", B=1, H=4, n=700)
    a = run(torch, wl)["out"]
    b = run(torch, wl)["out"]
    assert np.array_equal(a, b)


def test_workspace_argument_and_too_small(torch):
    wl = make_workload("standard", B=1, H=2, n=200)
    q, k, v = to_device(wl)
    need = lla.workspace_bytes(1, 2, 200, 128, "bf16", MFMA)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    out = lla.forward(q, k, v, wl.lam, 16, 0.0, workspace=ws, kernel=MFMA)
    ref = lla.forward(q, k, v, wl.lam, 16, 0.0, kernel=MFMA)
    torch.cuda.synchronize()
    assert torch.equal(out, ref)
    with pytest.raises(lla.LlaError) as ei:
        lla.forward(q, k, v, wl.lam, 16, 0.0, workspace=ws[: need - 256], kernel=MFMA)
    assert ei.value.status == -4


# --- full-size workloads, sampled rows ----------------------------------------

FULL = {"standard": [(0, 0), (1, 3), (3, 7)],
        "long": [(0, 0), (0, 11)],
        "recall": [(0, 0), (5, 9), (7, 15)]}


@pytest.mark.parametrize("name", ["standard", "long", "recall"])
def test_full_size_sampled_rows(torch, name):
    wl = make_workload(name)
    res = run(torch, wl, extras=True, flags=FLAGS[name])
    heads_rows = [((b, h), O.sample_rows(wl.n, seed=17 * b + h)) for b, h in FULL[name]]
    stats = check_parity(wl, res["out"], heads_rows, BF16_TOL, label=f"full {name}",
                         solver=mfma_solver(FLAGS[name], wl.cg_max_iters, wl.cg_rel_tol))
    it = res["cg_iters"]
    print(f"[cg] {name} iterations mean={it.mean():.2f} max={it.max()} "
          f"resid p50={np.median(res['cg_resid']):.2e} max={res['cg_resid'].max():.2e}",
          flush=True)
    assert it.max() <= wl.cg_max_iters
    assert np.isfinite(res["out"]).all()
    assert stats["rows"] > 0


@pytest.mark.parametrize("d", [64, 128])
def test_output_given_rho_with_rising_scores(torch, d):
    # the one-sweep output for a supplied rho starts its score reference at
    # the first tile's max; key norms growing 10-20 fold along the sequence
    # make it raise (and rescale) on most rows
    wl = make_random(1, 2, 512, d, "bf16", seed=40 + d, qk_scale=8.0, key_ramp={64: 9.0, 128: 19.0}[d])
    given_rho_cases(torch, wl, MFMA, BF16_TOL, f"mfma rising scores d={d}", lam=1e3)


@pytest.mark.parametrize("d", [64, 128])
def test_output_given_rho(torch, d):
    if d == 128:
        wl = make_workload("standard", B=1, H=2, n=300)
    else:
        wl = make_random(1, 2, 200, 64, "bf16", seed=12, qk_scale=4.0)
    given_rho_cases(torch, wl, MFMA, BF16_TOL, f"mfma d={d}")
