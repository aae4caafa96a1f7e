"""GPU parity of the decode path (one query per head against an n-key cache)
with the float64 oracle: the decode output is the last row of the causal
forward whose query sits at position n - 1."""
import numpy as np
import pytest

from tests._support import ensure_built, oracle_rows, row_errors
from local_linear_attention_flashlla_amd.workloads import make_random, make_workload
import local_linear_attention_flashlla_amd as lla

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-3, "bf16": 2e-2}


@pytest.fixture(scope="module")
def torch():
    import torch as _t
    assert _t.cuda.is_available(), "GPU tests need a HIP device"
    ensure_built()
    return _t


def upload(torch, a, dtype):
    a = np.ascontiguousarray(a)
    if dtype == "f32":
        return torch.from_numpy(a).cuda()
    return torch.from_numpy(a.view(np.int16)).cuda().view(torch.bfloat16)


def run_decode(torch, wl, T, tol, lam, extras=True):
    print(f"\n[case] decode {wl.name} B={wl.B} H={wl.H} n={wl.n} d={wl.d} dtype={wl.dtype} "
          f"T={T} tol={tol} lam={lam}", flush=True)
    n = wl.n
    q = upload(torch, wl.q_dev[:, :, n - 1], wl.dtype)
    k = upload(torch, wl.k_dev, wl.dtype)
    v = upload(torch, wl.v_dev, wl.dtype)
    shp = (wl.B, wl.H)
    kw = {}
    if extras:
        kw = dict(omega=torch.empty(shp, device="cuda"), rowmax=torch.empty(shp, device="cuda"),
                  rho=torch.empty(shp + (wl.d,), device="cuda"),
                  cg_iters=torch.empty(shp, dtype=torch.int32, device="cuda"),
                  cg_resid=torch.empty(shp, device="cuda"))
    out = lla.decode(q, k, v, lam, T, tol, **kw)
    torch.cuda.synchronize()
    res = {"out": out.cpu().numpy().astype(np.float64)}
    for key, t in kw.items():
        res[key] = t.cpu().numpy()
    return res


def check(wl, res, T, tol, lam, label):
    hr = [((b, h), [wl.n - 1]) for b in range(wl.B) for h in range(wl.H)]
    ex = oracle_rows(wl, hr, lam=lam)
    cg = oracle_rows(wl, hr, solver="cg_centred", T=T, tol=tol, lam=lam)
    e_gpu, e_cg = [], []
    for ((b, h), _), x, c in zip(hr, ex, cg):
        e_gpu.append(row_errors(res["out"][b, h][None], x["b"])[0])
        e_cg.append(row_errors(c["b"], x["b"])[0])
        np.testing.assert_allclose(res["omega"][b, h], x["omega"][0], rtol=2e-3)
        np.testing.assert_allclose(res["rowmax"][b, h], x["m"][0], rtol=0, atol=2e-3)
        assert 0 <= res["cg_iters"][b, h] <= T
    e_gpu, e_cg = np.array(e_gpu), np.array(e_cg)
    bound = TOL[wl.dtype] + 4.0 * e_cg
    print(f"[parity] decode {label} heads={e_gpu.size} max={e_gpu.max():.3e} "
          f"float64-CG err max {e_cg.max():.2e} worst e_gpu/bound {np.max(e_gpu / bound):.2f}",
          flush=True)
    assert np.all(e_gpu <= bound)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("n", [1, 2, 33, 300, 1000])
def test_decode_sizes(torch, n, d, dtype):
    wl = make_random(2, 3, n, d, dtype, seed=300 + n + d, qk_scale=4.0)
    res = run_decode(torch, wl, T=16, tol=0.0, lam=1.0)
    check(wl, res, 16, 0.0, 1.0, f"n={n} d={d} {dtype}")
    if n == 1:  # one key: the output is its value
        np.testing.assert_allclose(res["out"][:, :, :], wl.v[:, :, 0], rtol=2e-3, atol=2e-3)


@pytest.mark.parametrize("name", ["standard", "recall"])
def test_decode_recipes(torch, name):
    # the last row of the standard and recall recipes (recall: lambda = 1e-3,
    # clustered keys, CG to a tolerance)
    wl = make_workload(name, B=1, H=4, n=2048)
    res = run_decode(torch, wl, T=wl.cg_max_iters, tol=wl.cg_rel_tol, lam=wl.lam)
    check(wl, res, wl.cg_max_iters, wl.cg_rel_tol, wl.lam, name)


def test_decode_no_cg_is_softmax(torch):
    wl = make_random(1, 4, 500, 128, "bf16", seed=5, qk_scale=4.0)
    res = run_decode(torch, wl, T=0, tol=0.0, lam=1.0)
    hr = [((0, h), [wl.n - 1]) for h in range(wl.H)]
    ref = oracle_rows(wl, hr, solver="zero", lam=1.0)
    e = np.array([row_errors(res["out"][0, h][None], r["b"])[0] for h, r in zip(range(wl.H), ref)])
    print(f"[softmax] decode max={e.max():.2e}", flush=True)
    assert e.max() < 2e-3
    assert np.all(res["cg_iters"] == 0)


def test_decode_matches_forward_last_row(torch):
    # the decode call and the blocked forward answer the same question for
    # the last row; both are compared with the oracle above, here with each other
    wl = make_workload("standard", B=1, H=2, n=700)
    res = run_decode(torch, wl, T=16, tol=0.0, lam=1.0, extras=False)
    q, k, v = (upload(torch, a, wl.dtype) for a in (wl.q_dev, wl.k_dev, wl.v_dev))
    full = lla.forward(q, k, v, 1.0, 16, 0.0).cpu().numpy()
    e = row_errors(res["out"][0], full[0, :, -1])
    print(f"[decode vs forward] max={e.max():.2e}", flush=True)
    assert e.max() < 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_decode_scores_rising_along_the_cache(torch, dtype):
    """Keys pushed along the query's direction by a ramp, so that the scores
    rise by about 100 binades along the cache: with bf16 caches the one pass
    takes the first tile's max as its reference, a later tile passes it by far
    more than 2^40 in weight, and the chunk is formed again against its exact
    max. The oracle, as above, decides."""
    from local_linear_attention_flashlla_amd.workloads import (Spec, Workload, bf16_bits_to_f64,
                                                               f64_to_bf16_bits)
    base = make_random(1, 2, 700, 128, dtype, seed=21, qk_scale=4.0)
    n, d = base.n, base.d
    q, k, v = base.q.copy(), base.k.copy(), base.v.copy()
    for h in range(base.H):
        u = q[0, h, n - 1] / np.linalg.norm(q[0, h, n - 1])
        q[0, h, n - 1] = 16.0 * u
        k[0, h] += np.linspace(0.0, 50.0, n)[:, None] * u[None, :]
    if dtype == "f32":
        dev = [x.astype(np.float32) for x in (q, k, v)]
        exact = [x.astype(np.float64) for x in dev]
    else:
        dev = [f64_to_bf16_bits(x) for x in (q, k, v)]
        exact = [bf16_bits_to_f64(x) for x in dev]
    wl = Workload(Spec("rising", 1, base.H, n, d, dtype, 1.0, 16, 0.0), 1, base.H, n, d, *exact, *dev)
    s = exact[1][0, :, :, :] @ exact[0][0, :, n - 1, :, None]
    rise = (s.max() - s[:, :32].max()) * 1.4426950408889634 / np.sqrt(d)
    print(f"\n[case] rising scores: the first tile's max is passed by {rise:.0f} binades", flush=True)
    assert rise > 60
    res = run_decode(torch, wl, T=16, tol=0.0, lam=1.0)
    check(wl, res, 16, 0.0, 1.0, f"rising scores {dtype}")
