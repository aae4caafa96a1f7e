"""Pins for the float64 gradient oracle (oracle/lla_oracle_bwd.py): each test
checks it against something other than itself -- central finite differences
of the forward oracle, automatic differentiation of a separately written
PyTorch forward, textbook softmax-attention gradients in the lambda -> inf
limit, and identities that the exact gradient must satisfy -- so that a
dropped term, a wrong sign or a transposed operand fails one of them."""

import numpy as np
import pytest

from oracle import lla_oracle as O
from oracle import lla_oracle_bwd as OB
from local_linear_attention_flashlla_amd.workloads import make_workload


def _inputs(n, d, seed, norm=1.0):
    rng = np.random.default_rng(seed)
    q, k, v, g = (rng.standard_normal((n, d)) for _ in range(4))
    if norm is not None:
        q = q / np.linalg.norm(q, axis=1, keepdims=True) * norm
        k = k / np.linalg.norm(k, axis=1, keepdims=True) * norm
    return q, k, v, g


def _loss(q, k, v, g, lam):
    out = O.oracle_head(q, k, v, lam)
    return float(np.sum(out["b"] * g))


# --- central finite differences of the forward oracle ------------------------

@pytest.mark.parametrize("n,d,lam,seed,norm", [
    (6, 3, 0.3, 0, 1.0), (7, 4, 2.0, 1, 2.0), (5, 2, 0.05, 2, None), (8, 3, 1.0, 3, 4.0)])
def test_gradient_matches_finite_differences(n, d, lam, seed, norm):
    q, k, v, g = _inputs(n, d, seed, norm)
    dq, dk, dv = OB.backward_head(q, k, v, g, lam)
    for name, x, grad in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            h = 1e-5 * max(1.0, abs(x[idx]))
            xp = x.copy(); xp[idx] += h
            xm = x.copy(); xm[idx] -= h
            args = {"q": q, "k": k, "v": v}
            args[name] = xp
            lp = _loss(args["q"], args["k"], args["v"], g, lam)
            args[name] = xm
            lm = _loss(args["q"], args["k"], args["v"], g, lam)
            fd[idx] = (lp - lm) / (2 * h)
        scale = max(1.0, np.abs(fd).max())
        assert np.abs(grad - fd).max() <= 2e-7 * scale, (name, np.abs(grad - fd).max())


# --- automatic differentiation of a separately written forward --------------

def _torch_forward(q, k, v, lam):
    """Eqs. (6)-(8) as plain PyTorch float64 ops, one row at a time, with a
    general linear solve (not the oracle's code path)."""
    import torch
    n, d = q.shape
    c = 1.0 / np.sqrt(d)
    outs = []
    for i in range(n):
        s = c * (k[:i + 1] @ q[i])
        w = torch.exp(s - torch.max(s))
        Z = k[:i + 1] - q[i]
        Sig = Z.T @ (w[:, None] * Z) + lam * torch.eye(d, dtype=q.dtype)
        mu = Z.T @ w
        rho = torch.linalg.solve(Sig, mu)
        a = w * (1.0 - Z @ rho)
        outs.append((a @ v[:i + 1]) / a.sum())
    return torch.stack(outs)


@pytest.mark.parametrize("n,d,lam,seed,norm", [
    (24, 5, 0.5, 10, 2.0), (16, 8, 1e-2, 11, 1.0), (20, 4, 3.0, 12, None)])
def test_gradient_matches_autograd_of_independent_forward(n, d, lam, seed, norm):
    import torch
    q, k, v, g = _inputs(n, d, seed, norm)
    tq, tk, tv = (torch.tensor(a, dtype=torch.float64, requires_grad=True) for a in (q, k, v))
    loss = (_torch_forward(tq, tk, tv, lam) * torch.tensor(g)).sum()
    loss.backward()
    dq, dk, dv = OB.backward_head(q, k, v, g, lam)
    for ours, ref in ((dq, tq.grad), (dk, tk.grad), (dv, tv.grad)):
        ref = ref.numpy()
        assert np.abs(ours - ref).max() <= 1e-9 * max(1.0, np.abs(ref).max())


# --- the lambda -> inf limit: textbook softmax-attention gradients ----------

def test_large_lambda_gives_softmax_attention_gradient():
    n, d = 40, 6
    q, k, v, g = _inputs(n, d, 20, 2.0)
    c = 1.0 / np.sqrt(d)
    S = c * (q @ k.T)
    S = np.where(np.tril(np.ones((n, n), bool)), S, -np.inf)
    P = np.exp(S - S.max(axis=1, keepdims=True))
    P /= P.sum(axis=1, keepdims=True)
    dP = g @ v.T
    dS = P * (dP - np.sum(P * dP, axis=1, keepdims=True))
    ref = (c * dS @ k, c * dS.T @ q, P.T @ g)
    ours = OB.backward_head(q, k, v, g, 1e12)
    for a, b in zip(ours, ref):
        assert np.abs(a - b).max() <= 1e-8 * max(1.0, np.abs(b).max())


# --- identities of the exact gradient -----------------------------------------

@pytest.mark.parametrize("name", ["tiny", "standard"])
def test_scale_identity_and_value_shift(name):
    """Scaling every weight by a common factor is the same as dividing lam by
    it, so sum_j w_j dL/dw_j = -lam dL/dlam; shifting every value by t
    shifts every output by t, so sum_j dv_j = sum_i g_i."""
    wl = make_workload(name, n=48 if name == "standard" else None, B=1, H=1)
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    g = np.random.default_rng(5).standard_normal(q.shape)
    n = q.shape[0]
    for i in (0, 1, n // 2, n - 1):
        r = OB.backward_row(q[i], k[:i + 1], v[:i + 1], g[i], wl.lam)
        lhs = float(r["w"] @ r["dw"])
        assert abs(lhs - (-wl.lam * r["dlam"])) <= 1e-9 * max(1.0, abs(lhs))
    dq, dk, dv = OB.backward_head(q, k, v, g, wl.lam)
    assert np.allclose(dv.sum(axis=0), g.sum(axis=0), rtol=1e-10, atol=1e-10)
    # row 0 sees only its own key: b_0 = v_0 whatever q_0 and k_0 are
    r0 = OB.backward_row(q[0], k[:1], v[:1], g[0], wl.lam)
    assert np.abs(r0["dq"]).max() <= 1e-12 and np.abs(r0["dK"]).max() <= 1e-12
    assert np.allclose(r0["dV"][0], g[0], rtol=0, atol=1e-14)


@pytest.mark.parametrize("name,lam", [("tiny", None), ("standard", None), ("recall", None),
                                      ("standard", 1e-3)])
def test_centred_form_equals_pages_form(name, lam):
    wl = make_workload(name, n=64, B=1, H=1)
    lam = wl.lam if lam is None else lam
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    g = np.random.default_rng(6).standard_normal(q.shape)
    a = OB.backward_head(q, k, v, g, lam, form="pages")
    b = OB.backward_head(q, k, v, g, lam, form="centred")
    for x, y in zip(a, b):
        assert np.abs(x - y).max() <= 1e-8 * max(1.0, np.abs(x).max())
    # and the identity sum_j w_j dL/dw_j = -lam y.rho_c in the centred form
    for i in (3, 40, 63):
        r = OB.backward_row_centred(q[i], k[:i + 1], v[:i + 1], g[i], lam)
        assert abs(float(r["w"] @ r["dw"]) - r["msum"]) <= 1e-8 * max(1.0, abs(r["msum"]))


def test_centred_cg_gradient_converges_to_exact():
    wl = make_workload("standard", n=80, B=1, H=1)
    q, k, v = wl.q[0, 0], wl.k[0, 0], wl.v[0, 0]
    g = np.random.default_rng(7).standard_normal(q.shape)
    d = q.shape[1]
    ex = OB.backward_head(q, k, v, g, wl.lam)
    cg = OB.backward_head(q, k, v, g, wl.lam, form="centred", solver="cg",
                          cg_max_iters=4 * d, cg_rel_tol=1e-14)
    for x, y in zip(ex, cg):
        assert np.abs(x - y).max() <= 1e-7 * max(1.0, np.abs(x).max())
    # a truncated solve is visibly different (the test above is not vacuous)
    tr = OB.backward_head(q, k, v, g, 1e-3, form="centred", solver="cg", cg_max_iters=2)
    ex2 = OB.backward_head(q, k, v, g, 1e-3)
    assert np.abs(tr[0] - ex2[0]).max() > 1e-3 * np.abs(ex2[0]).max()


def test_finite_difference_pin_detects_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the gradient oracle (on the CPU) -- the max
    routed nowhere, a sign flipped in the adjoint, the score scale dropped --
    and check that the finite-difference pin rejects each one."""
    n, d, lam = 6, 3, 0.3
    q, k, v, g = _inputs(n, d, 31, 2.0)

    def fd_grad(x_name):
        base = {"q": q, "k": k, "v": v}
        x = base[x_name]
        fd = np.zeros_like(x)
        for idx in np.ndindex(*x.shape):
            h = 1e-5
            for sgn in (1, -1):
                xp = x.copy(); xp[idx] += sgn * h
                args = dict(base); args[x_name] = xp
                fd[idx] += sgn * _loss(args["q"], args["k"], args["v"], g, lam) / (2 * h)
        return fd

    fd = {name: fd_grad(name) for name in ("q", "k")}

    def pin_ok():
        dq, dk, _ = OB.backward_head(q, k, v, g, lam)
        return all(np.abs(a - fd[nm]).max() <= 2e-7 * max(1.0, np.abs(fd[nm]).max())
                   for a, nm in ((dq, "q"), (dk, "k")))

    assert pin_ok()
    monkeypatch.setattr(OB, "_route_max", lambda sig, js: sig.copy())
    assert not pin_ok(), "dropping the max's gradient went unnoticed"
    monkeypatch.undo()
    good_solve = OB.cholesky_solve
    calls = {"n": 0}

    def flipped(S, r):
        calls["n"] += 1
        x = good_solve(S, r)
        return -x if calls["n"] % 2 == 0 else x   # the adjoint (second) solve of a row
    monkeypatch.setattr(OB, "cholesky_solve", flipped)
    assert not pin_ok(), "a sign error in the adjoint solve went unnoticed"
    monkeypatch.undo()
    monkeypatch.setattr(OB, "_scale", lambda d_, sc: 1.0)
    assert not pin_ok(), "a dropped score scale went unnoticed"
