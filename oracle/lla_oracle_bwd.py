"""Float64 CPU oracle for the gradient of the causal LLA forward pass.

TEST INFRASTRUCTURE ONLY, like ``lla_oracle``: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it; the HIP library and
its binding never do, and nothing here imports them.

The loss is L = sum_i g_i . b_i for a supplied upstream gradient g = dL/db
(any loss reduces to this form at a point). The pages state that the
backward pass of LLA needs additional linear systems per query ("Local
Linear Attention: reading notes", section 2.2, the remark on training and
appendix D) but print none, so the gradient below is derived here by
implicit differentiation of the pages' own equations ([LLA] section 2.1,
Eqs. (6)-(8)), per query row i, with the row's notation of ``lla_oracle``:

    w_j = exp(s_j - m), s_j = c q.k_j, m = max_l s_l   (j = 0..i)
    z_j = k_j - q, omega = sum w_j, mu = sum w_j z_j,
    Sigma = sum w_j z_j z_j^T + lam I, rho = Sigma^{-1} mu,
    a_j = w_j (1 - z_j.rho), S = sum_j a_j = omega - mu.rho, b = sum a_j v_j / S.

Chain rule, outermost first:

    dL/dv_j = (a_j / S) g
    delta_j = dL/da_j = (g.v_j - g.b) / S
    dL/drho = -xi,  xi = sum_j delta_j w_j z_j
    adjoint solve   Sigma zeta = -xi          (so dL/dmu = zeta,
                                               dL/dSigma = -zeta rho^T)
    dL/dw_j = (1 - z_j.rho)(delta_j + z_j.zeta)
    dL/dz_j = w_j [(1 - z_j.rho) zeta - (delta_j + z_j.zeta) rho]
    dL/ds_j = w_j dL/dw_j - [j = j*] sum_l w_l dL/dw_l

The last line is the max: m = s_{j*} at the maximising key j*, and w depends
on m because lam breaks the scale invariance of the fit (the gradient of a
max is that of the selected entry; ties have measure zero). Then s_j = c q.k_j
and z_j = k_j - q give

    dq   += c sum_j dL/ds_j k_j - sum_j dL/dz_j
    dk_j += c dL/ds_j q + dL/dz_j.

``backward_row`` is this derivation with explicit Cholesky solves (the exact
gradient). ``backward_row_centred`` differentiates the same function written
around the weighted key mean kbar (the form the forward's CG solves, see
``lla_oracle.centred_moments``): b = vbar - C rho_c with C = sum_j (w_j /
omega) v_j (k_j - kbar)^T and Sigma_c rho_c = omega (kbar - q). Its chain
rule, with c_j = k_j - kbar, A_j = 1 - c_j.rho_c, beta_j = g.v_j - g.vbar:

    dL/dv_j = (w_j A_j / omega) g
    h = C^T g,  adjoint solve  Sigma_c y = h
    e_j = beta_j / omega - c_j.y,  tau = h.rho_c / omega - y.(kbar - q)
    dL/dw_j = A_j e_j + tau
    dL/dk_j (besides the score) = -w_j (A_j y + e_j rho_c),  dL/dq (same) = omega y

and the same score and max steps as above. With exact solves both forms give
the same gradient; with CG iterates (``solver="cg"``, the stop rule of
``lla_oracle.cg_solve`` on both the forward and the adjoint system) the
centred form is the float64 counterpart of a truncated-CG backward.
"""

from __future__ import annotations

from typing import Optional

import numpy as np

from .lla_oracle import cg_solve, cholesky_solve, prefix_preconditioner

__all__ = ["backward_row", "backward_row_centred", "backward_head"]


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def _route_max(sig: np.ndarray, jstar: int) -> np.ndarray:
    """dL/ds from sigma_j = w_j dL/dw_j: the max's share goes to key j*."""
    ds = sig.copy()
    ds[jstar] -= np.sum(sig)
    return ds


def backward_row(q_i, K, V, g_i, lam, scale=None, jstar: Optional[int] = None):
    """Gradient of g_i . b_i for one query row against its causal prefix
    (K = k_0..k_i, V = v_0..v_i), in the pages' variables, exact solves.

    Returns a dict with dq (d,), dK (i+1, d), dV (i+1, d) -- the row's
    contributions -- and diagnostics: rho, zeta, dw (dL/dw_j), dlam (dL/dlam)
    and jstar. ``jstar`` overrides the maximising key (default: argmax of the
    float64 scores)."""
    q_i = np.asarray(q_i, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    g_i = np.asarray(g_i, np.float64)
    d = q_i.shape[0]
    c = _scale(d, scale)
    s = c * (K @ q_i)
    js = int(np.argmax(s)) if jstar is None else int(jstar)
    w = np.exp(s - s[js])
    Z = K - q_i[None, :]
    omega = float(np.sum(w))
    mu = Z.T @ w
    Sigma = (Z * w[:, None]).T @ Z + lam * np.eye(d)
    rho = cholesky_solve(Sigma, mu)
    zr = Z @ rho
    a = w * (1.0 - zr)
    S = float(np.sum(a))
    b = (a @ V) / S
    dV = np.outer(a / S, g_i)
    delta = (V @ g_i - g_i @ b) / S
    xi = Z.T @ (delta * w)
    zeta = -cholesky_solve(Sigma, xi)
    zz = Z @ zeta
    dw = (1.0 - zr) * (delta + zz)
    dZ = w[:, None] * ((1.0 - zr)[:, None] * zeta[None, :] - (delta + zz)[:, None] * rho[None, :])
    ds = _route_max(w * dw, js)
    dq = c * (ds @ K) - np.sum(dZ, axis=0)
    dK = c * np.outer(ds, q_i) + dZ
    return {"dq": dq, "dK": dK, "dV": dV, "rho": rho, "zeta": zeta, "dw": dw,
            "w": w, "dlam": float(-zeta @ rho), "jstar": js, "b": b}


def backward_row_centred(q_i, K, V, g_i, lam, scale=None, solver="cholesky",
                         cg_max_iters=0, cg_rel_tol=0.0, jstar: Optional[int] = None):
    """The same gradient through the centred form (module docstring).
    ``solver="cholesky"``: exact solves; ``solver="cg"``: rho_c and y are CG
    iterates under the oracle's stop rule, each system started from zero;
    ``solver="pcg"``: the same with the row's prefix-Gram preconditioner
    (``lla_oracle.prefix_preconditioner``) on both systems.
    Returns the dict of ``backward_row`` (dq, dK, dV, dw, jstar) plus rho_c,
    y, the adjoint iteration count and the identity term -lam y.rho_c."""
    q_i = np.asarray(q_i, np.float64)
    K = np.asarray(K, np.float64)
    V = np.asarray(V, np.float64)
    g_i = np.asarray(g_i, np.float64)
    d = q_i.shape[0]
    c = _scale(d, scale)
    s = c * (K @ q_i)
    js = int(np.argmax(s)) if jstar is None else int(jstar)
    w = np.exp(s - s[js])
    omega = float(np.sum(w))
    kbar = (K.T @ w) / omega
    Cj = K - kbar[None, :]
    u = kbar - q_i
    Sigma_c = (Cj * w[:, None]).T @ Cj + lam * np.eye(d)
    rhs = omega * u
    P = prefix_preconditioner(K, lam) if solver == "pcg" else None
    if solver == "cholesky":
        rho_c = cholesky_solve(Sigma_c, rhs)
    elif solver in ("cg", "pcg"):
        rho_c, _, _ = cg_solve(Sigma_c, rhs, cg_max_iters, cg_rel_tol, precond=P)
    else:
        raise ValueError(solver)
    A = 1.0 - Cj @ rho_c
    gv = V @ g_i
    vbar = (V.T @ w) / omega
    beta = gv - g_i @ vbar
    h = Cj.T @ (w * gv) / omega
    if solver == "cholesky":
        y = cholesky_solve(Sigma_c, h)
        adj_iters = -1
    else:
        y, adj_iters, _ = cg_solve(Sigma_c, h, cg_max_iters, cg_rel_tol, precond=P)
    e = beta / omega - Cj @ y
    tau = (h @ rho_c) / omega - y @ u
    dw = A * e + tau
    dV = np.outer(w * A / omega, g_i)
    dKz = -w[:, None] * (A[:, None] * y[None, :] + e[:, None] * rho_c[None, :])
    ds = _route_max(w * dw, js)
    dq = c * (ds @ K) + omega * y
    dK = c * np.outer(ds, q_i) + dKz
    return {"dq": dq, "dK": dK, "dV": dV, "dw": dw, "w": w, "jstar": js, "rho_c": rho_c,
            "y": y, "adj_iters": adj_iters, "msum": float(-lam * (y @ rho_c))}


def backward_head(q, k, v, g, lam, scale=None, form="pages", solver="cholesky",
                  cg_max_iters=0, cg_rel_tol=0.0, jstar=None, rows=None):
    """dq, dk, dv ([n, d] each) of L = sum_i g_i . b_i for one head, summing
    the rows' contributions (all rows, or only ``rows``: then dk and dv hold
    those rows' share). ``form`` is "pages" (exact) or "centred" (with
    ``solver``); ``jstar`` is an optional [n] array of maximising keys."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g = np.asarray(g, np.float64)
    n, d = q.shape
    dq = np.zeros((n, d))
    dk = np.zeros((n, d))
    dv = np.zeros((n, d))
    rows = range(n) if rows is None else rows
    for i in rows:
        js = None if jstar is None else int(jstar[i])
        if form == "pages":
            r = backward_row(q[i], k[:i + 1], v[:i + 1], g[i], lam, scale, js)
        elif form == "centred":
            r = backward_row_centred(q[i], k[:i + 1], v[:i + 1], g[i], lam, scale, solver,
                                     cg_max_iters, cg_rel_tol, js)
        else:
            raise ValueError(form)
        dq[i] += r["dq"]
        dk[:i + 1] += r["dK"]
        dv[:i + 1] += r["dV"]
    return dq, dk, dv
