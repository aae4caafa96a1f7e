"""Float64 CPU oracle for the causal Local Linear Attention (LLA) forward pass.

TEST INFRASTRUCTURE ONLY. This module is the slow, obviously correct
reference that the GPU library is checked against. Only the test suite, the
smoke check and the benchmark's CPU-baseline leg may import it. The product
path (the HIP library and its Python binding) never imports, links or calls
anything here, and nothing here imports the product path.

Sources (the pages):
  [LLA] "Local Linear Attention: reading notes" on arXiv:2510.01450v1
        (Zuo et al., ICLR 2026): section 2.1 "per-query intercept",
        Eqs. (6)-(8) and Eq. (9); section 2.2 "memory primitives and
        blocked execution", Eqs. (10)-(12), Algorithm 1.
  [PLX] "Parallax: Parameterized Local Linear Attention for Language
        Modeling" (summary page): the covariance rewrite of LLA.
  [KM]  "Linear attention seen as kernel methods" (blog), chapter 1: scaled
        dot-product attention as Nadaraya-Watson regression, scale 1/sqrt(d).

What is computed, per head and per query row i (j runs over 0..i, causal,
diagonal included):
  s_ij  = c * q_i . k_j,  c = 1/sqrt(d)                         [KM ch. 1]
  m_i   = max_{j<=i} s_ij;  w_ij = exp(s_ij - m_i)  (largest weight is 1)
  z_ij  = k_j - q_i                                              [LLA 2.1]
  omega_i = sum_j w_ij;  mu_i = sum_j w_ij z_ij
  Sigma_i = sum_j w_ij z_ij z_ij^T + lam I;  rho_i = Sigma_i^{-1} mu_i
                                                    [LLA 2.1, Eqs. (6)-(7)]
  s_ij  = w_ij (1 - z_ij^T rho_i) / (omega_i - mu_i^T rho_i)
  b_i   = sum_j s_ij v_j                            [LLA 2.1, Eq. (8)]

Readings taken where the pages leave a step open:
  * weights are max-normalised over the causal prefix (the online row max of
    Algorithm 1 in [LLA] 2.2); lambda is not scale invariant, so this fixes
    the problem being solved;
  * the ridge penalty is the one that makes Sigma_i carry exactly lam I, i.e.
    the objective sum_j w_ij ||v_j - b - W z_ij||^2 + lam ||W||_F^2 (the
    printed objective carries a 1/2 on the data term only; Sigma_i as printed
    governs, because the whole algorithm is built on it);
  * rho_i is the exact solution (explicit Cholesky), not a CG iterate;
    ``cg_solve`` gives the CG iterate under the stop rule below separately,
    on the pages' system or on the same system expanded around the weighted
    key mean (``centred_moments``), which has the same exact solution.
  * CG ([LLA] 2.2: matrix-free CG on Sigma_i rho_i = mu_i; the stop rule is
    not printed): x0 = 0, r0 = p0 = mu_i; a query stops at the first k with
    ||r_k|| <= tol * ||r_0|| (recurrence residual), on breakdown
    (p^T Sigma p <= 0 or r = 0), or at k = max_iters. tol = 0 runs exactly
    max_iters steps unless the residual is exactly zero.
  * Preconditioned CG (not on the pages, which only mention early stopping;
    used where the iteration budget cannot otherwise reach the answer): the
    same recurrence with z = P^{-1} r in place of r in the direction update.
    P is the prefix-Gram preconditioner (``prefix_group_length``,
    ``prefix_preconditioner``): a unit-weight scatter matrix plus lam I. For
    rows i < 256 it scatters the row's whole prefix about a point shared by
    its group of 32 queries; from row 256 on, the first N keys of the
    prefix about their mean, N <= 32 floor(i/32) shared by groups of rows.
"""

from __future__ import annotations

import dataclasses
from typing import Iterable, Optional, Sequence

import numpy as np
from scipy.linalg import solve_triangular

__all__ = [
    "RowResult",
    "causal_weights",
    "pairwise_moments",
    "cholesky_solve",
    "cg_solve",
    "intercept_from_rho",
    "centred_moments",
    "centred_intercept",
    "oracle_row",
    "oracle_head",
    "ridge_bruteforce",
    "eq9_intercept",
    "covariance_form_intercept",
    "tilde_moments",
    "prefix_group_length",
    "prefix_preconditioner",
]


@dataclasses.dataclass
class RowResult:
    b: np.ndarray          # (d,) output b_i
    omega: float           # omega_i
    mu: np.ndarray         # (d,) mu_i
    rho: np.ndarray        # (d,) rho_i used for b_i
    m: float               # row max of the scaled scores
    schur: float           # omega_i - mu_i^T rho_i
    s: np.ndarray          # (i+1,) output weights s_ij
    w: np.ndarray          # (i+1,) kernel weights w_ij
    Sigma: np.ndarray      # (d, d) Sigma_i
    cg_iters: int = -1     # CG steps taken (-1: exact solve)
    cg_resid: float = 0.0  # ||r_k|| / ||r_0|| at exit (0: exact solve)


def _scale(d: int, scale: Optional[float]) -> float:
    return 1.0 / np.sqrt(d) if scale is None else float(scale)


def causal_weights(q_i: np.ndarray, K_prefix: np.ndarray, scale: float):
    """Scaled scores, their max over the prefix, and max-normalised weights
    w_ij = exp(s_ij - m_i) over the causal prefix K_prefix = k_0..k_i.
    [KM ch. 1 for the score; LLA 2.2 Algorithm 1 for the running max]"""
    s = scale * (K_prefix @ q_i)
    m = float(np.max(s))
    w = np.exp(s - m)
    return s, m, w


def pairwise_moments(q_i, K_prefix, w, lam):
    """The naive moments with the explicit pairwise differences z_ij = k_j - q_i
    ([LLA] 2.1, Eqs. (6)-(7); the naive implementation of [LLA] 2.2).
    Returns Z, omega, mu, Sigma."""
    Z = K_prefix - q_i[None, :]
    omega = float(np.sum(w))
    mu = Z.T @ w
    Sigma = (Z * w[:, None]).T @ Z + lam * np.eye(Z.shape[1])
    return Z, omega, mu, Sigma


def cholesky_solve(Sigma: np.ndarray, rhs: np.ndarray) -> np.ndarray:
    """rho = Sigma^{-1} rhs through an explicit Cholesky factor Sigma = L L^T."""
    L = np.linalg.cholesky(Sigma)
    y = solve_triangular(L, rhs, lower=True)
    return solve_triangular(L.T, y, lower=False)


def prefix_group_length(i: int) -> int:
    """Number N of leading keys whose scatter matrix preconditions row i.

    Rows are grouped in 32s, group g = floor(i / 32). Group 0 gets no
    preconditioner (N = 0). Groups 1..7 use N = 32 g, the keys every query of
    the group sees. From group 8 on, N is 32 g rounded down to a multiple of
    32 * 2^(floor(log2 g) - 2): four prefix lengths per doubling of g, each
    shared by the groups up to the next, so a head needs only a few
    preconditioners. Always N <= 32 g <= i."""
    g = int(i) // 32
    if g == 0:
        return 0
    if g < 8:
        return 32 * g
    step = 1 << (g.bit_length() - 3)
    return 32 * (g // step) * step


def prefix_preconditioner(K_prefix: np.ndarray, lam: float):
    """P for the last row of K_prefix (row i = len(K_prefix) - 1), with
    g = floor(i / 32) and N = prefix_group_length(i):

      g < 8:  P = sum_{j<=i} (k_j - m)(k_j - m)^T + lam I, the whole prefix
              scattered about m = k_0 (g = 0) or the plain mean of
              k_0..k_{N-1} (g >= 1). Below 256 keys a prefix spans a part of
              the key space that its first N keys can miss (up to 31
              directions, each a near-zero eigenvalue of the system at a small
              lam), so the row's own keys are kept; the point m is shared by
              the group, so the rows of a group differ by a rank-r update
              (r <= 32) of one matrix;
      g >= 8: P = sum_{j<N} (k_j - m)(k_j - m)^T + lam I with m the mean of
              those N keys (the prefix is long enough that its first N keys
              span what the rest does).

    Every key used is visible to row i."""
    i = K_prefix.shape[0] - 1
    g = i // 32
    N = prefix_group_length(i)
    if g < 8:
        K = np.asarray(K_prefix, dtype=np.float64)
        m = K[0] if g == 0 else K[:N].mean(axis=0)
    else:
        K = np.asarray(K_prefix[:N], dtype=np.float64)
        m = K.mean(axis=0)
    D = K - m[None, :]
    return D.T @ D + lam * np.eye(K.shape[1])


def cg_solve(Sigma: np.ndarray, rhs: np.ndarray, max_iters: int, rel_tol: float, precond=None):
    """Conjugate gradient on Sigma x = rhs with the stop rule in the module
    docstring ([LLA] 2.2: matrix-free CG; only products Sigma p are used).
    ``precond``: None, or an SPD matrix P; then the preconditioned recurrence
    (z = P^{-1} r, applied by a Cholesky solve, and r^T z in place of r^T r).
    Returns (x, iterations, ||r|| / ||r_0||)."""
    def apply(r):
        return r.copy() if precond is None else cholesky_solve(precond, r)
    x = np.zeros_like(rhs)
    r = rhs.astype(np.float64).copy()
    rr = float(r @ r)
    r0 = np.sqrt(rr)
    if r0 == 0.0:
        return x, 0, 0.0
    z = apply(r)
    rz = float(r @ z)
    p = z.copy()
    it = 0
    for _ in range(max_iters):
        Sp = Sigma @ p
        pSp = float(p @ Sp)
        if not pSp > 0.0:
            break
        alpha = rz / pSp
        x = x + alpha * p
        r = r - alpha * Sp
        rr = float(r @ r)
        it += 1
        if np.sqrt(rr) <= rel_tol * r0 or rr == 0.0:
            break
        z = apply(r)
        rz_new = float(r @ z)
        p = z + (rz_new / rz) * p
        rz = rz_new
    return x, it, float(np.sqrt(rr) / r0)


def intercept_from_rho(w, Z, V_prefix, omega, mu, rho):
    """b_i and s_ij for a given rho ([LLA] 2.1, Eq. (8)). The denominator is
    the Schur complement omega_i - mu_i^T rho_i."""
    schur = float(omega - mu @ rho)
    s = w * (1.0 - Z @ rho) / schur
    return s @ V_prefix, s, schur


def centred_moments(q_i, K_prefix, w, lam):
    """The same local fit expanded around the weighted key mean
    kbar_i = sum_j w_ij k_j / omega_i instead of q_i, with explicit pairwise
    differences k_j - kbar_i:
        Sigma_c = sum_j w_ij (k_j - kbar_i)(k_j - kbar_i)^T + lam I.
    By the parallel-axis identity Sigma_i = Sigma_c + omega_i u u^T with
    u = kbar_i - q_i, and mu_i = omega_i u ([LLA] 2.1, Eqs. (6)-(7) rewritten).
    Returns Zc, omega, kbar, mu, Sigma_c."""
    omega = float(np.sum(w))
    kbar = (K_prefix.T @ w) / omega
    Zc = K_prefix - kbar[None, :]
    mu = omega * (kbar - q_i)
    Sigma_c = (Zc * w[:, None]).T @ Zc + lam * np.eye(K_prefix.shape[1])
    return Zc, omega, kbar, mu, Sigma_c


def centred_intercept(w, Zc, V_prefix, rho_c):
    """Output for a solution rho_c of Sigma_c rho_c = mu_i: with
    a_ij = w_ij (1 - (k_j - kbar_i)^T rho_c), b_i = sum_j a_ij v_j / sum_j a_ij.
    For the exact rho_c this is [LLA] Eq. (8) exactly (Sherman-Morrison on the
    rank-one term above; sum_j a_ij = omega_i because sum_j w_ij (k_j - kbar_i)
    = 0); the pages' rho_i = rho_c / (1 + (kbar_i - q_i)^T rho_c)."""
    a = w * (1.0 - Zc @ rho_c)
    den = float(np.sum(a))
    return (a @ V_prefix) / den, a / den, den


def oracle_row(q_i, K_prefix, V_prefix, lam, scale=None, solver="cholesky",
               cg_max_iters=0, cg_rel_tol=0.0) -> RowResult:
    """One row of causal LLA in float64.

    ``solver="cholesky"``: exact rho_i (the definition).
    ``solver="cg"``: rho_i is the CG iterate of ``cg_solve`` on the pages'
    system Sigma_i rho_i = mu_i; the output is then Eq. (8) with that rho_i.
    ``solver="cg_centred"``: CG (same stop rule) on Sigma_c rho_c = mu_i, the
    system centred at the weighted key mean (``centred_moments``); output by
    ``centred_intercept``; ``rho`` is reported as the pages' rho_i.
    ``solver="pcg_centred"``: the same with the prefix-Gram preconditioner of
    the row's group (``prefix_preconditioner``).
    ``solver="zero"``: rho_i = 0, the local-constant (softmax) limit."""
    q_i = np.asarray(q_i, dtype=np.float64)
    K_prefix = np.asarray(K_prefix, dtype=np.float64)
    V_prefix = np.asarray(V_prefix, dtype=np.float64)
    c = _scale(q_i.shape[0], scale)
    _, m, w = causal_weights(q_i, K_prefix, c)
    if solver in ("cg_centred", "pcg_centred"):
        Zc, omega, kbar, mu, Sigma_c = centred_moments(q_i, K_prefix, w, lam)
        P = prefix_preconditioner(K_prefix, lam) if solver == "pcg_centred" else None
        rho_c, iters, resid = cg_solve(Sigma_c, mu, cg_max_iters, cg_rel_tol, precond=P)
        b, s, _ = centred_intercept(w, Zc, V_prefix, rho_c)
        rho = rho_c / (1.0 + (kbar - q_i) @ rho_c)
        schur = float(omega - mu @ rho)
        return RowResult(b, omega, mu, rho, m, schur, s, w, Sigma_c, iters, resid)
    Z, omega, mu, Sigma = pairwise_moments(q_i, K_prefix, w, lam)
    iters, resid = -1, 0.0
    if solver == "cholesky":
        rho = cholesky_solve(Sigma, mu)
    elif solver == "cg":
        rho, iters, resid = cg_solve(Sigma, mu, cg_max_iters, cg_rel_tol)
    elif solver == "zero":
        rho = np.zeros_like(mu)
    else:
        raise ValueError(solver)
    b, s, schur = intercept_from_rho(w, Z, V_prefix, omega, mu, rho)
    return RowResult(b, omega, mu, rho, m, schur, s, w, Sigma, iters, resid)


def oracle_head(q, k, v, lam, rows: Optional[Iterable[int]] = None, scale=None,
                solver="cholesky", cg_max_iters=0, cg_rel_tol=0.0):
    """Rows of one head (q, k, v shaped [n, d]); all rows when ``rows`` is None.
    Returns a dict of stacked per-row results."""
    n = q.shape[0]
    rows = list(range(n)) if rows is None else [int(r) for r in rows]
    out = {"rows": np.array(rows, dtype=np.int64), "b": [], "omega": [], "rho": [],
           "m": [], "schur": [], "cg_iters": [], "cg_resid": []}
    for i in rows:
        r = oracle_row(q[i], k[:i + 1], v[:i + 1], lam, scale, solver,
                       cg_max_iters, cg_rel_tol)
        out["b"].append(r.b)
        out["omega"].append(r.omega)
        out["rho"].append(r.rho)
        out["m"].append(r.m)
        out["schur"].append(r.schur)
        out["cg_iters"].append(r.cg_iters)
        out["cg_resid"].append(r.cg_resid)
    for key in ("b", "omega", "rho", "m", "schur", "cg_iters", "cg_resid"):
        out[key] = np.array(out[key]) if out[key] else np.zeros((0,))
    return out


# ---------------------------------------------------------------------------
# Independent formulations, used only to pin the oracle above.
# ---------------------------------------------------------------------------

def ridge_bruteforce(q_i, K_prefix, V_prefix, lam, scale=None):
    """Minimise sum_j w_ij ||v_j - b - W z_ij||^2 + lam ||W||_F^2 over (b, W)
    directly, as one weighted least-squares problem solved by numpy's lstsq
    ([LLA] 2.1, the objective, with the penalty reading in the module
    docstring). Returns (b, W) with W of shape (d_v, d)."""
    q_i = np.asarray(q_i, dtype=np.float64)
    d = q_i.shape[0]
    c = _scale(d, scale)
    _, _, w = causal_weights(q_i, K_prefix, c)
    Z = K_prefix - q_i[None, :]
    sw = np.sqrt(w)[:, None]
    A_data = np.hstack([np.ones((Z.shape[0], 1)), Z]) * sw
    Y_data = V_prefix * sw
    A_pen = np.hstack([np.zeros((d, 1)), np.sqrt(lam) * np.eye(d)])
    Y_pen = np.zeros((d, V_prefix.shape[1]))
    A = np.vstack([A_data, A_pen])
    Y = np.vstack([Y_data, Y_pen])
    theta, *_ = np.linalg.lstsq(A, Y, rcond=None)
    b = theta[0]
    W = theta[1:].T
    return b, W


def eq9_intercept(q_i, K_prefix, V_prefix, W_hat, scale=None):
    """b_i = W_i q_i + sum_j wbar_ij (v_j - W_i k_j), wbar = w / omega
    ([LLA] 2.1, Eq. (9)), for a given slope W_i."""
    d = q_i.shape[0]
    _, _, w = causal_weights(q_i, K_prefix, _scale(d, scale))
    wbar = w / np.sum(w)
    return W_hat @ q_i + wbar @ (V_prefix - K_prefix @ W_hat.T)


def covariance_form_intercept(q_i, K_prefix, V_prefix, rho, scale=None):
    """b_i = vbar_i - eta_i C_i rho_i with vbar, kbar the softmax means,
    C_i = sum_j wbar_ij (v_j - vbar)(k_j - kbar)^T the softmax-weighted
    value-key covariance and eta_i = omega_i / (omega_i - mu_i^T rho_i).
    [PLX] states LLA as the softmax output minus a covariance correction
    scaled by a boundary amplification factor; the form above is that
    statement written out by algebra on [LLA] Eq. (8)."""
    d = q_i.shape[0]
    _, _, w = causal_weights(q_i, K_prefix, _scale(d, scale))
    omega = np.sum(w)
    wbar = w / omega
    vbar = wbar @ V_prefix
    kbar = wbar @ K_prefix
    C = ((V_prefix - vbar) * wbar[:, None]).T @ (K_prefix - kbar)
    mu = omega * (kbar - q_i)
    eta = omega / (omega - mu @ rho)
    return vbar - eta * (C @ rho)


def tilde_moments(q_i, K_prefix, w, lam):
    """The memory-primitive form of the moments ([LLA] 2.2, Eqs. (10)-(12)):
    mu~ = sum w k, mu = mu~ - omega q, Sigma~ = sum w k k^T + lam I,
    Sigma = Sigma~ - mu~ q^T - q mu~^T + omega q q^T."""
    omega = float(np.sum(w))
    mu_t = K_prefix.T @ w
    mu = mu_t - omega * q_i
    Sig_t = (K_prefix * w[:, None]).T @ K_prefix + lam * np.eye(K_prefix.shape[1])
    Sigma = Sig_t - np.outer(mu_t, q_i) - np.outer(q_i, mu_t) + omega * np.outer(q_i, q_i)
    return omega, mu_t, mu, Sigma


def sample_rows(n: int, seed: int, n_first: int = 64, n_last: int = 32,
                n_uniform: int = 64) -> np.ndarray:
    """A seeded, stratified row sample for large heads: the first rows (where
    the fit is nearly an interpolation), the last rows, and uniform rows."""
    rng = np.random.default_rng(seed)
    first = np.arange(min(n_first, n))
    last = np.arange(max(0, n - n_last), n)
    uni = rng.integers(0, n, size=min(n_uniform, n))
    return np.unique(np.concatenate([first, last, uni]))
