"""Pins for the float64 oracle: each test checks it against something other
than itself -- a library routine, a closed form, a textbook special case or
a property the pages state -- so that a dropped term, a wrong sign or index
or a transposed operand in the oracle fails at least one of them."""

import numpy as np
import pytest
from scipy.special import softmax

import oracle
from oracle import lla_oracle as O
from tests._support import load_golden, pad, worked_example_inputs
from local_linear_attention_flashlla_amd.workloads import make_workload, make_random


def _head(w, b=0, h=0):
    return w.q[b, h], w.k[b, h], w.v[b, h]


def _tiny_inputs(n, d, seed, scale_qk=1.0):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((n, d))
    k = rng.standard_normal((n, d))
    v = rng.standard_normal((n, d))
    if scale_qk is not None:
        q = q / np.linalg.norm(q, axis=1, keepdims=True) * scale_qk
        k = k / np.linalg.norm(k, axis=1, keepdims=True) * scale_qk
    return q, k, v


# --- [LLA] 2.1, the objective: brute-force weighted ridge least squares -----

@pytest.mark.parametrize("n,d,lam,seed,scale", [
    (12, 4, 0.3, 0, 1.0), (40, 8, 0.1, 1, 2.0), (64, 8, 1.0, 2, None),
    (5, 8, 0.05, 3, 1.0), (30, 3, 10.0, 4, 4.0), (64, 6, 1e-3, 5, 1.0)])
def test_intercept_is_ridge_argmin(n, d, lam, seed, scale):
    q, k, v = _tiny_inputs(n, d, seed, scale)
    for i in range(n):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], lam)
        b_ls, _ = O.ridge_bruteforce(q[i], k[:i + 1], v[:i + 1], lam)
        scale_b = max(1.0, np.linalg.norm(b_ls))
        assert np.linalg.norm(r.b - b_ls) <= 1e-8 * scale_b, (i, r.b, b_ls)


def test_ridge_pin_detects_planted_mistakes(monkeypatch):
    """Plant plausible mistakes in the oracle (on the CPU) and check that the
    ridge pin above rejects each one."""
    q, k, v = _tiny_inputs(20, 4, 7, 1.0)
    lam = 0.3

    def pin_ok():
        for i in (3, 9, 19):
            r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], lam)
            b_ls, _ = O.ridge_bruteforce(q[i], k[:i + 1], v[:i + 1], lam)
            if np.linalg.norm(r.b - b_ls) > 1e-8 * max(1, np.linalg.norm(b_ls)):
                return False
        return True

    assert pin_ok()
    good_moments = O.pairwise_moments
    good_intercept = O.intercept_from_rho

    def lam_doubled(q_i, K, w, lam_):
        return good_moments(q_i, K, w, 2 * lam_)

    # (flipping the sign of z and mu together is an exact symmetry: rho flips
    # too; a sign error on mu alone is a mistake)
    def mu_sign_flipped(q_i, K, w, lam_):
        Z, om, mu, S = good_moments(q_i, K, w, lam_)
        return Z, om, -mu, S

    def lam_dropped(q_i, K, w, lam_):
        return good_moments(q_i, K, w, 0.0 * lam_ + 1e-12)

    def denominator_omega(w, Z, V, omega, mu, rho):
        s = w * (1.0 - Z @ rho) / omega
        return s @ V, s, omega

    def plus_sign(w, Z, V, omega, mu, rho):
        schur = float(omega + mu @ rho)
        s = w * (1.0 + Z @ rho) / schur
        return s @ V, s, schur

    for name, fn in [("lam_doubled", lam_doubled), ("mu_sign", mu_sign_flipped),
                     ("lam_dropped", lam_dropped)]:
        monkeypatch.setattr(O, "pairwise_moments", fn)
        assert not pin_ok(), name
        monkeypatch.setattr(O, "pairwise_moments", good_moments)
    for name, fn in [("denominator_omega", denominator_omega), ("plus_sign", plus_sign)]:
        monkeypatch.setattr(O, "intercept_from_rho", fn)
        assert not pin_ok(), name
        monkeypatch.setattr(O, "intercept_from_rho", good_intercept)
    assert pin_ok()


# --- [LLA] 2.1, stated properties of the weights s_ij ------------------------

@pytest.mark.parametrize("name", ["tiny", "piecewise"])
def test_output_weights_sum_to_one_and_schur_positive(name):
    w = make_workload(name)
    q, k, v = _head(w)
    n = q.shape[0]
    neg = 0
    for i in list(range(0, n, max(1, n // 50))) + [n - 1]:
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], w.lam)
        assert abs(r.s.sum() - 1.0) < 1e-12
        assert r.schur > 0.0
        # the denominator is the Schur complement: it equals the row sum of
        # the unnormalised weights w (1 - z^T rho) for any rho
        Z = k[:i + 1] - q[i]
        assert abs((r.w * (1 - Z @ r.rho)).sum() - r.schur) <= 1e-10 * r.omega
        neg += int((r.s < 0).sum())
    # local linear weights are not a convex combination: some are negative
    assert neg > 0


def test_weight_convention_max_normalised():
    """w_ij = exp(s_ij - max_l s_il): the largest weight is exactly 1 and the
    normalised weights are scipy's softmax of the scaled scores."""
    q, k, v = _tiny_inputs(50, 8, 11, 3.0)
    for i in (0, 7, 49):
        s, m, w = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(8))
        assert w.max() == 1.0
        ref = softmax(k[:i + 1] @ q[i] / np.sqrt(8))
        np.testing.assert_allclose(w / w.sum(), ref, rtol=1e-13)


# --- limits and special cases -------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "piecewise"])
def test_lambda_to_infinity_is_causal_softmax(name):
    """lam -> inf gives rho -> 0 and s -> w / omega ([LLA] 2.1), i.e. causal
    scaled dot-product attention ([KM] ch. 1), here from scipy's softmax."""
    w = make_workload(name)
    q, k, v = _head(w)
    d = q.shape[1]
    for i in (0, 1, 17, q.shape[0] - 1):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], 1e12)
        ref = softmax(k[:i + 1] @ q[i] / np.sqrt(d)) @ v[:i + 1]
        np.testing.assert_allclose(r.b, ref, rtol=0, atol=1e-9 * max(1, np.abs(ref).max()))
        z = O.oracle_row(q[i], k[:i + 1], v[:i + 1], 1.0, solver="zero")
        np.testing.assert_allclose(z.b, ref, rtol=0, atol=1e-12 * max(1, np.abs(ref).max()))


@pytest.mark.parametrize("lam", [1e-3, 0.1, 1.0, 100.0])
def test_first_row_returns_first_value(lam):
    q, k, v = _tiny_inputs(3, 8, 2, 1.0)
    r = O.oracle_row(q[0], k[:1], v[:1], lam)
    np.testing.assert_allclose(r.b, v[0], rtol=1e-13, atol=1e-14)


def test_affine_targets_are_reproduced():
    """A local line reproduces an affine target exactly: v_j = A k_j + c with a
    vanishing ridge gives b_i = A q_i + c (the first-order bias removal that
    motivates LLA, [LLA] section 1 and 2.1)."""
    n, d = 40, 5
    q, k, _ = _tiny_inputs(n, d, 3, None)
    rng = np.random.default_rng(9)
    A = rng.standard_normal((d, d))
    c = rng.standard_normal(d)
    v = k @ A.T + c
    for i in range(d + 1, n):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], 1e-10)
        np.testing.assert_allclose(r.b, A @ q[i] + c, rtol=0, atol=1e-6)


def test_exact_interpolation_through_d_plus_one_points():
    """With exactly d+1 affinely independent keys and a vanishing ridge the
    local line interpolates them; b_i is the unique affine interpolant at q_i,
    whatever the (positive) weights are."""
    d = 4
    q, k, v = _tiny_inputs(d + 1, d, 21, None)
    i = d
    M = np.hstack([k[:i + 1], np.ones((i + 1, 1))])
    coef = np.linalg.solve(M, v[:i + 1])
    expect = np.append(q[i], 1.0) @ coef
    r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], 1e-11)
    np.testing.assert_allclose(r.b, expect, rtol=0, atol=1e-6)


def test_two_keys_in_one_dimension_is_linear_interpolation():
    """d = 1, two keys, vanishing ridge: the line through (k0, v0), (k1, v1)."""
    k = np.array([[0.3], [1.7]])
    v = np.array([[2.0], [-1.0]])
    q = np.array([0.9])
    r = O.oracle_row(q, k, v, 1e-12)
    expect = 2.0 + (-1.0 - 2.0) * (0.9 - 0.3) / (1.7 - 0.3)
    assert abs(r.b[0] - expect) < 1e-9


@pytest.mark.parametrize("d", [3, 16])
def test_equal_scores_worked_example(d):
    """The hand-derived example in tests/golden (every weight exactly 1, exact
    fractions from Eqs. (6)-(8)); zero-padding the head dimension changes
    nothing."""
    g = load_golden("equal_scores_worked_example.txt")
    q, k, v = worked_example_inputs(g, d)
    lam = g["lambda"][0]
    for i in range(q.shape[0]):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], lam)
        np.testing.assert_allclose(r.w, 1.0, rtol=0, atol=1e-15)
        assert abs(r.m - g["score"][0] / np.sqrt(d)) < 1e-15
        assert abs(r.omega - g[f"omega{i}"][0]) < 1e-12
        np.testing.assert_allclose(r.rho, pad(g[f"rho{i}"], d), rtol=0, atol=1e-12)
        assert abs(r.schur - g[f"schur{i}"][0]) < 1e-12
        np.testing.assert_allclose(r.s, g[f"s{i}"], rtol=0, atol=1e-12)
        np.testing.assert_allclose(r.b, pad(g[f"b{i}"], d), rtol=0, atol=1e-12)


# --- [LLA] Eq. (9) and the [PLX] covariance form ------------------------------

@pytest.mark.parametrize("n,d,lam,seed", [(30, 6, 0.2, 0), (64, 8, 1.0, 1)])
def test_eq9_linear_prediction_plus_local_residual(n, d, lam, seed):
    q, k, v = _tiny_inputs(n, d, seed, 2.0)
    for i in (0, 5, n // 2, n - 1):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], lam)
        _, W = O.ridge_bruteforce(q[i], k[:i + 1], v[:i + 1], lam)
        b9 = O.eq9_intercept(q[i], k[:i + 1], v[:i + 1], W)
        np.testing.assert_allclose(r.b, b9, rtol=0, atol=1e-8 * max(1, np.abs(r.b).max()))


@pytest.mark.parametrize("name", ["tiny", "piecewise"])
def test_covariance_form(name):
    w = make_workload(name)
    q, k, v = _head(w)
    for i in (0, 3, 100, q.shape[0] - 1):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], w.lam)
        bc = O.covariance_form_intercept(q[i], k[:i + 1], v[:i + 1], r.rho)
        np.testing.assert_allclose(r.b, bc, rtol=0, atol=1e-10 * max(1, np.abs(r.b).max()))


# --- [LLA] 2.2, Eqs. (10)-(12): the memory-primitive rewrite ------------------

@pytest.mark.parametrize("name", ["tiny", "piecewise"])
def test_tilde_moments_equal_pairwise(name):
    w = make_workload(name)
    q, k, v = _head(w)
    d = q.shape[1]
    for i in (0, 9, q.shape[0] - 1):
        _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(d))
        Z, om, mu, S = O.pairwise_moments(q[i], k[:i + 1], wt, w.lam)
        om2, mu_t, mu2, S2 = O.tilde_moments(q[i], k[:i + 1], wt, w.lam)
        assert abs(om - om2) <= 1e-13 * om
        np.testing.assert_allclose(mu, mu2, rtol=0, atol=1e-12 * max(1, np.abs(mu_t).max()))
        np.testing.assert_allclose(S, S2, rtol=0, atol=1e-12 * np.abs(S2).max())


# --- the solve ---------------------------------------------------------------

def test_cholesky_solve_matches_eigh_and_residual():
    w = make_workload("piecewise")
    q, k, v = _head(w, h=1)
    d = q.shape[1]
    for i in (2, 63, 64, 500, 1023):
        _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(d))
        _, _, mu, S = O.pairwise_moments(q[i], k[:i + 1], wt, w.lam)
        rho = O.cholesky_solve(S, mu)
        evals, evecs = np.linalg.eigh(S)
        rho_e = evecs @ ((evecs.T @ mu) / evals)
        np.testing.assert_allclose(rho, rho_e, rtol=1e-9, atol=1e-12)
        assert np.linalg.norm(S @ rho - mu) <= 1e-12 * np.linalg.norm(mu) * max(1, np.linalg.cond(S) / 1e2)


def _krylov_minimiser(S, b, k):
    """The k-th CG iterate from x0 = 0 is the minimiser of the S-norm error
    over span{b, Sb, ..., S^{k-1} b}: the Galerkin solution on that space."""
    vecs = [b / np.linalg.norm(b)]
    for _ in range(k - 1):
        vecs.append(S @ vecs[-1])
    Qb, _ = np.linalg.qr(np.stack(vecs, axis=1))
    return Qb @ np.linalg.solve(Qb.T @ S @ Qb, Qb.T @ b)


def test_cg_one_step_closed_form():
    q, k, v = _tiny_inputs(30, 6, 4, 1.0)
    for i in (3, 29):
        _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(6))
        _, _, mu, S = O.pairwise_moments(q[i], k[:i + 1], wt, 0.1)
        x, it, _ = O.cg_solve(S, mu, 1, 0.0)
        assert it == 1
        np.testing.assert_allclose(x, (mu @ mu) / (mu @ S @ mu) * mu, rtol=1e-13)


@pytest.mark.parametrize("steps", [2, 3, 5])
def test_cg_iterates_are_krylov_minimisers(steps):
    q, k, v = _tiny_inputs(40, 8, 6, 1.0)
    i = 39
    _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(8))
    _, _, mu, S = O.pairwise_moments(q[i], k[:i + 1], wt, 1.0)
    x, it, _ = O.cg_solve(S, mu, steps, 0.0)
    assert it == steps
    np.testing.assert_allclose(x, _krylov_minimiser(S, mu, steps), rtol=1e-8, atol=1e-12)


def test_cg_converges_to_cholesky_and_stop_rule():
    w = make_workload("tiny")
    q, k, v = _head(w)
    for i in (20, 255):
        _, _, wt = O.causal_weights(q[i], k[:i + 1], 0.25)
        _, _, mu, S = O.pairwise_moments(q[i], k[:i + 1], wt, w.lam)
        exact = O.cholesky_solve(S, mu)
        x, it, res = O.cg_solve(S, mu, 64, 1e-10)
        np.testing.assert_allclose(x, exact, rtol=1e-8, atol=1e-12)
        assert res <= 1e-10 and 1 <= it <= 64
        # the stop rule: the first step whose true residual is under tol
        tol = 1e-3
        x3, it3, res3 = O.cg_solve(S, mu, 64, tol)
        norms = []
        for kk in range(1, it3 + 1):
            xk = _krylov_minimiser(S, mu, kk)
            norms.append(np.linalg.norm(mu - S @ xk) / np.linalg.norm(mu))
        assert norms[-1] <= tol * (1 + 1e-6)
        assert all(nr > tol * (1 - 1e-6) for nr in norms[:-1])
        # tol = 0 runs exactly max_iters steps; max_iters = 0 gives rho = 0
        _, it0, _ = O.cg_solve(S, mu, 7, 0.0)
        assert it0 == 7
        xz, itz, rz = O.cg_solve(S, mu, 0, 0.0)
        assert itz == 0 and not xz.any() and rz == 1.0


def test_row_sample_is_sorted_unique_and_in_range():
    rows = oracle.sample_rows(4096, 3)
    assert rows[0] == 0 and rows[-1] == 4095
    assert np.all(np.diff(rows) > 0)


def test_workloads_recipes():
    """The generator's own contract: shapes, casts, unit rows and the
    piecewise 'query = next key' structure."""
    w = make_workload("piecewise")
    assert w.q.shape == (1, 2, 1024, 64) and w.q_dev.dtype == np.float32
    np.testing.assert_array_equal(w.q[0, 0, :-1], w.k[0, 0, 1:])
    np.testing.assert_allclose(np.linalg.norm(w.k[0, 0], axis=1), 1, rtol=1e-6)
    s = make_workload("standard", B=1, H=2, n=64)
    assert s.q_dev.dtype == np.uint16
    np.testing.assert_allclose(np.linalg.norm(s.q[0, 0], axis=1), 4, rtol=1e-2)
    # bf16 cast is round-to-nearest-even of the float32 value
    from local_linear_attention_flashlla_amd.workloads import f64_to_bf16_bits, bf16_bits_to_f64
    # ties go to the even mantissa: 1 + 2^-8 -> 1, 1 + 3*2^-8 -> 1 + 2^-6
    x = np.array([1.0, 1 + 2**-8, 1 + 3 * 2**-8, 1 + 2**-8 + 2**-20, -3.0e-3])
    got = bf16_bits_to_f64(f64_to_bf16_bits(x))
    np.testing.assert_array_equal(got[:4], [1.0, 1.0, 1 + 2**-6, 1 + 2**-7])
    assert got[4] == -197 / 128 * 2.0**-9
    r = make_random(1, 1, 10, 16, "bf16", qk_scale=None)
    assert r.k.shape == (1, 1, 10, 16)


# --- the mean-centred system: same exact answer --------------------------------

@pytest.mark.parametrize("name", ["tiny", "piecewise"])
def test_centred_system_exact_solution_equals_definition(name):
    """Solving Sigma_c rho_c = mu_i exactly and forming the centred output gives
    [LLA] Eq. (8) with the exact rho_i; the Sherman-Morrison map gives rho_i."""
    w = make_workload(name)
    q, k, v = _head(w)
    d = q.shape[1]
    for i in (0, 1, 5, 63, 64, 200, q.shape[0] - 1):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], w.lam)
        _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(d))
        Zc, om, kbar, mu, Sc = O.centred_moments(q[i], k[:i + 1], wt, w.lam)
        # parallel-axis identity against the explicit pairwise Sigma_i
        u = kbar - q[i]
        np.testing.assert_allclose(Sc + om * np.outer(u, u), r.Sigma, rtol=0,
                                   atol=1e-11 * np.abs(r.Sigma).max())
        rho_c = np.linalg.solve(Sc, mu)
        b, _, den = O.centred_intercept(wt, Zc, v[:i + 1], rho_c)
        assert abs(den - om) <= 1e-9 * om
        np.testing.assert_allclose(b, r.b, rtol=0, atol=1e-9 * max(1, np.abs(r.b).max()))
        np.testing.assert_allclose(rho_c / (1 + u @ rho_c), r.rho, rtol=1e-8, atol=1e-12)


def test_centred_cg_converges_to_definition():
    w = make_workload("piecewise")
    q, k, v = _head(w)
    for i in (3, 100, 700):
        r = O.oracle_row(q[i], k[:i + 1], v[:i + 1], w.lam)
        g = O.oracle_row(q[i], k[:i + 1], v[:i + 1], w.lam, solver="cg_centred",
                         cg_max_iters=400, cg_rel_tol=1e-13)
        assert g.cg_resid <= 1e-13
        np.testing.assert_allclose(g.b, r.b, rtol=0, atol=1e-8 * max(1, np.abs(r.b).max()))
        np.testing.assert_allclose(g.rho, r.rho, rtol=1e-6, atol=1e-10)
        assert abs(g.omega - r.omega) <= 1e-12 * r.omega


def test_centred_output_weights_sum_to_one_any_rho():
    """sum_j a_ij / sum_j a_ij = 1 trivially; the content is den = omega_i for
    any rho_c, because the centred differences have zero weighted mean."""
    q, k, v = _tiny_inputs(30, 6, 12, 2.0)
    rng = np.random.default_rng(0)
    i = 29
    _, _, wt = O.causal_weights(q[i], k[:i + 1], 1 / np.sqrt(6))
    Zc, om, kbar, mu, Sc = O.centred_moments(q[i], k[:i + 1], wt, 0.5)
    for _ in range(3):
        _, _, den = O.centred_intercept(wt, Zc, v[:i + 1], rng.standard_normal(6) * 10)
        assert abs(den - om) <= 1e-10 * om
