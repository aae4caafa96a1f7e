"""A numpy model of the rounding in the matrix-core forward kernel.

TEST INFRASTRUCTURE ONLY, and not the oracle: the oracle (``oracle/``) is the
plain definition in float64. This module runs, per query, the algorithm the
matrix-core kernel runs, as its header (include/lla.h) and comments describe
it -- conjugate gradient on the system centred at the weighted key mean, with
fp16 operands under power-of-two scales and fp32 accumulation -- and rounds
where that description says the kernel rounds. It shares no code with the
HIP library and imports nothing from it. Its one use is to say how far an
honest fp16/fp32 implementation of the same CG lands from the float64 CG
iterate, so that the GPU parity tests' allowance for unconverged rows and the
CG-iterate tolerances are derived from data rather than chosen to pass.

Rounding modelled (every other operation is exact, i.e. float64):
  * keys, values: s k and sv v in fp16, s and sv powers of two from the
    head's largest key and value row norms (exact for bf16 inputs in range);
  * the query operand: fp16(q log2(e) / (sqrt(d) s)), so scores come out in
    log2 units; score sums rounded to fp32;
  * moment phase: weights exp2(S - mref) rounded to fp16 against a reference
    mref (the first 32-key tile's max, raised when a weight would pass 2^15),
    then omega and mu~ scaled by exp2(mref - m) with m the exact row max;
  * CG: direction d = fp16(p / sp) with sp a power of two, kbar rounded to
    fp16 as the expansion point, T = K d - kbar.d in fp32, U = fp16(w T)
    (two fp16 terms for the first 128 queries of a head when preconditioned,
    and everywhere with split_u), Y = sum U k and sum U in fp32; exact line search
    along d, Fletcher-Reeves beta; r, x, p held in fp32; the stop rule of
    lla.h;
  * output phase: rho in two fp16 terms, a / sA = w (1 - (k - kbar).rho) / sA
    rounded to fp16, sums in fp32.

``exact=True`` turns every rounding off; the model then runs the float64
CG of the oracle's ``cg_centred`` solver step for step (a CPU test pins it to
that), which is what makes its rounded runs a measurement of rounding alone.
"""
from __future__ import annotations

import numpy as np

LOG2E = 1.4426950408889634
ROW_NORM_CAP = 128.0


def _pow2_floor(x):
    return 2.0 ** np.floor(np.log2(x))


def _pow2_ceil(x):
    return 1.0 if not x > 0 else 2.0 ** np.ceil(np.log2(x))


class _R:
    """Rounding helpers; identity when exact."""

    def __init__(self, exact):
        self.exact = exact

    def h(self, x):      # to fp16 and back
        return np.asarray(x, np.float64) if self.exact else np.asarray(x, np.float16).astype(np.float64)

    def f(self, x):      # to fp32 and back
        return np.asarray(x, np.float64) if self.exact else np.asarray(x, np.float32).astype(np.float64)


def head_scales(q_head, k_head, v_head):
    """Power-of-two scales s (keys; queries enter as q / s) and sv (values)
    that bring the head's largest key row norm and largest value row norm to
    at most 128."""
    a = np.linalg.norm(k_head, axis=-1).max()
    b = np.linalg.norm(v_head, axis=-1).max()
    s = _pow2_floor(ROW_NORM_CAP / a) if a > 0 else 1.0
    sv = _pow2_floor(ROW_NORM_CAP / b) if b > 0 else 1.0
    return float(s), float(sv)


def _apply_two_term(R, M, r):
    """z = M r with M and r each carried as two fp16 terms under power-of-two
    scales (hi hi + hi lo + lo hi, fp32 accumulation)."""
    if R.exact:
        return M @ r
    sm = _pow2_ceil(np.abs(M).max())
    sr = _pow2_ceil(np.abs(r).max()) if np.any(r) else 1.0
    mh = R.h(M / sm)
    ml = R.h(M / sm - mh)
    rh = R.h(r / sr)
    rl = R.h(r / sr - rh)
    return R.f((mh @ rh + mh @ rl + ml @ rh) * (sm * sr))


def _two(R, x):
    """x as two fp16 terms (hi, lo) under a power-of-two scale: (hi, lo, scale)."""
    sc = _pow2_ceil(np.abs(x).max()) if np.any(x) else 1.0
    hi = R.h(x / sc)
    return hi, R.h(x / sc - hi), sc


class WoodGroup:
    """Group g < 8 of 32 rows as the kernel preconditions it (lla.h): the
    group's matrix M_g (the fp32 inverse of the scatter of its first 32 g keys
    about the group's point m, plus lam I; None for g = 0, where M = I / lam)
    and its 32 keys less m, U (d x 32, input units; columns past the head's
    end zero). The kernel's precomputation in fp32 (M U from M_g as applied,
    in two fp16 terms; A = I + U^T M U; its Cholesky factor L; V = L^{-1}) and
    its per-query products in two fp16 terms are modelled in ``apply``."""

    def __init__(self, Mg, U, lam):
        self.Mg, self.U, self.lam = Mg, U, lam
        self._cache = {}

    def _pre(self, R, s):
        key = (R.exact, s)
        if key not in self._cache:
            d = self.U.shape[0]
            lam_s = self.lam * s * s
            Us = self.U * s
            if self.Mg is None:
                M2 = np.eye(d) / lam_s
                Ms = None
            else:
                Ms = R.f(self.Mg / (s * s))
                if R.exact:
                    M2 = Ms
                else:
                    mh, ml, sm = _two(R, Ms)
                    M2 = (mh + ml) * sm
            MU = R.f(M2 @ Us)
            A = R.f(np.eye(32) + Us.T @ MU)
            if R.exact:
                V = np.linalg.inv(np.linalg.cholesky(A))
            else:
                L = np.linalg.cholesky(A.astype(np.float32))
                V = np.linalg.inv(L).astype(np.float32).astype(np.float64)
            self._cache[key] = (Ms, lam_s, _two(R, Us), _two(R, V), _two(R, -MU))
        return self._cache[key]

    def apply(self, R, r, s, nk):
        """z = P_i^{-1} r in scaled units for the row whose own keys are the
        group's first nk."""
        Ms, lam_s, (uh, ul, su), (vh, vl, sv), (nh, nl, smu) = self._pre(R, s)
        z = r / lam_s if Ms is None else _apply_two_term(R, Ms, r)
        keep = (np.arange(32) < nk).astype(float)
        zh, zl, sz = _two(R, z)
        t = R.f(uh.T @ zh + uh.T @ zl + ul.T @ zh) * (su * sz) * keep
        for vhh, vll in ((vh, vl), (vh.T, vl.T)):
            th, tl, st = _two(R, t)
            t = R.f(vhh @ th + vhh @ tl + vll @ th) * (sv * st) * keep
        xh, xl, sx = _two(R, t)
        return R.f(z + R.f(nh @ xh + nh @ xl + nl @ xh) * (smu * sx))


class WoodRow:
    def __init__(self, group, nk):
        self.group, self.nk = group, nk


def model_row(q_i, K, V, lam, cg_max_iters, cg_rel_tol, s, sv, split_u=False, exact=False,
              precond=None, first_block_split=None):
    """Row i of the causal forward (K, V: the prefix k_0..k_i, v_0..v_i) as
    the kernel computes it. ``precond``: None (plain CG) or the preconditioner
    matrix M (in input units, as the oracle defines it); it is rounded to fp32
    and applied in two fp16 terms. ``first_block_split``: whether the first
    128 queries of a head carry U in two terms (the kernel does so in its
    preconditioned mode;
    default: whether ``precond`` is given). Returns dict(b, rho_c, iters)."""
    if first_block_split is None:
        first_block_split = precond is not None
    R = _R(exact)
    d = q_i.shape[0]
    ks = R.h(s * K)                                    # fp16 scaled keys
    vs = R.h(sv * V)
    qop = R.h(q_i * (LOG2E / np.sqrt(d) / s))          # log2-unit query operand
    S = R.f(ks @ qop)                                  # scores, log2 units
    m = float(S.max())
    # moment phase against a reference raised only when needed
    mref = float(S[:32].max())
    om, mut = 0.0, np.zeros(d)
    for t0 in range(0, S.size, 32):
        st = S[t0:t0 + 32]
        if st.max() - mref > 15.0:
            nref = mref + (st.max() - mref)
            om *= 2.0 ** (mref - nref)
            mut = mut * 2.0 ** (mref - nref)
            mref = nref
        w16 = R.h(2.0 ** (st - mref))
        om += w16.sum()
        mut = mut + w16 @ ks[t0:t0 + 32]
    beta = 2.0 ** (mref - m)
    om, mut = float(R.f(om * beta)), R.f(mut * beta)
    kbar = R.f(mut / om)
    qs = s * q_i
    r = R.f(mut - om * qs)                             # mu in scaled units
    x = np.zeros(d)
    w = R.f(2.0 ** (S - m))                            # CG weights, fp32
    kb16 = R.h(kbar)
    lam_s = lam * s * s
    rr = float(r @ r)
    r0 = np.sqrt(rr)
    thr = cg_rel_tol * r0
    active = rr > 0.0 and cg_max_iters > 0
    iters = 0
    if isinstance(precond, WoodRow):
        def pz(rv):
            return precond.group.apply(R, rv, s, precond.nk)
    else:
        Ms = None if precond is None else R.f(np.asarray(precond) / (s * s))   # scaled units

        def pz(rv):
            return rv if Ms is None else _apply_two_term(R, Ms, rv)
    z = pz(r)
    rz = float(r @ z)
    sp = _pow2_ceil(np.abs(z).max()) if rr > 0 else 1.0
    dv = R.h(z / sp)
    for _ in range(cg_max_iters):
        if not active:
            break
        kbd = float(R.f(kb16 @ dv))
        T = R.f(ks @ dv - kbd)
        u = w * T
        if split_u or (first_block_split and K.shape[0] <= 128):
            # two fp16 terms: with split_u, and in the preconditioned mode in
            # a head's first block of 128 queries (prefixes of at most 128 keys)
            uh = R.h(u)
            U = uh + R.h(u - uh)
        else:
            U = R.h(u)
        Y = R.f(U @ ks)
        usum = float(R.f(U.sum()))
        Sd = R.f(Y - usum * kb16 + lam_s * dv)
        dAd = float(dv @ Sd)
        rd = float(r @ dv)
        if not dAd > 0.0:
            break
        al = rd / dAd
        r = R.f(r - al * Sd)
        x = R.f(x + al * dv)
        rrn = float(r @ r)
        iters += 1
        if np.sqrt(rrn) <= thr or rrn == 0.0:
            rr = rrn
            break
        z = pz(r)
        rzn = float(r @ z)
        be = rzn / rz * sp
        p = R.f(z + be * dv)
        sp = _pow2_ceil(np.abs(p).max())
        dv = R.h(p / sp)
        rr, rz = rrn, rzn
    # output phase: rho in two fp16 terms around kbar (fp32)
    srho = _pow2_ceil(np.abs(x).max()) if np.any(x) else 1.0
    rhi = R.h(x / srho)
    rlo = R.h(x / srho - rhi)
    rho2 = (rhi + rlo) * srho
    zr = R.f(ks @ rho2 - kbar @ rho2)                  # (k - kbar).rho
    nn = float(np.sqrt(x @ x))
    inv_sA = 1.0 / _pow2_ceil(1.0 + 2.0 * ROW_NORM_CAP * nn)
    a = R.h(w * (1.0 - zr) * inv_sA)
    den = float(R.f(a.sum()))
    out = R.f(a @ vs) / (den * sv)
    return {"b": out, "rho_c": x * s, "iters": iters}


def group_prefix(i):
    """Keys (a prefix) whose scatter matrix preconditions row i, as lla.h
    defines it: 0 for the first 32 rows; 32 g for group g = i // 32 < 8;
    beyond, 32 g rounded down to a multiple of 32 * 2^(floor(log2 g) - 2)."""
    g = i // 32
    if g < 8:
        return 32 * g
    e = int(g).bit_length() - 1
    step = 2 ** (e - 2)
    return 32 * (g // step) * step


def _group_inverse(Kp, m, lam, d):
    D = np.asarray(Kp, np.float64) - m
    P = np.asarray(D.T @ D + lam * np.eye(d), np.float32)
    M = np.linalg.inv(P).astype(np.float64)
    return 0.5 * (M + M.T)


def preconditioners(k, lam):
    """A function i -> the preconditioner of row i as lla.h defines it. From
    row 256 on, M = the fp32 inverse (symmetrised) of the scatter of the first
    N keys about their mean plus the ridge, one matrix per N as the kernel
    builds it. Below row 256, a WoodRow: the row's whole prefix about its
    group's point (k_0 for rows 0..31, else the mean of the first 32 g keys),
    applied as the kernel does, the group's matrix and the rank-r correction
    by the group's own keys (WoodGroup)."""
    k = np.asarray(k, np.float64)
    n, d = k.shape
    cache = {}

    def f(i):
        g = i // 32
        if g >= 8:
            N = group_prefix(i)
            if N not in cache:
                Kp = k[:N]
                cache[N] = _group_inverse(Kp, Kp.mean(axis=0), lam, d)
            return cache[N]
        if ("g", g) not in cache:
            m = k[0] if g == 0 else k[:32 * g].mean(axis=0)
            Mg = None if g == 0 else _group_inverse(k[:32 * g], m, lam, d)
            U = np.zeros((d, 32))
            top = min(32 * g + 32, n)
            U[:, :top - 32 * g] = (k[32 * g:top] - m).T
            cache[("g", g)] = WoodGroup(Mg, U, lam)
        return WoodRow(cache[("g", g)], i - 32 * g + 1)
    return f


def model_head(q, k, v, lam, cg_max_iters, cg_rel_tol, rows=None, split_u=False, exact=False,
               scales=None, precond=None):
    """Rows of one head ([n, d] arrays, the values the GPU reads, in float64).
    ``scales``: (s, sv) of the whole head (the kernel takes them over every
    row of the head, including rows after the ones asked for). ``precond``:
    None, or a function (i) -> preconditioner matrix of row i (or None)."""
    n = q.shape[0]
    rows = range(n) if rows is None else rows
    s, sv = head_scales(q, k, v) if scales is None else scales
    res = [model_row(q[i], k[:i + 1], v[:i + 1], lam, cg_max_iters, cg_rel_tol, s, sv,
                     split_u=split_u, exact=exact,
                     precond=None if precond is None else precond(i),
                     first_block_split=precond is not None) for i in rows]
    return {key: np.array([r[key] for r in res]) for key in ("b", "rho_c", "iters")}
