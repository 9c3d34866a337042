"""Pins of the fp64 oracle against facts that do not depend on its own code.

Every check here derives its expected value from the mathematics of the Mesa
layer's objective (MesaNet page, technical summary, "Mesa layer" section) by a
route that shares nothing with ``oracle/mesa_oracle.py``: a brute-force
least-squares fit of the objective, a library ridge regression, exact rational
Krylov projections, closed forms of one CG step and of the first token, and
exact invariances.  A plausible slip in the oracle (a dropped decay, a wrong
sign, a transposed state, a mis-indexed forget factor) fails at least one of
them; ``test_oracle_mutations.py`` plants such slips and checks that.
"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import cg_solve, mesa_forward, mesa_decode_step

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


# ---------------------------------------------------------------------------
# independent references
# ---------------------------------------------------------------------------

def zeta(gamma, beta, t, tp):
    """Forget weight of token tp seen at time t: beta_tp * prod_{i=tp+1..t} gamma_i."""
    w = float(beta[tp])
    for i in range(tp + 1, t + 1):
        w *= float(gamma[i])
    return w


def brute_force_objective(q, k, v, gamma, beta, Lam):
    """Minimise the layer's objective directly, one output row at a time.

    For each t and output row i: min_phi sum_{t'<=t} zeta_{tt'} (v_{t'i} - phi.k_{t'})^2
    + phi^T Lambda phi, solved as an ordinary least-squares problem on the
    stacked system [sqrt(zeta) K ; L^T] phi = [sqrt(zeta) v_i ; 0] with
    Lambda = L L^T.  Single (b, h) slice: q, k [T, dk]; v [T, dv].
    """
    T, dk = k.shape
    dv = v.shape[1]
    Lt = np.linalg.cholesky(Lam).T
    out = np.zeros((T, dv))
    for t in range(T):
        z = np.array([zeta(gamma, beta, t, tp) for tp in range(t + 1)])
        sz = np.sqrt(z)[:, None]
        Asys = np.vstack([sz * k[: t + 1], Lt])
        Phi = np.zeros((dv, dk))
        for i in range(dv):
            rhs = np.concatenate([sz[:, 0] * v[: t + 1, i], np.zeros(dk)])
            Phi[i] = np.linalg.lstsq(Asys, rhs, rcond=None)[0]
        out[t] = Phi @ q[t]
    return out


def rand_slice(rng, T, dk, dv, gamma_lo=0.5):
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    gamma = rng.uniform(gamma_lo, 1.0, (1, 1, T))
    beta = rng.uniform(0.05, 1.0, (1, 1, T))
    return q, k, v, gamma, beta


def rel(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return np.linalg.norm(a - b) / (den if den > 0 else 1.0)


# ---------------------------------------------------------------------------
# P1: the exact solution is the minimiser of the objective
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,T,dk,dv,full_lam", [
    (0, 8, 2, 2, False), (1, 10, 3, 2, False), (2, 12, 4, 3, False),
    (3, 9, 3, 4, True), (4, 12, 4, 4, True),
])
def test_p1_exact_solution_minimises_objective(seed, T, dk, dv, full_lam):
    rng = np.random.default_rng(seed)
    q, k, v, gamma, beta = rand_slice(rng, T, dk, dv)
    if full_lam:
        M = rng.standard_normal((dk, dk))
        lam = (M @ M.T + 0.5 * np.eye(dk))[None]
        Lam = lam[0]
    else:
        lam = rng.uniform(0.2, 1.5, (1, dk))
        Lam = np.diag(lam[0])
    ref = brute_force_objective(q[0, 0], k[0, 0], v[0, 0], gamma[0, 0], beta[0, 0], Lam)
    res = mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0)
    assert rel(res["o_exact"][0, 0], ref) < 1e-10
    # dk CG steps reach the exact solve (finite termination, P3) on these tiny systems
    assert rel(res["o_cg"][0, 0], ref) < 1e-8


@pytest.mark.parametrize("alpha", [0.3, 2.0])
def test_p1_no_forgetting_is_prefix_ridge_regression(alpha):
    """gamma = beta = 1, Lambda = alpha I: every prefix is a plain ridge fit."""
    from sklearn.linear_model import Ridge
    rng = np.random.default_rng(11)
    T, dk, dv = 10, 4, 3
    q = rng.standard_normal((1, 1, T, dk))
    k = rng.standard_normal((1, 1, T, dk))
    v = rng.standard_normal((1, 1, T, dv))
    ones = np.ones((1, 1, T))
    res = mesa_forward(q, k, v, ones, ones, np.full((1, dk), alpha), max_steps=dk, tol=0.0)
    for t in range(T):
        model = Ridge(alpha=alpha, fit_intercept=False, solver="svd")
        model.fit(k[0, 0, : t + 1], v[0, 0, : t + 1])
        ref = model.coef_ @ q[0, 0, t]
        assert rel(res["o_exact"][0, 0, t], ref) < 1e-10


# ---------------------------------------------------------------------------
# P2: H_t is symmetric, H_t + Lambda is SPD with the stated spectrum bounds
# ---------------------------------------------------------------------------

def test_p2_state_symmetric_spd_with_bounds():
    rng = np.random.default_rng(5)
    T, d = 40, 6
    q, k, v, gamma, beta = rand_slice(rng, T, d, d, gamma_lo=0.7)
    lam = rng.uniform(0.25, 1.0, (1, d))
    res = mesa_forward(q, k, v, gamma, beta, lam, max_steps=3, tol=0.0, record_every=1)
    for (t1, Hs, _Gs) in res["states"]:
        Ht = Hs[0, 0]
        assert np.array_equal(Ht, Ht.T)
        t = t1 - 1
        ev = np.linalg.eigvalsh(Ht + np.diag(lam[0]))
        upper = lam.max() + sum(zeta(gamma[0, 0], beta[0, 0], t, j) * float(k[0, 0, j] @ k[0, 0, j])
                                for j in range(t + 1))
        assert ev.min() >= lam.min() * (1 - 1e-12)
        assert ev.max() <= upper * (1 + 1e-12)
        # H_t = sum_j zeta_tj k_j k_j^T, assembled without the recurrence
        direct = sum(zeta(gamma[0, 0], beta[0, 0], t, j) * np.outer(k[0, 0, j], k[0, 0, j])
                     for j in range(t + 1))
        assert rel(Ht, direct) < 1e-12


def test_p2_cross_state_orientation():
    """G_t = sum_j zeta_tj v_j k_j^T with rows indexed by the value dimension."""
    rng = np.random.default_rng(6)
    T, dk, dv = 7, 3, 5
    q, k, v, gamma, beta = rand_slice(rng, T, dk, dv)
    res = mesa_forward(q, k, v, gamma, beta, np.ones((1, dk)), max_steps=1, tol=0.0)
    direct = sum(zeta(gamma[0, 0], beta[0, 0], T - 1, j) * np.outer(v[0, 0, j], k[0, 0, j])
                 for j in range(T))
    assert res["G_final"].shape == (1, 1, dv, dk)
    assert rel(res["G_final"][0, 0], direct) < 1e-12


# ---------------------------------------------------------------------------
# P3: finite termination on the configurations' own distributions
# ---------------------------------------------------------------------------

LM_DIST = dict(lam=("uniform", 0.25, 1.0), gamma_logit=(2.0, 6.0), beta=("uniform", 0.0, 1.0))
LONG_DIST = dict(lam=("const", 0.25), gamma_logit=(4.0, 9.0), beta=("beta", 5.0, 1.0))


@pytest.mark.parametrize("d,dist", [(16, "lm"), (32, "lm"), (64, "lm"), (128, "lm"), (128, "long")])
def test_p3_d_steps_equal_exact_solve(d, dist):
    """d CG steps reproduce the Cholesky solve, at the head dims of the workloads
    and on their distributions (language-model gates; near-one gates with
    Beta(5,1) writes and Lambda = 0.25 I)."""
    from test_regression_sequence_amd.inputs import small_fwd, make_fwd_inputs
    cfg = small_fwd(B=1, H=2, T=48, d=d, chunk=16, dtype="f32", max_steps=d,
                    **(LM_DIST if dist == "lm" else LONG_DIST))
    x = make_fwd_inputs(cfg)
    res = mesa_forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"],
                       max_steps=d, tol=0.0)
    assert rel(res["o_cg"], res["o_exact"]) < 1e-10
    assert rel(res["x_cg"], res["x_exact"]) < 1e-10


def test_exact_solve_rejects_a_system_that_is_not_positive_definite():
    """The exact solve is a Cholesky factorisation: a Lambda that makes H_t + Lambda
    indefinite (outside the pages' SPD regulariser) raises instead of solving."""
    rng = np.random.default_rng(19)
    q, k, v, gamma, beta = rand_slice(rng, 5, 4, 3)
    lam = np.array([[0.5, 0.5, -50.0, 0.5]])
    with pytest.raises(np.linalg.LinAlgError):
        mesa_forward(q, k, v, gamma, beta, lam, max_steps=2, tol=0.0, exact=True)
    # the CG schedule alone does not factorise, so it still runs
    mesa_forward(q, k, v, gamma, beta, lam, max_steps=2, tol=0.0, exact=False)


# ---------------------------------------------------------------------------
# P4: n-step CG is the A-norm projection onto the Krylov space (exact rationals)
# ---------------------------------------------------------------------------

def _frac_solve(M, b):
    n = len(M)
    A = [[Fraction(x) for x in row] + [Fraction(bb)] for row, bb in zip(M, b)]
    for c in range(n):
        piv = next(r for r in range(c, n) if A[r][c] != 0)
        A[c], A[piv] = A[piv], A[c]
        for r in range(n):
            if r != c and A[r][c] != 0:
                f = A[r][c] / A[c][c]
                A[r] = [a - f * bcol for a, bcol in zip(A[r], A[c])]
    return [A[i][n] / A[i][i] for i in range(n)]


def _krylov_iterate(A, q, n, x0=None):
    """The n-th CG iterate characterised without the CG recurrence, exactly.

    From x0 = 0: x_n = V (V^T A V)^{-1} V^T q with V = [q, Aq, ..., A^{n-1} q],
    the A-norm projection of the solution onto the Krylov space.  From a
    guess x0: x_n = x0 + V (V^T A V)^{-1} V^T r0 with r0 = q - A x0 and V a
    basis of K_n(A, r0), the projection onto the affine space x0 + K_n.
    """
    d = len(q)
    matvec = lambda x: [sum(A[i][j] * x[j] for j in range(d)) for i in range(d)]
    if x0 is None:
        x0 = [Fraction(0)] * d
    Ax0 = matvec(x0)
    r0 = [q[i] - Ax0[i] for i in range(d)]
    if n == 0 or all(z == 0 for z in r0):
        return list(x0)
    V = [r0]
    for _ in range(n - 1):
        V.append(matvec(V[-1]))
    AV = [matvec(vv) for vv in V]
    M = [[sum(V[a][i] * AV[b][i] for i in range(d)) for b in range(n)] for a in range(n)]
    rhs = [sum(V[a][i] * r0[i] for i in range(d)) for a in range(n)]
    c = _frac_solve(M, rhs)
    return [x0[i] + sum(c[a] * V[a][i] for a in range(n)) for i in range(d)]


@pytest.mark.parametrize("seed,d", [(0, 3), (1, 4), (2, 5), (3, 6)])
def test_p4_cg_iterates_are_krylov_projections(seed, d):
    rng = np.random.default_rng(seed)
    Mi = rng.integers(-3, 4, (d, d))
    A = (Mi @ Mi.T + np.diag(rng.integers(1, 4, d))).astype(np.int64)
    q = rng.integers(-4, 5, d).astype(np.int64)
    q[0] = q[0] if q[0] != 0 else 1
    Aq = [[Fraction(int(a)) for a in row] for row in A]
    qq = [Fraction(int(x)) for x in q]
    for n in range(1, d + 1):
        ref = np.array([float(z) for z in _krylov_iterate(Aq, qq, n)])
        x, steps = cg_solve(A[None].astype(float), q[None].astype(float), n, 0.0)
        assert steps[0] == n
        assert rel(x[0], ref) < 1e-9, (n, x[0], ref)
    check_residual_history(cg_solve, A, q, Aq, qq)


def _exact_residual_norm(Aq, qq, xq):
    d = len(qq)
    r = [qq[i] - sum(Aq[i][j] * xq[j] for j in range(d)) for i in range(d)]
    return float(sum(z * z for z in r)) ** 0.5


def check_residual_history(cg, A, q, Aq, qq):
    """The residual history of an n-step run: entry n is ||q - A x_n|| of the exact
    n-th Krylov projection (the recursive residual equals the true one in exact
    arithmetic); entries past the last executed step are NaN."""
    d = len(qq)
    forced = np.array([d - 1])
    x, steps, hist = cg(A[None].astype(float), q[None].astype(float), d + 2, 0.0,
                        forced_steps=forced, history=True)
    assert hist.shape == (1, d + 3)
    qn = float(sum(z * z for z in qq)) ** 0.5
    for n in range(d):
        ref = _exact_residual_norm(Aq, qq, _krylov_iterate(Aq, qq, n))
        assert abs(hist[0, n] - ref) <= 1e-9 * qn, (n, hist[0, n], ref)
    assert np.all(np.isnan(hist[0, d:]))


# ---------------------------------------------------------------------------
# forced step counts (the mode every dynamic-CG parity check runs the oracle in)
# ---------------------------------------------------------------------------

def test_forced_counts_are_krylov_projections_per_system(seed=20, d=5):
    """Each system of a batch, forced to its own count n_s below the cap, lands on
    its n_s-th A-norm Krylov projection (exact rationals); no system runs past
    its count and none stops short."""
    rng = np.random.default_rng(seed)
    S = 6
    As, qs, Aq, qq = [], [], [], []
    for _ in range(S):
        Mi = rng.integers(-3, 4, (d, d))
        A = (Mi @ Mi.T + np.diag(rng.integers(1, 4, d))).astype(np.int64)
        qv = rng.integers(-4, 5, d).astype(np.int64)
        qv[0] = qv[0] if qv[0] != 0 else 1
        As.append(A); qs.append(qv)
        Aq.append([[Fraction(int(a)) for a in row] for row in A])
        qq.append([Fraction(int(z)) for z in qv])
    forced = np.array([0, 1, 2, 3, 4, 2])
    x, steps = cg_solve(np.stack(As).astype(float), np.stack(qs).astype(float), d + 3, 0.0,
                        forced_steps=forced)
    assert np.array_equal(steps, forced)
    for s_ in range(S):
        ref = np.array([float(z) for z in _krylov_iterate(Aq[s_], qq[s_], int(forced[s_]))])
        assert rel(x[s_], ref) < 1e-9, (s_, forced[s_])
    # the tolerance plays no part once counts are forced
    x2, steps2 = cg_solve(np.stack(As).astype(float), np.stack(qs).astype(float), d + 3, 1e3,
                          forced_steps=forced)
    assert np.array_equal(steps2, forced) and np.array_equal(x2, x)


def test_forced_counts_reproduce_free_runs_bitwise(seed=21):
    """Forcing every token to n equals the fixed-step mode at n; forcing the
    counts a tolerance run chose reproduces that run's x and o bit for bit."""
    rng = np.random.default_rng(seed)
    T, d = 14, 16
    q, k, v, gamma, beta = rand_slice(rng, T, d, d, gamma_lo=0.8)
    lam = rng.uniform(0.25, 1.0, (1, d))
    for n in (1, 3, 5):
        fixed = mesa_forward(q, k, v, gamma, beta, lam, max_steps=n, tol=0.0, exact=False)
        forced = mesa_forward(q, k, v, gamma, beta, lam, max_steps=n + 4, tol=0.0, exact=False,
                              forced_steps=np.full((1, 1, T), n))
        assert np.array_equal(forced["o_cg"], fixed["o_cg"])
        assert np.array_equal(forced["x_cg"], fixed["x_cg"])
        assert np.all(forced["steps"] == n)
    free = mesa_forward(q, k, v, gamma, beta, lam, max_steps=12, tol=1e-3, exact=False)
    assert len(np.unique(free["steps"])) > 3 and free["steps"].max() == 12
    again = mesa_forward(q, k, v, gamma, beta, lam, max_steps=12, tol=1e-3, exact=False,
                         forced_steps=free["steps"])
    for key in ("o_cg", "x_cg", "steps", "res_norm", "res_prev"):
        assert np.array_equal(again[key], free[key]), key


# ---------------------------------------------------------------------------
# solving at selected tokens only (how long sequences are sampled)
# ---------------------------------------------------------------------------

def test_solve_at_matches_the_objective_and_the_full_run(seed=22):
    """Outputs at the selected tokens are the objective's minimiser (brute force)
    and the full run's outputs bit for bit; other tokens stay zero; the states
    still absorb every token."""
    rng = np.random.default_rng(seed)
    T, dk, dv = 11, 4, 3
    q, k, v, gamma, beta = rand_slice(rng, T, dk, dv)
    lam = rng.uniform(0.3, 1.2, (1, dk))
    at = np.zeros(T, bool)
    at[[0, 3, 4, 9]] = True
    part = mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0, solve_at=at,
                        record_every=2)
    full = mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0, record_every=2)
    ref = brute_force_objective(q[0, 0], k[0, 0], v[0, 0], gamma[0, 0], beta[0, 0], np.diag(lam[0]))
    assert rel(part["o_exact"][0, 0][at], ref[at]) < 1e-10
    for key in ("o_cg", "x_cg", "o_exact", "steps"):
        assert np.array_equal(part[key][0, 0][at], full[key][0, 0][at]), key
        assert np.all(part[key][0, 0][~at] == 0), key
    assert np.array_equal(part["H_final"], full["H_final"])
    assert np.array_equal(part["G_final"], full["G_final"])
    assert [t for t, _, _ in part["states"]] == [t for t, _, _ in full["states"]]
    for (_, Hp, Gp), (_, Hf, Gf) in zip(part["states"], full["states"]):
        assert np.array_equal(Hp, Hf) and np.array_equal(Gp, Gf)
    # no token solved: the final states are the weighted sums of the whole prefix
    none = mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0, solve_at=np.zeros(T, bool))
    direct = sum(zeta(gamma[0, 0], beta[0, 0], T - 1, j) * np.outer(v[0, 0, j], k[0, 0, j])
                 for j in range(T))
    assert rel(none["G_final"][0, 0], direct) < 1e-12
    assert np.all(none["o_cg"] == 0)


# ---------------------------------------------------------------------------
# P4w, P3w, P7w: CG from a warm start
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("seed,d", [(4, 3), (5, 4), (6, 5)])
def test_p4w_warm_iterates_are_affine_krylov_projections(seed, d):
    rng = np.random.default_rng(seed)
    Mi = rng.integers(-3, 4, (d, d))
    A = (Mi @ Mi.T + np.diag(rng.integers(1, 4, d))).astype(np.int64)
    q = rng.integers(-4, 5, d).astype(np.int64)
    x0 = rng.integers(-3, 4, d).astype(np.int64)
    Aq = [[Fraction(int(a)) for a in row] for row in A]
    qq = [Fraction(int(z)) for z in q]
    xq = [Fraction(int(z)) for z in x0]
    for n in range(0, d + 1):
        ref = np.array([float(z) for z in _krylov_iterate(Aq, qq, n, xq)])
        x, steps = cg_solve(A[None].astype(float), q[None].astype(float), n, 0.0,
                            x0=x0[None].astype(float))
        assert rel(x[0], ref) < 1e-9, (n, x[0], ref)


def test_p3w_warm_start_d_steps_reach_the_solution():
    rng = np.random.default_rng(16)
    S, d = 6, 16
    M = rng.standard_normal((S, d, d))
    A = np.matmul(M, M.transpose(0, 2, 1)) / d + np.eye(d)
    q = rng.standard_normal((S, d))
    x0 = 3.0 * rng.standard_normal((S, d))
    x, steps = cg_solve(A, q, d, 0.0, x0=x0)
    ref = np.stack([np.linalg.solve(A[s], q[s]) for s in range(S)])
    assert rel(x, ref) < 1e-10


def test_p7w_exact_guess_takes_no_step():
    A = np.eye(3)[None] * 2.0
    q = np.array([[1.0, 0.0, 0.0]])
    x0 = np.array([[0.5, 0.0, 0.0]])
    for tol in (1e-6, 0.0):
        x, n = cg_solve(A, q, 10, tol, x0=x0)
        assert n[0] == 0 and np.array_equal(x, x0)


def test_p4w_warm_sequence_chains_previous_solution():
    """Token t starts from token t-1's n-step result: chained affine Krylov projections,
    with the states, forget factors and outputs in exact rationals."""
    rng = np.random.default_rng(17)
    T, d, n = 5, 3, 2
    ki = rng.integers(-2, 3, (T, d)); vi = rng.integers(-2, 3, (T, d)); qi = rng.integers(-3, 4, (T, d))
    gnum = rng.integers(1, 4, T); bnum = rng.integers(1, 4, T); lnum = rng.integers(1, 4, d)
    gam = [Fraction(int(a), 4) for a in gnum]       # in (0, 1)
    bet = [Fraction(int(a), 2) for a in bnum]
    lam = [Fraction(int(a), 2) for a in lnum]
    x_init = [Fraction(int(a)) for a in rng.integers(-1, 2, d)]
    Hq = [[Fraction(0)] * d for _ in range(d)]
    Gq = [[Fraction(0)] * d for _ in range(d)]
    xp = list(x_init)
    ref_o = []
    for t in range(T):
        kk = [Fraction(int(a)) for a in ki[t]]; vv = [Fraction(int(a)) for a in vi[t]]
        Hq = [[gam[t] * Hq[i][j] + bet[t] * kk[i] * kk[j] for j in range(d)] for i in range(d)]
        Gq = [[gam[t] * Gq[i][j] + bet[t] * vv[i] * kk[j] for j in range(d)] for i in range(d)]
        Aq = [[Hq[i][j] + (lam[i] if i == j else 0) for j in range(d)] for i in range(d)]
        xp = _krylov_iterate(Aq, [Fraction(int(a)) for a in qi[t]], n, xp)
        ref_o.append([float(sum(Gq[i][j] * xp[j] for j in range(d))) for i in range(d)])
    res = mesa_forward(qi[None, None].astype(float), ki[None, None].astype(float),
                       vi[None, None].astype(float),
                       np.array([[[float(g) for g in gam]]]), np.array([[[float(b) for b in bet]]]),
                       np.array([[float(l) for l in lam]]), max_steps=n, tol=0.0, exact=False,
                       warm_start=True, x_init=np.array([[[float(a) for a in x_init]]]))
    assert rel(res["o_cg"][0, 0], np.array(ref_o)) < 1e-10


def test_p4w_chunked_warm_start_chains_within_chunks(T=7, d=3, n=2, lag=2, chunk=4):
    """The chunked warm start: token t starts from token t-lag's n-step result when
    both lie in the same chunk of `chunk` tokens, otherwise from 0 -- chained
    affine Krylov projections with states, forget factors and outputs in exact
    rationals (tokens 0, 1 and 4, 5 start cold; 2, 3, 6 from 0, 1, 4)."""
    rng = np.random.default_rng(23)
    ki = rng.integers(-2, 3, (T, d)); vi = rng.integers(-2, 3, (T, d)); qi = rng.integers(-3, 4, (T, d))
    gam = [Fraction(int(a), 4) for a in rng.integers(1, 4, T)]
    bet = [Fraction(int(a), 2) for a in rng.integers(1, 4, T)]
    lam = [Fraction(int(a), 2) for a in rng.integers(1, 4, d)]
    Hq = [[Fraction(0)] * d for _ in range(d)]
    Gq = [[Fraction(0)] * d for _ in range(d)]
    xs, ref_o = [], []
    for t in range(T):
        kk = [Fraction(int(a)) for a in ki[t]]; vv = [Fraction(int(a)) for a in vi[t]]
        Hq = [[gam[t] * Hq[i][j] + bet[t] * kk[i] * kk[j] for j in range(d)] for i in range(d)]
        Gq = [[gam[t] * Gq[i][j] + bet[t] * vv[i] * kk[j] for j in range(d)] for i in range(d)]
        Aq = [[Hq[i][j] + (lam[i] if i == j else 0) for j in range(d)] for i in range(d)]
        same_chunk = t - lag >= 0 and (t - lag) // chunk == t // chunk
        x0 = xs[t - lag] if same_chunk else [Fraction(0)] * d
        xs.append(_krylov_iterate(Aq, [Fraction(int(a)) for a in qi[t]], n, x0))
        ref_o.append([float(sum(Gq[i][j] * xs[-1][j] for j in range(d))) for i in range(d)])
    res = mesa_forward(qi[None, None].astype(float), ki[None, None].astype(float),
                       vi[None, None].astype(float),
                       np.array([[[float(g) for g in gam]]]), np.array([[[float(b) for b in bet]]]),
                       np.array([[float(l) for l in lam]]), max_steps=n, tol=0.0, exact=False,
                       warm_start=True, warm_lag=lag, warm_chunk=chunk)
    assert rel(res["o_cg"][0, 0], np.array(ref_o)) < 1e-10
    assert rel(res["x_cg"][0, 0], np.array([[float(z) for z in x] for x in xs])) < 1e-10


# ---------------------------------------------------------------------------
# P5: one CG step is a normalised gated-linear-attention read-out
# ---------------------------------------------------------------------------

def test_p5_one_step_is_scaled_gla():
    rng = np.random.default_rng(7)
    T, dk, dv = 20, 5, 4
    q, k, v, gamma, beta = rand_slice(rng, T, dk, dv)
    lam = rng.uniform(0.3, 1.0, (1, dk))
    res = mesa_forward(q, k, v, gamma, beta, lam, max_steps=1, tol=0.0, exact=False)
    g, b = gamma[0, 0], beta[0, 0]
    for t in range(T):
        qt = q[0, 0, t]
        scores = [zeta(g, b, t, j) * float(k[0, 0, j] @ qt) for j in range(t + 1)]
        quad = float(qt @ (lam[0] * qt)) + sum(zeta(g, b, t, j) * float(k[0, 0, j] @ qt) ** 2
                                              for j in range(t + 1))
        alpha = float(qt @ qt) / quad
        ref = alpha * sum(s * v[0, 0, j] for j, s in enumerate(scores))
        assert rel(res["o_cg"][0, 0, t], ref) < 1e-12
        assert res["steps"][0, 0, t] == 1


# ---------------------------------------------------------------------------
# P6: first token, closed form (Sherman-Morrison)
# ---------------------------------------------------------------------------

def test_p6_first_token_sherman_morrison():
    rng = np.random.default_rng(8)
    dk, dv = 6, 5
    q, k, v, gamma, beta = rand_slice(rng, 1, dk, dv)
    lam = rng.uniform(0.3, 1.2, (1, dk))
    res = mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0)
    kk, qq, vv, bb = k[0, 0, 0], q[0, 0, 0], v[0, 0, 0], beta[0, 0, 0]
    li = 1.0 / lam[0]
    ref = bb * vv * float(kk @ (li * qq)) / (1.0 + bb * float(kk @ (li * kk)))
    assert rel(res["o_exact"][0, 0, 0], ref) < 1e-12
    assert rel(res["o_cg"][0, 0, 0], ref) < 1e-10


# ---------------------------------------------------------------------------
# P7: special cases
# ---------------------------------------------------------------------------

def test_p7_zero_steps_gives_zero_output():
    rng = np.random.default_rng(9)
    q, k, v, gamma, beta = rand_slice(rng, 6, 4, 4)
    res = mesa_forward(q, k, v, gamma, beta, np.ones((1, 4)), max_steps=0, tol=0.0)
    assert np.all(res["o_cg"] == 0) and np.all(res["steps"] == 0)


def test_p7_no_writes_gives_zero_output_and_one_step_solve():
    rng = np.random.default_rng(10)
    q, k, v, gamma, _ = rand_slice(rng, 6, 4, 3)
    beta = np.zeros_like(gamma)
    for tol in (0.0, 1e-6):
        res = mesa_forward(q, k, v, gamma, beta, np.full((1, 4), 0.5), max_steps=5, tol=tol)
        assert np.all(res["o_cg"] == 0)
        # H = 0, Lambda = 0.5 I: one step lands on q / 0.5, then rho == 0 stops CG
        assert np.allclose(res["x_cg"], q / 0.5, rtol=1e-15, atol=0)
        assert np.all(res["steps"] == 1)


def test_p7_tolerance_stops_before_iteration():
    """A residual already at or under tol runs zero iterations."""
    A = np.eye(3)[None] * 2.0
    qv = np.array([[1e-7, 0.0, 0.0]])
    x, n = cg_solve(A, qv, 10, 1e-6)
    assert n[0] == 0 and np.all(x == 0)
    x, n = cg_solve(A, qv * 100, 10, 1e-6)
    assert n[0] == 1 and np.allclose(x, qv * 50)


# ---------------------------------------------------------------------------
# P8: invariances
# ---------------------------------------------------------------------------

def test_p8_joint_scaling_of_beta_lambda_states():
    rng = np.random.default_rng(12)
    T, d = 16, 5
    q, k, v, gamma, beta = rand_slice(rng, T, d, d)
    lam = rng.uniform(0.25, 1.0, (1, d))
    h0 = rng.standard_normal((1, 1, d, d)); h0 = h0 @ h0.transpose(0, 1, 3, 2)
    g0 = rng.standard_normal((1, 1, d, d))
    c = 4.0
    for tol in (0.0, 1e-3):
        a = mesa_forward(q, k, v, gamma, beta, lam, h0=h0, g0=g0, max_steps=4, tol=tol, exact=False)
        b = mesa_forward(q, k, v, gamma, c * beta, c * lam, h0=c * h0, g0=c * g0,
                         max_steps=4, tol=tol, exact=False)
        assert np.array_equal(a["steps"], b["steps"])
        assert rel(b["o_cg"], a["o_cg"]) < 1e-14
        assert rel(c * b["x_cg"], a["x_cg"]) < 1e-14


def test_p8_linear_in_values():
    rng = np.random.default_rng(13)
    q, k, v, gamma, beta = rand_slice(rng, 12, 4, 4)
    lam = np.full((1, 4), 0.7)
    a = mesa_forward(q, k, v, gamma, beta, lam, max_steps=3, tol=0.0, exact=False)
    b = mesa_forward(q, k, -2.0 * v, gamma, beta, lam, max_steps=3, tol=0.0, exact=False)
    assert rel(b["o_cg"], -2.0 * a["o_cg"]) < 1e-14


def test_p8_energy_error_monotone():
    rng = np.random.default_rng(14)
    d = 12
    M = rng.standard_normal((d, d))
    A = M @ M.T / d + 0.5 * np.eye(d)
    qv = rng.standard_normal(d)
    xs = np.linalg.solve(A, qv)
    errs = []
    for n in range(d + 1):
        x, _ = cg_solve(A[None], qv[None], n, 0.0)
        e = x[0] - xs
        errs.append(float(e @ A @ e))
    assert all(errs[i + 1] <= errs[i] * (1 + 1e-9) + 1e-28 for i in range(d))
    assert errs[-1] < 1e-20 * errs[0]


# ---------------------------------------------------------------------------
# decode step == one more token of the forward recurrence
# ---------------------------------------------------------------------------

def test_decode_step_continues_forward():
    rng = np.random.default_rng(15)
    T, d = 9, 4
    q, k, v, gamma, beta = rand_slice(rng, T + 1, d, d)
    lam = rng.uniform(0.25, 1.0, (1, d))
    full = mesa_forward(q, k, v, gamma, beta, lam, max_steps=3, tol=0.0)
    pre = mesa_forward(q[:, :, :T], k[:, :, :T], v[:, :, :T], gamma[:, :, :T], beta[:, :, :T],
                       lam, max_steps=3, tol=0.0)
    dec = mesa_decode_step(q[:, :, T], k[:, :, T], v[:, :, T], gamma[:, :, T], beta[:, :, T], lam,
                           pre["H_final"], pre["G_final"], max_steps=3, tol=0.0)
    assert rel(dec["o"], full["o_cg"][:, :, T]) < 1e-13
    assert rel(dec["h"], full["H_final"]) < 1e-14


def test_decode_step_warm_continues_warm_forward():
    rng = np.random.default_rng(18)
    T, d = 7, 4
    q, k, v, gamma, beta = rand_slice(rng, T + 1, d, d)
    lam = rng.uniform(0.25, 1.0, (1, d))
    full = mesa_forward(q, k, v, gamma, beta, lam, max_steps=2, tol=0.0, warm_start=True)
    pre = mesa_forward(q[:, :, :T], k[:, :, :T], v[:, :, :T], gamma[:, :, :T], beta[:, :, :T],
                       lam, max_steps=2, tol=0.0, warm_start=True)
    dec = mesa_decode_step(q[:, :, T], k[:, :, T], v[:, :, T], gamma[:, :, T], beta[:, :, T], lam,
                           pre["H_final"], pre["G_final"], max_steps=2, tol=0.0,
                           x0=pre["x_cg"][:, :, T - 1])
    assert rel(dec["o"], full["o_cg"][:, :, T]) < 1e-13
    assert rel(dec["x"], full["x_cg"][:, :, T]) < 1e-13
