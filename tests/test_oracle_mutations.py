"""Plant plausible slips in a private copy of the oracle and check the pins catch them.

Each mutation edits the oracle's source text, loads it as a throwaway module
(on the CPU; the real oracle is untouched) and runs the independent checks of
``test_oracle_pins`` against it.  Every mutation must make at least one check
fail, which shows the pins constrain each part of the oracle's arithmetic.
"""
import importlib.util
import os
import types

import numpy as np
import pytest

import test_oracle_backward as bwd
import test_oracle_pins as pins
import test_oracle_preprocess as prep

SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                   "oracle", "mesa_oracle.py")

MUTATIONS = {
    "no_decay_on_G": ("Gs = g_t * Gs + b_t", "Gs = Gs + b_t"),
    "no_decay_on_H": ("Hs = g_t * Hs + b_t", "Hs = Hs + b_t"),
    "no_write_strength_on_H": ("Hs = g_t * Hs + b_t * (", "Hs = g_t * Hs + ("),
    "G_transposed": ("(vf[:, t][:, :, None] * kt[:, None, :])", "(kt[:, :, None] * vf[:, t][:, None, :])"),
    "lambda_decayed": ("A = Hs + Lam", "A = Hs + g_t * Lam"),
    "lambda_dropped": ("A = Hs + Lam", "A = Hs + 1e-3 * Lam"),
    "solve_before_update": [("kt = kf[:, t]\n", "kt = kf[:, t]\n        Hprev = Hs\n"),
                            ("A = Hs + Lam", "A = Hprev + Lam")],
    "residual_sign": ("r -= alpha[:, None] * w", "r += alpha[:, None] * w"),
    "cg_beta_inverted": ("beta = np.where(go, rho_new / np.where(go, rho, 1.0), 0.0)",
                         "beta = np.where(go, rho / np.where(go, rho_new, 1.0), 0.0)"),
    "step_length_wrong": ("alpha = np.where(go, rho / np.where(go, pw, 1.0), 0.0)",
                          "alpha = np.where(go, 1.0 / np.where(go, pw, 1.0), 0.0)"),
    "output_reads_query": ("o_cg[:, t] = np.matmul(Gs, xs[:, :, None])[:, :, 0]",
                           "o_cg[:, t] = np.matmul(Gs, qf[:, t][:, :, None])[:, :, 0]"),
    "forget_factor_shifted": ("g_t = gf[:, t][:, None, None]",
                              "g_t = gf[:, max(t - 1, 0)][:, None, None]"),
    "tolerance_ignored": ("go = np.sqrt(rho) > tol", "go = np.ones(S, dtype=bool)"),
    "direction_not_updated": ("p = np.where(go[:, None], r + beta[:, None] * p, p)",
                              "p = np.where(go[:, None], r, p)"),
    "warm_residual_not_shifted": ("r = q - np.matmul(A, x[:, :, None])[:, :, 0]", "r = q.copy()"),
    "warm_guess_dropped": ("x = np.array(x0, dtype=np.float64).reshape(q.shape)",
                           "x = np.zeros_like(q)"),
    "warm_chain_not_advanced": ("        x_prev = xs\n", "\n"),
    "prep_taps_reversed": ("y += w[None, :, None, :, i] * seq", "y += w[None, :, None, :, W - 1 - i] * seq"),
    "prep_history_reversed": ("seq = np.concatenate([pre, x], axis=2)",
                              "seq = np.concatenate([pre[:, :, ::-1], x], axis=2)"),
    "prep_norm_over_time": ("nrm = np.linalg.norm(y, axis=-1, keepdims=True)",
                            "nrm = np.linalg.norm(y, axis=-2, keepdims=True)"),
    "prep_history_out_shifted": ("return out, seq[:, :, T:]", "return out, seq[:, :, T - 1:-1]"),
    "prep_current_token_dropped": ("for i in range(W):\n        y +=", "for i in range(1, W):\n        y +="),
    "bwd_adjoint_previous_state": ("dxt = Gt.T @ dot", "dxt = Gp.T @ dot"),
    "bwd_H_adjoint_sign": ("Hhat = Hhat - np.outer(yt, xt)", "Hhat = Hhat + np.outer(yt, xt)"),
    "bwd_dk_one_sided": ("bt * ((Hhat + Hhat.T) @ kt", "bt * ((2 * Hhat) @ kt"),
    "bwd_no_decay_on_G_adjoint": ("Ghat = gf[s_, t] * Ghat", "Ghat = Ghat"),
    "bwd_dgamma_current_state": ("np.sum(Hhat * Hp) + np.sum(Ghat * Gp)", "np.sum(Hhat * Ht) + np.sum(Ghat * Gt)"),
    "bwd_dbeta_without_G": ("kt @ Hhat @ kt + vt @ Ghat @ kt", "kt @ Hhat @ kt"),
    "bwd_dlam_sign": ("dlam[h] -= yt * xt", "dlam[h] += yt * xt"),
    "bwd_full_dlam_transposed": ("dlam[h] -= np.outer(yt, xt)", "dlam[h] -= np.outer(xt, yt)"),
    "bwd_full_lambda_read_as_diagonal": ("Lam = lam[h] if full else np.diag(lam[h])",
                                         "Lam = np.diag(np.diagonal(lam[h])) if full else np.diag(lam[h])"),
    "bwd_dq_is_solution": ('out["dq"][s_, t] = yt', 'out["dq"][s_, t] = xt'),
    "bwd_dv_reads_solution": ('out["dv"][s_, t] = bt * (Ghat @ kt)', 'out["dv"][s_, t] = bt * (Ghat @ xt)'),
    "forced_steps_one_extra": ("go = it < forced_steps", "go = it <= forced_steps"),
    "forced_steps_ignored": ("            go = it < forced_steps\n", "            go = np.ones(S, dtype=bool)\n"),
    "forced_steps_as_a_cap": ("            go = it < forced_steps\n",
                              "            go = (it < forced_steps) & ((np.sqrt(rho) > tol) if tol > 0 else True)\n"),
    "solve_at_skips_state_update": (
        "        Hs = g_t * Hs + b_t * (kt[:, :, None] * kt[:, None, :])\n",
        "        Hs = (g_t * Hs + b_t * (kt[:, :, None] * kt[:, None, :])) if (solve_at is None or solve_at[t]) else Hs\n"),
    "solve_at_shifted": ("if solve_at is not None and not solve_at[t]:",
                         "if solve_at is not None and not solve_at[max(t - 1, 0)]:"),
    "exact_solve_wrong_triangle": ("cho_solve(cho_factor(A[s], lower=True), b[s])",
                                   "cho_solve((np.linalg.cholesky(A[s]), False), b[s])"),
    "history_index_shifted": ("hist[go, it + 1] = np.sqrt(rho_new[go])", "hist[go, it] = np.sqrt(rho_new[go])"),
    "history_squared": ("hist[go, it + 1] = np.sqrt(rho_new[go])", "hist[go, it + 1] = rho_new[go]"),
    "chunked_warm_lag_ignored": ("x0 = x_cg[:, t - warm_lag]", "x0 = x_cg[:, t - 1]"),
    "chunked_warm_crosses_chunks": ("(warm_chunk is None or (t - warm_lag) // warm_chunk == t // warm_chunk)",
                                    "(warm_chunk is None or True)"),
    "warm_chain_from_exact_solution": [("        x_prev = xs\n", "\n"),
                                       ("            x_ex[:, t] = xe\n",
                                        "            x_ex[:, t] = xe\n            x_prev = xe\n")],
}


def load_mutant(name):
    edits = MUTATIONS[name]
    if isinstance(edits, tuple):
        edits = [edits]
    src = open(SRC).read()
    for old, new in edits:
        assert src.count(old) >= 1, f"mutation anchor missing: {old!r}"
        src = src.replace(old, new, 1)
    mod = types.ModuleType(f"mutant_{name}")
    exec(compile(src, f"<mutant {name}>", "exec"), mod.__dict__)
    return mod


def run_pins(m):
    """Independent checks; return the list of those that fail for module m."""
    failed = []
    rng = np.random.default_rng(0)
    # P1: brute-force objective, diagonal and full Lambda, dk != dv
    for seed, T, dk, dv, full in [(2, 12, 4, 3, False), (3, 9, 3, 4, True)]:
        rng = np.random.default_rng(seed)
        q, k, v, gamma, beta = pins.rand_slice(rng, T, dk, dv)
        if full:
            M = rng.standard_normal((dk, dk)); lam = (M @ M.T + 0.5 * np.eye(dk))[None]; Lam = lam[0]
        else:
            lam = rng.uniform(0.2, 1.5, (1, dk)); Lam = np.diag(lam[0])
        ref = pins.brute_force_objective(q[0, 0], k[0, 0], v[0, 0], gamma[0, 0], beta[0, 0], Lam)
        try:
            res = m.mesa_forward(q, k, v, gamma, beta, lam, max_steps=dk, tol=0.0)
            if pins.rel(res["o_exact"][0, 0], ref) > 1e-10 or pins.rel(res["o_cg"][0, 0], ref) > 1e-8:
                failed.append("P1")
        except Exception:
            failed.append("P1-crash")
    # P4: Krylov projections
    d = 4
    rng = np.random.default_rng(1)
    Mi = rng.integers(-3, 4, (d, d))
    A = (Mi @ Mi.T + np.diag(rng.integers(1, 4, d))).astype(np.int64)
    qv = np.array([1, -2, 3, 1])
    from fractions import Fraction
    Aq = [[Fraction(int(a)) for a in row] for row in A]
    qq = [Fraction(int(x)) for x in qv]
    for n in range(1, d + 1):
        ref = np.array([float(z) for z in pins._krylov_iterate(Aq, qq, n)])
        x, steps = m.cg_solve(A[None].astype(float), qv[None].astype(float), n, 0.0)
        if pins.rel(x[0], ref) > 1e-9:
            failed.append("P4")
            break
    try:
        pins.check_residual_history(m.cg_solve, A, qv, Aq, qq)
    except AssertionError:
        failed.append("P4-history")
    # P5: one step == scaled GLA
    rng = np.random.default_rng(7)
    T, dk, dv = 10, 5, 4
    q, k, v, gamma, beta = pins.rand_slice(rng, T, dk, dv)
    lam = rng.uniform(0.3, 1.0, (1, dk))
    try:
        res = m.mesa_forward(q, k, v, gamma, beta, lam, max_steps=1, tol=0.0, exact=False)
        g, b = gamma[0, 0], beta[0, 0]
        for t in range(T):
            qt = q[0, 0, t]
            sc = [pins.zeta(g, b, t, j) * float(k[0, 0, j] @ qt) for j in range(t + 1)]
            quad = float(qt @ (lam[0] * qt)) + sum(s * float(k[0, 0, j] @ qt) for j, s in enumerate(sc))
            ref = float(qt @ qt) / quad * sum(s * v[0, 0, j] for j, s in enumerate(sc))
            if pins.rel(res["o_cg"][0, 0, t], ref) > 1e-12:
                failed.append("P5")
                break
    except Exception:
        failed.append("P5-crash")
    # P4w: warm-started iterates are affine Krylov projections
    xw = np.array([1, 0, -2, 1])
    xq = [Fraction(int(z)) for z in xw]
    for n in range(0, d + 1):
        ref = np.array([float(z) for z in pins._krylov_iterate(Aq, qq, n, xq)])
        x, steps = m.cg_solve(A[None].astype(float), qv[None].astype(float), n, 0.0,
                              x0=xw[None].astype(float))
        if pins.rel(x[0], ref) > 1e-9:
            failed.append("P4w")
            break
    # chained warm start over a sequence, recurrent and chunked (exact rationals)
    saved = pins.mesa_forward
    try:
        pins.mesa_forward = m.mesa_forward
        for tag, fn in (("P4w-seq", pins.test_p4w_warm_sequence_chains_previous_solution),
                        ("P4w-chunked", pins.test_p4w_chunked_warm_start_chains_within_chunks)):
            try:
                fn()
            except AssertionError:
                failed.append(tag)
            except Exception:
                failed.append(tag + "-crash")
    finally:
        pins.mesa_forward = saved
    # preprocessing against library convolution and normalisation
    saved = prep.qk_preprocess
    try:
        prep.qk_preprocess = m.qk_preprocess
        for fn in (lambda: prep.test_matches_library_convolution_and_normalisation(3),
                   prep.test_short_sequences_carry_history_through):
            try:
                fn()
            except AssertionError:
                failed.append("prep")
                break
    finally:
        prep.qk_preprocess = saved
    # backward: finite differences of the brute-force objective and of the forward
    saved = (bwd.mesa_backward, bwd.mesa_forward)
    try:
        bwd.mesa_backward, bwd.mesa_forward = m.mesa_backward, m.mesa_forward
        for fn in (lambda: bwd.test_gradients_match_finite_differences_of_the_objective(0, 1),
                   bwd.test_state_gradients_match_finite_differences_of_the_forward,
                   bwd.test_homogeneity_identities,
                   bwd.test_full_lambda_gradient_along_symmetric_directions_matches_the_objective,
                   bwd.test_full_lambda_gradient_is_the_partial_derivative_of_each_entry):
            try:
                fn()
            except AssertionError:
                failed.append("bwd")
                break
            except Exception:
                failed.append("bwd-crash")
                break
    finally:
        bwd.mesa_backward, bwd.mesa_forward = saved
    # forced step counts and solving at selected tokens
    saved = (pins.mesa_forward, pins.cg_solve)
    try:
        pins.mesa_forward, pins.cg_solve = m.mesa_forward, m.cg_solve
        for tag, fn in (("forced", pins.test_forced_counts_are_krylov_projections_per_system),
                        ("forced-free", pins.test_forced_counts_reproduce_free_runs_bitwise),
                        ("solve_at", pins.test_solve_at_matches_the_objective_and_the_full_run)):
            try:
                fn()
            except AssertionError:
                failed.append(tag)
            except Exception:
                failed.append(tag + "-crash")
    finally:
        pins.mesa_forward, pins.cg_solve = saved
    # P7: tolerance stops before an iteration
    x, n = m.cg_solve(np.eye(3)[None] * 2.0, np.array([[1e-7, 0.0, 0.0]]), 10, 1e-6)
    if n[0] != 0:
        failed.append("P7")
    return failed


def test_unmutated_oracle_passes_all():
    import oracle.mesa_oracle as real
    assert run_pins(real) == []


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name):
    assert run_pins(load_mutant(name)), f"mutation {name} slipped past every pin"
