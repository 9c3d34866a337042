"""Pins of the oracle's backward pass (implicit differentiation of the solves).

The gradients are checked against central finite differences of the layer's
objective solved by brute force (``test_oracle_pins.brute_force_objective``:
least squares on the stacked forget-weighted system, no oracle code), against
finite differences of the exact forward for the initial and final states, and
against identities that follow from the layer's homogeneity: o is linear in
q, linear in (v, g0) jointly, and unchanged when (beta, Lambda, h0, g0) are
scaled together.  With d CG steps for both solves the CG-schedule gradients
equal the exact ones.
"""
import numpy as np
import pytest

import test_oracle_pins as pins
from oracle import mesa_backward, mesa_forward

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def tiny(seed, T=5, dk=3, dv=2, H=1):
    rng = np.random.default_rng(seed)
    q, k, v, gamma, beta = pins.rand_slice(rng, T, dk, dv)
    if H > 1:
        q, k, v = (np.concatenate([a] + [rng.standard_normal(a.shape) for _ in range(H - 1)], axis=1)
                   for a in (q, k, v))
        gamma = np.concatenate([gamma] + [rng.uniform(0.5, 1.0, gamma.shape) for _ in range(H - 1)], axis=1)
        beta = np.concatenate([beta] + [rng.uniform(0.05, 1.0, beta.shape) for _ in range(H - 1)], axis=1)
    lam = rng.uniform(0.3, 1.2, (H, dk))
    d_o = rng.standard_normal((1, H, T, dv))
    return q, k, v, gamma, beta, lam, d_o


def loss_brute(q, k, v, gamma, beta, lam, d_o):
    tot = 0.0
    for h in range(q.shape[1]):
        o = pins.brute_force_objective(q[0, h], k[0, h], v[0, h], gamma[0, h], beta[0, h], np.diag(lam[h]))
        tot += float(np.sum(d_o[0, h] * o))
    return tot


def fd_grad(f, arr, eps=1e-6):
    g = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        i = it.multi_index
        old = arr[i]
        arr[i] = old + eps
        fp = f()
        arr[i] = old - eps
        fm = f()
        arr[i] = old
        g[i] = (fp - fm) / (2 * eps)
    return g


@pytest.mark.parametrize("seed,H", [(0, 1), (1, 2)])
def test_gradients_match_finite_differences_of_the_objective(seed, H):
    q, k, v, gamma, beta, lam, d_o = tiny(seed, H=H)
    g = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, chunk=2)
    args = [q, k, v, gamma, beta, lam]
    for name, idx in (("dq", 0), ("dk", 1), ("dv", 2), ("dgamma", 3), ("dbeta", 4), ("dlam", 5)):
        ref = fd_grad(lambda: loss_brute(*args, d_o), args[idx])
        assert pins.rel(g[name], ref) < 1e-6, name


def full_lambda(rng, H, dk):
    M = rng.standard_normal((H, dk, dk))
    return 0.3 * M @ M.transpose(0, 2, 1) / dk + np.stack([np.diag(rng.uniform(0.3, 1.2, dk)) for _ in range(H)])


def test_full_lambda_gradient_along_symmetric_directions_matches_the_objective():
    """A full SPD Lambda: <dLambda, E> for symmetric directions E against central
    differences of the brute-force objective (which depends on Lambda's
    symmetric part only)."""
    q, k, v, gamma, beta, _, d_o = tiny(6, H=2)
    lam = full_lambda(np.random.default_rng(7), 2, 3)
    g = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, chunk=2)
    assert g["dlam"].shape == (2, 3, 3)

    def loss():
        return sum(float(np.sum(d_o[0, h] * pins.brute_force_objective(q[0, h], k[0, h], v[0, h], gamma[0, h],
                                                                       beta[0, h], lam[h])))
                   for h in range(2))

    eps = 1e-6
    for h in range(2):
        for i in range(3):
            for j in range(i, 3):
                E = np.zeros_like(lam)
                E[h, i, j] += 1.0
                E[h, j, i] += 1.0 if i != j else 0.0
                lam += eps * E
                fp = loss()
                lam -= 2 * eps * E
                fm = loss()
                lam += eps * E
                assert abs(np.sum(g["dlam"] * E) - (fp - fm) / (2 * eps)) < 1e-6 * (1 + abs(fp)), (h, i, j)


def test_full_lambda_gradient_is_the_partial_derivative_of_each_entry():
    """Every entry on its own (a non-symmetric perturbation of the solves):
    dLambda = -sum_t y_t x_t^T against central differences of the exact
    forward; a diagonal Lambda's gradient is the diagonal of the full one."""
    q, k, v, gamma, beta, lamd, d_o = tiny(8)
    lam = full_lambda(np.random.default_rng(9), 1, 3)
    g = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, chunk=2)

    T = q.shape[2]

    def loss():
        # sum_t d_o_t . G_t (H_t + Lambda)^{-1} q_t with the states assembled from the
        # forget weights and a general (LU) solve: a non-symmetric perturbation of one
        # entry is a different system, which a symmetric factorisation cannot represent
        tot = 0.0
        for t in range(T):
            z = [pins.zeta(gamma[0, 0], beta[0, 0], t, j) for j in range(t + 1)]
            Ht = sum(zj * np.outer(k[0, 0, j], k[0, 0, j]) for j, zj in enumerate(z))
            Gt = sum(zj * np.outer(v[0, 0, j], k[0, 0, j]) for j, zj in enumerate(z))
            tot += float(d_o[0, 0, t] @ (Gt @ np.linalg.solve(Ht + lam[0], q[0, 0, t])))
        return tot

    assert pins.rel(g["dlam"], fd_grad(loss, lam)) < 1e-6
    gd = mesa_backward(q, k, v, gamma, beta, lamd, d_o, max_steps=4, tol=0.0, chunk=2)
    gf = mesa_backward(q, k, v, gamma, beta, np.stack([np.diag(r) for r in lamd]), d_o, max_steps=4, tol=0.0,
                       chunk=2)
    assert np.allclose(gd["dlam"], np.diagonal(gf["dlam"], axis1=1, axis2=2), rtol=1e-12, atol=1e-12)
    for name in ("dq", "dk", "dv", "dgamma", "dbeta"):
        assert np.allclose(gd[name], gf[name], rtol=1e-12, atol=1e-12), name


def test_state_gradients_match_finite_differences_of_the_forward():
    q, k, v, gamma, beta, lam, d_o = tiny(2, dv=3)
    rng = np.random.default_rng(3)
    M = rng.standard_normal((1, 1, 3, 3))
    h0 = M @ M.transpose(0, 1, 3, 2) * 0.3
    g0 = rng.standard_normal((1, 1, 3, 3))
    Dh = rng.standard_normal((1, 1, 3, 3))
    Dg = rng.standard_normal((1, 1, 3, 3))

    def loss():
        r = mesa_forward(q, k, v, gamma, beta, lam, max_steps=0, tol=0.0, h0=h0, g0=g0)
        return float(np.sum(d_o * r["o_exact"]) + np.sum(Dh * r["H_final"]) + np.sum(Dg * r["G_final"]))

    g = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, h0=h0, g0=g0,
                      dh_final=Dh, dg_final=Dg, chunk=3)
    assert pins.rel(g["dg0"], fd_grad(loss, g0)) < 1e-6
    # h0 is a symmetric state: derivatives along symmetric directions
    eps = 1e-6
    for i in range(3):
        for j in range(i, 3):
            E = np.zeros((1, 1, 3, 3))
            E[0, 0, i, j] += 1.0
            E[0, 0, j, i] += 1.0 if i != j else 0.0
            h0 += eps * E
            fp = loss()
            h0 -= 2 * eps * E
            fm = loss()
            h0 += eps * E
            assert abs(np.sum(g["dh0"] * E) - (fp - fm) / (2 * eps)) < 1e-6 * (1 + abs(fp))
    # the remaining inputs, with states at both ends
    for name, arr in (("dk", k), ("dgamma", gamma), ("dbeta", beta), ("dv", v)):
        assert pins.rel(g[name], fd_grad(loss, arr)) < 1e-6, name


def test_homogeneity_identities():
    q, k, v, gamma, beta, lam, d_o = tiny(4, T=7, dk=4, dv=4, H=2)
    rng = np.random.default_rng(5)
    M = rng.standard_normal((1, 2, 4, 4))
    h0 = M @ M.transpose(0, 1, 3, 2) * 0.2
    g0 = rng.standard_normal((1, 2, 4, 4))
    Dh = rng.standard_normal((1, 2, 4, 4))
    Dg = rng.standard_normal((1, 2, 4, 4))
    f = mesa_forward(q, k, v, gamma, beta, lam, max_steps=0, tol=0.0, h0=h0, g0=g0)
    g = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, h0=h0, g0=g0,
                      dh_final=Dh, dg_final=Dg, chunk=3)
    L_o = np.sum(d_o * f["o_exact"])
    L_h, L_g = np.sum(Dh * f["H_final"]), np.sum(Dg * f["G_final"])
    assert abs(np.sum(q * g["dq"]) - L_o) < 1e-10 * (1 + abs(L_o))
    assert abs(np.sum(v * g["dv"]) + np.sum(g0 * g["dg0"]) - (L_o + L_g)) < 1e-10 * (1 + abs(L_o))
    scale = np.sum(beta * g["dbeta"]) + np.sum(lam * g["dlam"]) + np.sum(h0 * g["dh0"]) + np.sum(g0 * g["dg0"])
    assert abs(scale - (L_h + L_g)) < 1e-9 * (1 + abs(L_h) + abs(L_g))


def test_cg_schedule_with_d_steps_equals_exact():
    q, k, v, gamma, beta, lam, d_o = tiny(6, T=9, dk=4, dv=3, H=2)
    a = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=4, tol=0.0, chunk=4)
    b = mesa_backward(q, k, v, gamma, beta, lam, d_o, max_steps=0, tol=0.0, exact=True, chunk=4)
    for name in ("dq", "dk", "dv", "dgamma", "dbeta", "dlam", "dh0", "dg0"):
        assert pins.rel(a[name], b[name]) < 1e-9, name
    assert np.all(a["adj_steps"] == 4)
