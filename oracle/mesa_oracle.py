"""fp64 CPU oracle for the Mesa layer (test infrastructure, not product code).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this module.  It shares no code with the HIP path.

What it computes (MesaNet: "Sequence Modeling by Locally Optimal Test-Time
Training", technical summary, "Mesa layer" section):

* The layer's map at time t minimises the forget-weighted, Lambda-regularised
  squared error over the prefix (the section's objective, argmin over Phi of
  1/2 sum_{t'<=t} zeta_{tt'} ||v_t' - Phi k_t'||^2 + 1/2 Tr(Phi Lambda Phi^T)),
  and the output is Phi_t q_t.
* With zeta_{tt'} = beta_t' * prod_{i=t'+1..t} gamma_i (our reading of the
  "cumulative forget factor"; beta is the per-token write strength), the first
  order condition gives Phi_t = G_t (H_t + Lambda)^{-1} with
  H_t = gamma_t H_{t-1} + beta_t k_t k_t^T and G_t = gamma_t G_{t-1} + beta_t v_t k_t^T.
* The method does not invert: it solves (H_t + Lambda) x_t = q_t by conjugate
  gradient (same section: the optimal query response is found by CG), with a
  fixed number of steps or a stopping criterion whose step count varies per
  token ("dynamic compute" paragraph), and emits o_t = G_t x_t.

This file runs that recurrence token by token with explicit H_t and G_t, and
solves every system twice: by the CG schedule (the result the GPU path must
match) and exactly, by a Cholesky factorisation (the definition).  The same
section makes Lambda symmetric positive definite, so every H_t + Lambda is SPD;
the factorisation fails loudly on any system that is not, which makes every
exact solve also a check of that property.

CG variant (the pages say only "CG"): Hestenes-Stiefel conjugate gradient from
x_0 = 0 with the recursive residual, as in Saad, "Iterative Methods for Sparse
Linear Systems", 2nd ed., Algorithm 6.18.  A token stops before an iteration
when sqrt(rho) <= tol (tol > 0), when rho == 0, or when p.(A p) <= 0; a
stopped token never restarts.  ``steps`` counts executed alpha updates.

Warm start (the "significance" section names warm-started optimisation as a
way to cut the solver's cost, without details): on request CG starts from a
given x_0 with the residual r_0 = q - A x_0; in a sequence, token t starts from
token t-1's CG result (token 0 from a given guess, else 0).  The product A x_0
is not counted in ``steps``.
"""
from __future__ import annotations

import numpy as np

__all__ = ["cg_solve", "cholesky_solve", "mesa_forward", "mesa_decode_step", "diag_or_full", "qk_preprocess",
           "mesa_backward"]


def diag_or_full(lam: np.ndarray, H: int, d: int) -> np.ndarray:
    """Lambda per head as a full [H, d, d] matrix (accepts a [H, d] diagonal)."""
    lam = np.asarray(lam, dtype=np.float64)
    if lam.shape == (H, d):
        out = np.zeros((H, d, d))
        idx = np.arange(d)
        out[:, idx, idx] = lam
        return out
    if lam.shape == (H, d, d):
        return lam.copy()
    raise ValueError(f"lambda must be [H, d] or [H, d, d], got {lam.shape}")


def cg_solve(A: np.ndarray, q: np.ndarray, max_steps: int, tol: float,
             forced_steps: np.ndarray | None = None, residuals: bool = False,
             x0: np.ndarray | None = None, history: bool = False):
    """Batched conjugate gradient on A[s] x = q[s], fp64.

    A: [S, d, d] symmetric positive definite; q: [S, d].
    forced_steps: optional [S] ints -- run exactly that many iterations per
    system (the breakdown guard still applies) instead of the tolerance test.
    x0: optional [S, d] initial guesses (default 0); the residual starts at
    q - A x0.
    Returns (x [S, d], steps [S] int64); with ``residuals=True`` also the
    recursive residual norms ||r|| after the last executed iteration and
    before it (equal to ||r_0|| for systems that ran no iteration); with
    ``history=True`` also [S, max_steps + 1] norms ||r_n|| after each executed
    iteration n (column 0: ||r_0||; NaN past a system's last iteration).
    """
    A = np.asarray(A, dtype=np.float64)
    q = np.asarray(q, dtype=np.float64)
    S = q.shape[0]
    if x0 is None:
        x = np.zeros_like(q)
        r = q.copy()
    else:
        x = np.array(x0, dtype=np.float64).reshape(q.shape)
        r = q - np.matmul(A, x[:, :, None])[:, :, 0]
    p = r.copy()
    rho = np.einsum("sd,sd->s", r, r)
    rho_prev = rho.copy()
    steps = np.zeros(S, dtype=np.int64)
    stopped = np.zeros(S, dtype=bool)
    hist = np.full((S, int(max_steps) + 1), np.nan)
    hist[:, 0] = np.sqrt(rho)
    if forced_steps is not None:
        forced_steps = np.asarray(forced_steps).reshape(S)
    for it in range(int(max_steps)):
        if forced_steps is not None:
            go = it < forced_steps
        elif tol > 0:
            go = np.sqrt(rho) > tol
        else:
            go = np.ones(S, dtype=bool)
        go &= ~stopped
        go &= rho > 0
        stopped |= ~go
        if not go.any():
            break
        w = np.matmul(A, p[:, :, None])[:, :, 0]
        pw = np.einsum("sd,sd->s", p, w)
        ok = pw > 0
        stopped |= go & ~ok
        go &= ok
        alpha = np.where(go, rho / np.where(go, pw, 1.0), 0.0)
        x += alpha[:, None] * p
        r -= alpha[:, None] * w
        rho_new = np.einsum("sd,sd->s", r, r)
        beta = np.where(go, rho_new / np.where(go, rho, 1.0), 0.0)
        p = np.where(go[:, None], r + beta[:, None] * p, p)
        rho_prev = np.where(go, rho, rho_prev)
        rho = np.where(go, rho_new, rho)
        steps += go
        hist[go, it + 1] = np.sqrt(rho_new[go])
    out = (x, steps)
    if residuals:
        out += (np.sqrt(rho), np.sqrt(rho_prev))
    if history:
        out += (hist,)
    return out


def cholesky_solve(A: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Exact solve of the SPD systems A[s] x = b[s] by Cholesky, fp64.

    A: [S, d, d]; b: [S, d].  ``scipy.linalg.cho_factor`` raises
    ``numpy.linalg.LinAlgError`` when a system is not positive definite.
    """
    from scipy.linalg import cho_factor, cho_solve
    A = np.asarray(A, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    x = np.empty_like(b)
    for s in range(A.shape[0]):
        x[s] = cho_solve(cho_factor(A[s], lower=True), b[s])
    return x


def _flat(a, S, *tail):
    return np.asarray(a, dtype=np.float64).reshape(S, *tail)


def mesa_forward(q, k, v, gamma, beta, lam, *, max_steps: int, tol: float,
                 h0=None, g0=None, forced_steps=None, exact: bool = True,
                 record_every: int | None = None, solve_at=None,
                 warm_start: bool = False, x_init=None, residual_history: bool = False,
                 warm_lag: int = 1, warm_chunk: int | None = None):
    """Token-by-token Mesa layer over [B, H, T, d] inputs, fp64.

    q, k: [B, H, T, dk]; v: [B, H, T, dv]; gamma, beta: [B, H, T];
    lam: [H, dk] diagonal or [H, dk, dk] SPD; h0: [B, H, dk, dk]; g0: [B, H, dv, dk].
    forced_steps: optional [B, H, T] CG step counts (see :func:`cg_solve`).
    record_every: if given, H and G after every ``record_every``-th token
    (and after the last token) are returned in ``states``.
    solve_at: optional [T] bool -- solve and emit outputs only at these token
    positions (the state recurrence still runs over every token); outputs at
    other positions are left at zero.  Used to sample long sequences.
    warm_start: start token t's CG from token (t - warm_lag)'s CG result.  With
    warm_lag = 1 and no warm_chunk (the recurrent reading), token 0 starts from
    x_init ([B, H, dk], default 0).  With warm_chunk = C, a token whose
    predecessor t - warm_lag lies in an earlier chunk of C tokens (or before
    the sequence) starts from 0: the chunked reading, in which the chunks of a
    sequence are solved in parallel and only earlier tokens of the same chunk
    can hand over their solutions.  Needs every token solved (no solve_at).
    residual_history: also return ``res_hist`` [B, H, T, max_steps + 1], each
    solved token's recursive residual norm after every CG iteration (see
    :func:`cg_solve`; zero rows at tokens not solved).

    Returns a dict with o_cg, x_cg, steps, H_final, G_final (and o_exact,
    x_exact when ``exact``), shaped like the inputs.
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hh, T, dk = q.shape
    dv = np.asarray(v).shape[-1]
    S = B * Hh
    qf = _flat(q, S, T, dk)
    kf = _flat(k, S, T, dk)
    vf = _flat(v, S, T, dv)
    gf = _flat(gamma, S, T)
    bf = _flat(beta, S, T)
    Lam = diag_or_full(lam, Hh, dk)
    Lam = np.broadcast_to(Lam[None], (B, Hh, dk, dk)).reshape(S, dk, dk)
    Hs = np.zeros((S, dk, dk)) if h0 is None else _flat(h0, S, dk, dk).copy()
    Gs = np.zeros((S, dv, dk)) if g0 is None else _flat(g0, S, dv, dk).copy()
    fs = None if forced_steps is None else np.asarray(forced_steps).reshape(S, T)
    if warm_start and solve_at is not None:
        raise ValueError("warm start needs every token solved")
    if warm_lag < 1 or (warm_chunk is not None and (warm_chunk < 1 or x_init is not None)):
        raise ValueError("warm_lag >= 1; warm_chunk >= 1 and takes no x_init")
    x_prev = np.zeros((S, dk)) if x_init is None else _flat(x_init, S, dk).copy()

    o_cg = np.zeros((S, T, dv))
    x_cg = np.zeros((S, T, dk))
    steps = np.zeros((S, T), dtype=np.int64)
    res_norm = np.zeros((S, T))
    res_prev = np.zeros((S, T))
    res_hist = np.zeros((S, T, int(max_steps) + 1)) if residual_history else None
    o_ex = np.zeros((S, T, dv)) if exact else None
    x_ex = np.zeros((S, T, dk)) if exact else None
    states = []
    for t in range(T):
        kt = kf[:, t]
        g_t = gf[:, t][:, None, None]
        b_t = bf[:, t][:, None, None]
        # state update; k_i*k_j is formed first so H stays exactly symmetric
        Hs = g_t * Hs + b_t * (kt[:, :, None] * kt[:, None, :])
        Gs = g_t * Gs + b_t * (vf[:, t][:, :, None] * kt[:, None, :])
        if solve_at is not None and not solve_at[t]:
            if record_every and ((t + 1) % record_every == 0 or t == T - 1):
                states.append((t + 1, Hs.reshape(B, Hh, dk, dk).copy(),
                               Gs.reshape(B, Hh, dv, dk).copy()))
            continue
        A = Hs + Lam
        x0 = None
        if warm_start:
            if warm_lag == 1 and warm_chunk is None:
                x0 = x_prev
            elif t - warm_lag >= 0 and (warm_chunk is None or (t - warm_lag) // warm_chunk == t // warm_chunk):
                x0 = x_cg[:, t - warm_lag]
        xs, ns, rn, rp, rh = cg_solve(A, qf[:, t], max_steps, tol,
                                      None if fs is None else fs[:, t], residuals=True,
                                      x0=x0, history=True)
        if residual_history:
            res_hist[:, t] = rh
        x_prev = xs
        x_cg[:, t] = xs
        steps[:, t] = ns
        res_norm[:, t] = rn
        res_prev[:, t] = rp
        o_cg[:, t] = np.matmul(Gs, xs[:, :, None])[:, :, 0]
        if exact:
            xe = cholesky_solve(A, qf[:, t])
            x_ex[:, t] = xe
            o_ex[:, t] = np.matmul(Gs, xe[:, :, None])[:, :, 0]
        if record_every and ((t + 1) % record_every == 0 or t == T - 1):
            states.append((t + 1, Hs.reshape(B, Hh, dk, dk).copy(),
                           Gs.reshape(B, Hh, dv, dk).copy()))
    out = dict(
        o_cg=o_cg.reshape(B, Hh, T, dv),
        x_cg=x_cg.reshape(B, Hh, T, dk),
        steps=steps.reshape(B, Hh, T),
        res_norm=res_norm.reshape(B, Hh, T),
        res_prev=res_prev.reshape(B, Hh, T),
        H_final=Hs.reshape(B, Hh, dk, dk),
        G_final=Gs.reshape(B, Hh, dv, dk),
        states=states,
    )
    if residual_history:
        out["res_hist"] = res_hist.reshape(B, Hh, T, -1)
    if exact:
        out["o_exact"] = o_ex.reshape(B, Hh, T, dv)
        out["x_exact"] = x_ex.reshape(B, Hh, T, dk)
    return out


def mesa_decode_step(q, k, v, gamma, beta, lam, h, g, *, max_steps: int, tol: float,
                     forced_steps=None, exact: bool = False, x0=None):
    """One recurrent step for N sequences x H heads, fp64.

    q, k: [N, H, dk]; v: [N, H, dv]; gamma, beta: [N, H]; lam: [H, dk] or
    [H, dk, dk]; h: [N, H, dk, dk]; g: [N, H, dv, dk] (not modified).
    x0: optional [N, H, dk] warm start of the CG (the previous token's
    solution); default: CG from 0.
    Returns dict(o, x, steps, h, g[, o_exact]) for the new token.
    """
    q = np.asarray(q, dtype=np.float64)
    N, Hh, dk = q.shape
    dv = np.asarray(v).shape[-1]
    res = mesa_forward(q[:, :, None], np.asarray(k)[:, :, None], np.asarray(v)[:, :, None],
                       np.asarray(gamma)[:, :, None], np.asarray(beta)[:, :, None], lam,
                       max_steps=max_steps, tol=tol, h0=h, g0=g,
                       forced_steps=None if forced_steps is None
                       else np.asarray(forced_steps).reshape(N, Hh, 1),
                       exact=exact, warm_start=x0 is not None, x_init=x0, residual_history=True)
    out = dict(o=res["o_cg"][:, :, 0], x=res["x_cg"][:, :, 0], steps=res["steps"][:, :, 0],
               res_norm=res["res_norm"][:, :, 0], res_prev=res["res_prev"][:, :, 0],
               res_hist=res["res_hist"][:, :, 0], h=res["H_final"], g=res["G_final"])
    if exact:
        out["o_exact"] = res["o_exact"][:, :, 0]
    return out


def qk_preprocess(x, w, hist=None, eps: float = 1e-6):
    """Query/key preprocessing before the layer, fp64.

    The architecture section has queries and keys normalised and convolved
    with a small window before the Mesa layer.  Reading: a causal convolution
    along time with its own taps per channel (depthwise), then L2
    normalisation of each token vector, so the layer receives unit-norm
    queries and keys:
        y_t[j] = sum_{i < W} w[h, j, i] * x_{t-i}[j]
        out_t  = y_t / max(||y_t||_2, eps)
    x: [B, H, T, d] raw vectors; w: [H, d, W] taps (tap i weighs token t-i);
    hist: optional [B, H, W-1, d] raw vectors before t = 0, oldest first
    (default: zeros).  Returns (out [B, H, T, d], hist_out [B, H, W-1, d]:
    the last W-1 raw vectors, oldest first -- the history of the next call).
    """
    x = np.asarray(x, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    B, Hh, T, d = x.shape
    W = w.shape[-1]
    pre = np.zeros((B, Hh, W - 1, d)) if hist is None else np.asarray(hist, dtype=np.float64)
    seq = np.concatenate([pre, x], axis=2)      # token t sits at index t + W - 1
    y = np.zeros((B, Hh, T, d))
    for i in range(W):
        y += w[None, :, None, :, i] * seq[:, :, W - 1 - i:W - 1 - i + T]
    nrm = np.linalg.norm(y, axis=-1, keepdims=True)
    out = y / np.maximum(nrm, eps)
    return out, seq[:, :, T:]


def mesa_backward(q, k, v, gamma, beta, lam, d_o, *, max_steps: int, tol: float,
                  h0=None, g0=None, dh_final=None, dg_final=None, forced_steps=None,
                  adjoint_forced_steps=None, exact: bool = False, chunk: int = 64):
    """Gradients of the layer by implicit differentiation of its solves, fp64.

    The scalar differentiated is L = sum_t <d_o_t, o_t> + <dh_final, H_T> +
    <dg_final, G_T> (H_T, G_T: the states after the last token).  Each
    x_t = (H_t + Lambda)^{-1} q_t is treated as the solution of its system, so
    with the adjoint y_t = (H_t + Lambda)^{-1} G_t^T d_o_t:
        dL/dq_t = y_t,  dL/dH_t (local) = -y_t x_t^T,  dL/dG_t (local) = d_o_t x_t^T,
        dL/dlambda = -sum_t y_t * x_t  (diagonal Lambda [H, dk], summed over batch and time),
        dL/dLambda = -sum_t y_t x_t^T  (a full Lambda [H, dk, dk]: the partial derivative
                     of each entry, not symmetrised; its diagonal is the diagonal case).
    The state adjoints run backwards, Hhat_t = dH_t + gamma_{t+1} Hhat_{t+1}
    (Hhat_T starts at dh_final; the same for G), and give
        dk_t = beta_t ((Hhat_t + Hhat_t^T) k_t + Ghat_t^T v_t),  dv_t = beta_t Ghat_t k_t,
        dbeta_t = k_t^T Hhat_t k_t + v_t^T Ghat_t k_t,
        dgamma_t = <Hhat_t, H_{t-1}> + <Ghat_t, G_{t-1}>,
        dh0 = gamma_0 Hhat_0 (symmetrised: h0 is a symmetric state),  dg0 = gamma_0 Ghat_0.
    x_t and y_t come from exact solves (``exact``) or from the CG schedule:
    x_t as in :func:`mesa_forward` (``forced_steps`` as there); y_t by CG with
    the same max_steps, and the tolerance taken relative to ||G_t^T d_o_t||
    (CG on the normalised right-hand side, rescaled), optionally forced to
    ``adjoint_forced_steps`` [B, H, T].  The states are checkpointed every
    ``chunk`` tokens and recomputed chunk by chunk on the way back.

    Returns dict(dq, dk, dv [B,H,T,d], dgamma, dbeta [B,H,T], dlam [H,dk] or [H,dk,dk],
    dh0 [B,H,dk,dk], dg0 [B,H,dv,dk], x, y [B,H,T,dk], adj_steps [B,H,T]).
    """
    q = np.asarray(q, dtype=np.float64)
    B, Hh, T, dk = q.shape
    dv = np.asarray(v).shape[-1]
    S = B * Hh
    qf, kf = _flat(q, S, T, dk), _flat(k, S, T, dk)
    vf, of = _flat(v, S, T, dv), _flat(d_o, S, T, dv)
    gf, bf = _flat(gamma, S, T), _flat(beta, S, T)
    lam = np.asarray(lam, dtype=np.float64)
    full = lam.shape == (Hh, dk, dk)
    if not full and lam.shape != (Hh, dk):
        raise ValueError("the backward takes Lambda as a diagonal [H, dk] or a full [H, dk, dk]")
    fs = None if forced_steps is None else np.asarray(forced_steps).reshape(S, T)
    fa = None if adjoint_forced_steps is None else np.asarray(adjoint_forced_steps).reshape(S, T)
    out = {name: np.zeros((S, T, dd)) for name, dd in (("dq", dk), ("dk", dk), ("dv", dv),
                                                         ("x", dk), ("y", dk))}
    out.update(dgamma=np.zeros((S, T)), dbeta=np.zeros((S, T)), adj_steps=np.zeros((S, T), np.int64),
               dh0=np.zeros((S, dk, dk)), dg0=np.zeros((S, dv, dk)))
    dlam = np.zeros((Hh, dk, dk) if full else (Hh, dk))
    NC = (T + chunk - 1) // chunk
    for s_ in range(S):
        h = s_ % Hh
        Lam = lam[h] if full else np.diag(lam[h])
        Hs = np.zeros((dk, dk)) if h0 is None else _flat(h0, S, dk, dk)[s_].copy()
        Gs = np.zeros((dv, dk)) if g0 is None else _flat(g0, S, dv, dk)[s_].copy()

        def step(Hm, Gm, t):
            kt = kf[s_, t]
            return (gf[s_, t] * Hm + bf[s_, t] * (kt[:, None] * kt[None, :]),
                    gf[s_, t] * Gm + bf[s_, t] * (vf[s_, t][:, None] * kt[None, :]))

        # forward: checkpoints at chunk starts, and the solutions x_t
        ckpt = []
        for t in range(T):
            if t % chunk == 0:
                ckpt.append((Hs.copy(), Gs.copy()))
            Hs, Gs = step(Hs, Gs, t)
            A = Hs + Lam
            if exact:
                xt = cholesky_solve(A[None], qf[s_, t][None])[0]
            else:
                xs_, _ = cg_solve(A[None], qf[s_, t][None], max_steps, tol,
                                  None if fs is None else fs[s_, t:t + 1])
                xt = xs_[0]
            out["x"][s_, t] = xt
        # backward, chunk by chunk from the end
        Hhat = np.zeros((dk, dk)) if dh_final is None else _flat(dh_final, S, dk, dk)[s_].astype(np.float64).copy()
        Ghat = np.zeros((dv, dk)) if dg_final is None else _flat(dg_final, S, dv, dk)[s_].astype(np.float64).copy()
        for c in range(NC - 1, -1, -1):
            t0, t1 = c * chunk, min(T, (c + 1) * chunk)
            Hm, Gm = ckpt[c]
            states = [(Hm, Gm)]                 # states[i] = (H, G) before token t0 + i
            for t in range(t0, t1):
                states.append(step(*states[-1], t))
            for t in range(t1 - 1, t0 - 1, -1):
                Ht, Gt = states[t - t0 + 1]
                Hp, Gp = states[t - t0]
                xt, kt, vt, dot = out["x"][s_, t], kf[s_, t], vf[s_, t], of[s_, t]
                A = Ht + Lam
                dxt = Gt.T @ dot
                if exact:
                    yt = cholesky_solve(A[None], dxt[None])[0]
                    na = 0
                else:
                    nrm = np.linalg.norm(dxt)
                    if nrm > 0:
                        ys_, ns_ = cg_solve(A[None], (dxt / nrm)[None], max_steps, tol,
                                            None if fa is None else fa[s_, t:t + 1])
                        yt, na = ys_[0] * nrm, int(ns_[0])
                    else:
                        yt, na = np.zeros(dk), 0
                out["y"][s_, t] = yt
                out["adj_steps"][s_, t] = na
                out["dq"][s_, t] = yt
                if full:
                    dlam[h] -= np.outer(yt, xt)
                else:
                    dlam[h] -= yt * xt
                Hhat = Hhat - np.outer(yt, xt)
                Ghat = Ghat + np.outer(dot, xt)
                bt = bf[s_, t]
                out["dk"][s_, t] = bt * ((Hhat + Hhat.T) @ kt + Ghat.T @ vt)
                out["dv"][s_, t] = bt * (Ghat @ kt)
                out["dbeta"][s_, t] = kt @ Hhat @ kt + vt @ Ghat @ kt
                out["dgamma"][s_, t] = np.sum(Hhat * Hp) + np.sum(Ghat * Gp)
                Hhat = gf[s_, t] * Hhat
                Ghat = gf[s_, t] * Ghat
        out["dh0"][s_] = 0.5 * (Hhat + Hhat.T)
        out["dg0"][s_] = Ghat
    res = {key: val.reshape(B, Hh, *val.shape[1:]) for key, val in out.items()}
    res["dlam"] = dlam
    return res
