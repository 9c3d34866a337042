"""Shared test utilities: moving seeded inputs to the GPU and error metrics."""
import numpy as np
import torch


def rel_l2(a, b) -> float:
    """||a - b||_F / ||b||_F in fp64 (1.0 denominator when b == 0)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def dev_inputs(x: dict, device="cuda") -> dict:
    """torch device tensors of a generator dict (bf16 q/k/v when the config is bf16)."""
    cfg = x["cfg"]
    qkv_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device).to(qkv_dtype).contiguous()
    for key in ("gamma", "beta", "lam"):
        out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device, dtype=torch.float32)
    for key in ("h", "g"):
        if key in x:
            out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device, dtype=torch.float32)
    if cfg.dtype == "bf16":
        # the device values must be exactly the generator's (bf16-representable) values
        for key in ("q", "k", "v"):
            assert torch.equal(out[key].float().cpu(), torch.from_numpy(x[key]))
    return out


def slice_inputs(x: dict, idx) -> dict:
    """The (b, h) slices idx (flattened b*H + h) of a forward workload, as a B=len(idx), H=1 batch."""
    cfg = x["cfg"]
    B, H = cfg.B, cfg.H
    b = np.asarray(idx) // H
    h = np.asarray(idx) % H
    out = {}
    for key in ("q", "k", "v"):
        out[key] = x[key][b, h][:, None]
    for key in ("gamma", "beta"):
        out[key] = x[key][b, h][:, None]
    return out, h


def oracle_on_slices(x: dict, idx, steps_gpu=None, exact=False, solve_at=None, **kw):
    """Run the oracle on selected (b, h) slices; lambda follows each slice's head."""
    from oracle import mesa_forward
    sl, heads = slice_inputs(x, idx)
    cfg = x["cfg"]
    res = []
    for i, hh in enumerate(heads):
        fs = None if steps_gpu is None else steps_gpu[i][None, None]
        r = mesa_forward(sl["q"][i:i + 1], sl["k"][i:i + 1], sl["v"][i:i + 1],
                         sl["gamma"][i:i + 1], sl["beta"][i:i + 1], x["lam"][hh:hh + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=fs, exact=exact,
                         solve_at=solve_at, **kw)
        res.append(r)
    return res


# Stopping decisions of dynamic CG (MesaNet page, "Mesa layer", dynamic compute:
# the step count follows a stopping criterion and varies per token).  Step counts
# near the threshold are not unique in finite precision, so a GPU stop is checked
# against the fp64 oracle's recursive residuals after the same number of steps:
#   * no premature stop: a stop before the cap needs ||r_n|| <= tol (1 + eps);
#   * at most one step past the fp64 run's own crossing: ||r_{n-2}|| > tol.
# A lower-precision CG converges later, never earlier, than the exact one: its
# rounding disturbs the orthogonality of the directions, most visibly when
# H + Lambda has an isolated large eigenvalue (a key written several times).
# fp32 CG on such a system can sit at 1.4 tol where fp64 sits at 0.5 tol after
# the same 11 steps, so a band on ||r_{n-1}|| would reject correct arithmetic;
# the delay is one step.  eps bounds the premature direction: fp32 arithmetic
# 0.05; bf16 MFMA operands (relative rounding 2^-9 per operand) 0.25.
EPS_STOP = {"f32": 0.05, "bf16": 0.25}


def check_stops(n, res_hist, max_steps, tol, kind):
    """Check every token's stop; n: [N] GPU step counts, res_hist: [N, max_steps + 1]
    oracle residual norms after each step of a run forced to n.  Returns a report:
    the histogram of n_gpu - n_oracle (the fp64 run's own count under the same
    tolerance, which coincides with the forced run up to n_gpu; a token the fp64
    run would take past n_gpu counts as -1), and the extreme residual ratios."""
    eps = EPS_STOP[kind]
    n = np.asarray(n).ravel().astype(np.int64)
    hist = np.asarray(res_hist, dtype=np.float64).reshape(n.size, -1)
    N = n.size
    ar = np.arange(N)
    r_n = hist[ar, n]
    assert np.all(np.isfinite(r_n)), "oracle residual history shorter than the GPU's step counts"
    early = n < max_steps
    bad = early & ~(r_n <= tol * (1 + eps))
    assert not bad.any(), f"premature stops: {list(zip(ar[bad][:8], n[bad][:8], (r_n[bad] / tol)[:8]))}"
    r_nm2 = np.where(n >= 2, hist[ar, np.maximum(n - 2, 0)], np.inf)
    bad = ~(r_nm2 > tol)
    assert not bad.any(), f"two steps past convergence: {list(zip(ar[bad][:8], n[bad][:8], (r_nm2[bad] / tol)[:8]))}"
    took = n >= 1
    r_nm1 = hist[ar, np.maximum(n - 1, 0)]
    below = np.nan_to_num(hist, nan=np.inf) <= tol
    below &= np.arange(hist.shape[1])[None, :] <= n[:, None]
    first = np.where(below.any(axis=1), below.argmax(axis=1), np.minimum(n + 1, max_steps))
    vals, cnts = np.unique(n - first, return_counts=True)
    return dict(n_minus_oracle={int(v): int(c) for v, c in zip(vals, cnts)},
                max_stop_ratio=float((r_n[early] / tol).max()) if early.any() else None,
                min_prev_ratio=float((r_nm1[took] / tol).min()) if took.any() else None,
                early=int(early.sum()), tokens=N)


def true_residual(A, x, q):
    """||A x - q||_2 per system in fp64 (A: [N, d, d], x, q: [N, d])."""
    A = np.asarray(A, dtype=np.float64)
    return np.linalg.norm(np.matmul(A, np.asarray(x, np.float64)[:, :, None])[:, :, 0] - np.asarray(q, np.float64),
                          axis=-1)
