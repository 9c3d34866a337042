"""Chunked forward with a full symmetric positive definite Lambda per head.

The pages' objective regularises with a symmetric positive definite Lambda;
the oracle's forward takes it as a full matrix.  ``mesa_fwd_chunked_ex``
with ``lambda_full = 1`` is checked against the oracle at the GPU's step
counts: fixed and dynamic step counts, d = 64 and 128, ragged last chunks,
chunks decaying strongly enough for the unscaled kernel, and a sampled slice
of the LM-shaped workload.  A diagonal Lambda given as a full matrix must
agree with the diagonal path, and ``lambda_full = 0`` must be the diagonal
path itself.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs, oracle_on_slices, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_full_lambda, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu

TOL_BF16 = 2e-2


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def with_full_lambda(x):
    cfg = x["cfg"]
    return dict(x, lam=make_full_lambda(cfg.H, cfg.d, cfg.seed))


def fwd_ex(x, **kw):
    cfg = x["cfg"]
    d = dev_inputs(x)
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_steps=True)
    args.update(kw)
    res = mesa.fwd_chunked_ex(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **args)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def check(x, r, idx):
    cfg = x["cfg"]
    steps = r["steps"].reshape(cfg.B * cfg.H, cfg.T)[idx]
    refs = oracle_on_slices(x, idx, steps_gpu=steps)
    o_ref = np.stack([rr["o_cg"][0, 0] for rr in refs])
    x_ref = np.stack([rr["x_cg"][0, 0] for rr in refs])
    o = r["o"].reshape(cfg.B * cfg.H, cfg.T, cfg.d)[idx]
    e_o = rel_l2(o, o_ref)
    assert e_o <= TOL_BF16, e_o
    if "x" in r:
        e_x = rel_l2(r["x"].reshape(cfg.B * cfg.H, cfg.T, cfg.d)[idx], x_ref)
        assert e_x <= TOL_BF16, e_x
    return refs, e_o


@pytest.mark.parametrize("d,T,max_steps,tol", [(64, 200, 8, 0.0), (128, 130, 8, 0.0),
                                                (128, 257, 32, 1e-4), (64, 64, 32, 1e-4)])
def test_full_lambda_matches_oracle(d, T, max_steps, tol):
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol)
    x = with_full_lambda(make_fwd_inputs(cfg))
    r = fwd_ex(x, return_x=True, return_state=True)
    n = r["steps"]
    assert n.min() >= 1 and n.max() <= max_steps
    if tol == 0.0:
        assert np.all(n == max_steps)
    refs, err = check(x, r, [0, 1])
    # the states carried out are H and G alone: Lambda only enters the solves
    Hr = np.stack([rr["H_final"][0, 0] for rr in refs])
    Gr = np.stack([rr["G_final"][0, 0] for rr in refs])
    assert rel_l2(r["h_final"].reshape(2, d, d), Hr) < 1e-4
    assert rel_l2(r["g_final"].reshape(2, d, d), Gr) < 1e-4
    print(f"full Lambda d={d} T={T} steps<={max_steps}: rel L2 {err:.2e}, mean steps {n.mean():.2f}")


@pytest.mark.parametrize("d", [64, 128])
def test_full_lambda_strong_decay_chunks(d):
    """Chunks decaying past e^-40 are solved by the unscaled kernel, mixed with normal ones."""
    chunk = 64
    cfg = small_fwd(B=1, H=2, T=5 * chunk - 7, d=d, chunk=chunk, dtype="bf16", max_steps=8)
    x = with_full_lambda(make_fwd_inputs(cfg))
    g = x["gamma"].copy()
    for c in (1, 3):
        g[:, :, c * chunk:(c + 1) * chunk] = np.float32(0.3)
    g[:, 1, 4 * chunk:] = np.float32(0.05)
    x = dict(x, gamma=g)
    r = fwd_ex(x, return_x=True)
    refs, _ = check(x, r, [0, 1])
    o_ref = np.stack([rr["o_cg"][0, 0] for rr in refs])
    o = r["o"].reshape(2, cfg.T, d)
    for c in range(5):
        sl = slice(c * chunk, min((c + 1) * chunk, cfg.T))
        e = rel_l2(o[:, sl], o_ref[:, sl])
        assert e <= TOL_BF16, (c, e)


def test_diagonal_given_as_full_matrix():
    """A diagonal Lambda as a full matrix agrees with the diagonal path (which
    keeps Lambda in fp32 where the full path rounds it to bf16), and
    lambda_full = 0 runs the diagonal path itself."""
    cfg = small_fwd(B=1, H=2, T=190, d=128, chunk=64, dtype="bf16", max_steps=10)
    x = make_fwd_inputs(cfg)
    d = dev_inputs(x)
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol)
    r_diag = mesa.fwd_chunked(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **args)
    r_ex0 = mesa.fwd_chunked_ex(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **args)
    lam_full = torch.diag_embed(d["lam"]).contiguous()
    r_full = mesa.fwd_chunked_ex(d["q"], d["k"], d["v"], d["gamma"], d["beta"], lam_full, **args)
    torch.cuda.synchronize()
    assert torch.equal(r_diag["o"], r_ex0["o"])
    e = rel_l2(r_full["o"].cpu().numpy(), r_diag["o"].cpu().numpy())
    assert e < 1e-2, e


def test_lm_shape_sampled_slice():
    """The LM-shaped workload (B8 H16 T4096 d128, 30 fixed steps) with a full
    Lambda, in the launch the benchmark times; one (b, h) slice against the
    oracle."""
    cfg = CONFIGS[3]
    x = with_full_lambda(make_fwd_inputs(cfg))
    r = fwd_ex(x)
    assert np.all(r["steps"] == cfg.max_steps)
    assert np.isfinite(r["o"]).all()
    _, err = check(x, r, [cfg.B * cfg.H - 1])
    print(f"LM shape, full Lambda: slice rel L2 {err:.2e}")
