"""Backward pass with a full symmetric positive definite Lambda per head.

``mesa_bwd_chunked_ex`` with ``lambda_full = 1``: the adjoint solves take the
full matrix, and dLambda is the [H, d, d] partial derivative of each entry,
-sum_{b,t} y_t x_t^T.  Every gradient is compared with the fp64 oracle's
backward (which takes the full matrix, pinned by finite differences) at the
GPU's step counts for both solves, at the bf16 bar; a diagonal Lambda given
as a full matrix reproduces the diagonal backward's gradients, with dlambda
on the diagonal of dLambda.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_bwd_inputs, make_full_lambda, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dgamma", "dbeta", "dlam", "dh0", "dg0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def run_gpu(cfg, x, g, lam):
    a = dev_inputs(x)
    t = {key: torch.from_numpy(val).cuda() for key, val in g.items()}
    lam_d = torch.from_numpy(np.ascontiguousarray(lam)).cuda()
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, h0=t["h0"], g0=t["g0"])
    f = mesa.fwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_d, return_x=True, **args)
    b = mesa.bwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_d, f["x"], t["d_o"],
                            d_hfinal=t["d_hfinal"], d_gfinal=t["d_gfinal"], state_grads=True,
                            return_steps=True, **args)
    torch.cuda.synchronize()
    out = {key: val.cpu().numpy() for key, val in b.items()}
    out["steps"] = f["steps"].cpu().numpy()
    return out


@pytest.mark.parametrize("d,T,max_steps,tol,gates", [(64, 200, 10, 0.0, (2.0, 6.0)),
                                                     (128, 130, 32, 1e-4, (2.0, 6.0)),
                                                     (128, 150, 12, 0.0, (-3.0, 1.0))])
def test_full_lambda_gradients_match_oracle(d, T, max_steps, tol, gates):
    """The last case has strongly decaying gates (every chunk past e^-40: the
    unscaled full-Lambda kernel for every solve, and small gamma_t for dgamma)."""
    from oracle import mesa_backward
    cfg = small_fwd(B=2, H=2, T=T, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol, gamma_logit=gates)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    lam = make_full_lambda(cfg.H, d, cfg.seed)
    gpu = run_gpu(cfg, x, g, lam)
    assert gpu["dlam"].shape == (cfg.H, d, d)
    ref = mesa_backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, g["d_o"],
                        max_steps=cfg.max_steps, tol=cfg.tol, h0=g["h0"], g0=g["g0"],
                        dh_final=g["d_hfinal"], dg_final=g["d_gfinal"], forced_steps=gpu["steps"],
                        adjoint_forced_steps=gpu["adj_steps"], chunk=cfg.chunk)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in NAMES}
    print(f"full Lambda backward d={d} T={T}: " + ", ".join(f"{n} {e:.1e}" for n, e in errs.items()))
    assert all(e <= 2e-2 for e in errs.values()), errs


def test_diagonal_given_as_full_matrix_matches_the_diagonal_backward():
    cfg = small_fwd(B=1, H=2, T=150, d=128, chunk=64, dtype="bf16", max_steps=10)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    a = dev_inputs(x)
    t = {key: torch.from_numpy(val).cuda() for key, val in g.items()}
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol)
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], return_x=True, **args)
    bd = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], t["d_o"], **args)
    b0 = mesa.bwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], t["d_o"], **args)
    lam_full = torch.diag_embed(a["lam"]).contiguous()
    ff = mesa.fwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_full, return_x=True, **args)
    bf = mesa.bwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_full, ff["x"], t["d_o"], **args)
    torch.cuda.synchronize()
    for n in ("dq", "dk", "dv", "dgamma", "dbeta", "dlam"):
        assert torch.equal(bd[n], b0[n]), n        # lambda_full = 0 is the diagonal backward itself
    # Lambda rounded to bf16 on the full path: agreement at the bf16 level
    for n in ("dq", "dk", "dv", "dgamma", "dbeta"):
        e = rel_l2(bf[n].cpu().numpy(), bd[n].cpu().numpy())
        assert e < 2e-2, (n, e)
    diag = torch.diagonal(bf["dlam"], dim1=1, dim2=2)
    assert rel_l2(diag.cpu().numpy(), bd["dlam"].cpu().numpy()) < 2e-2
