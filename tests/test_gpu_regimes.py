"""Regimes outside the workloads' distributions (needs an MI355X).

* Fixed step counts past convergence.  With a constant Lambda a system can
  have few distinct eigenvalues (the first tokens of a sequence have a
  low-rank H), so CG reaches rounding level in a few steps.  In the fixed-step
  mode the loop goes on, and the recursive residual keeps shrinking until
  r.r underflows; every CG loop counts r.r and p.(A p) below the smallest
  normal float as zero and stops the token there (a reciprocal of such a value
  is not finite).  Outputs must stay finite and match the oracle at the GPU's
  step counts, in every kernel: the scaled and unscaled bf16 solves, the warm
  start, the full-Lambda solve, the fp32 path, the decode step and the
  backward's adjoint solves.
* No forgetting (gamma = 1 exactly): the page's objective without decay, the
  prefix ridge regression the oracle is pinned to.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_bwd_inputs, make_decode_inputs, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


@pytest.mark.parametrize("dtype,d,variant,gates", [
    ("bf16", 128, "plain", (2.0, 6.0)),
    ("bf16", 64, "plain", (2.0, 6.0)),
    ("bf16", 128, "plain", (-3.0, 1.0)),   # every chunk decays past e^-40: the unscaled kernel
    ("bf16", 128, "warm", (2.0, 6.0)),
    ("bf16", 128, "lfull", (2.0, 6.0)),
    ("f32", 64, "plain", (2.0, 6.0)),
])
def test_fixed_steps_past_convergence_stay_finite(dtype, d, variant, gates):
    from oracle import mesa_forward
    cfg = small_fwd(B=1, H=2, T=256, d=d, chunk=64, dtype=dtype, max_steps=30, tol=0.0, seed=77,
                    lam=("const", 1.0), gamma_logit=gates)
    x = make_fwd_inputs(cfg)
    a = dev_inputs(x)
    kw = dict(chunk=64, max_steps=30, tol=0.0, return_x=True)
    if variant == "lfull":
        lam = np.broadcast_to(np.eye(d, dtype=np.float32), (cfg.H, d, d)).copy()
        r = mesa.fwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], torch.from_numpy(lam).cuda(), **kw)
    else:
        lam = x["lam"]
        r = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], warm=variant == "warm", **kw)
    torch.cuda.synchronize()
    o, xs, n = r["o"].cpu().numpy(), r["x"].cpu().numpy(), r["steps"].cpu().numpy()
    assert np.isfinite(o).all() and np.isfinite(xs).all()
    assert (n < 30).any(), "no token reached rounding level: the case does not test the floor"
    warm = dict(warm_start=True, warm_lag=16, warm_chunk=64) if variant == "warm" else {}
    ref = mesa_forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, max_steps=30, tol=0.0,
                       forced_steps=n, exact=False, **warm)
    assert np.array_equal(ref["steps"], n)
    err = rel_l2(o, ref["o_cg"])
    print(f"{dtype} d={d} {variant}: tokens stopped at the floor {(n < 30).mean():.3f}, rel L2 {err:.2e}")
    assert err <= TOL[dtype]


@pytest.mark.parametrize("dtype,packed", [("bf16", False), ("bf16", True), ("f32", False)])
def test_decode_fixed_steps_past_convergence(dtype, packed):
    """A rank-one H (no prefix) and Lambda = I: two distinct eigenvalues."""
    from oracle import mesa_decode_step
    cfg = CONFIGS[5].replace(N=16, H=2, prefill=0, dtype=dtype, lam_dist=("const", 1.0), max_steps=32, tol=0.0)
    x = make_decode_inputs(cfg)
    a = dev_inputs(x)
    h = mesa.sym_pack(a["h"]) if packed else a["h"]
    r = mesa.decode_step_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], h, a["g"], packed_h=packed,
                            max_steps=32, tol=0.0)
    torch.cuda.synchronize()
    o, n = r["o"].cpu().numpy(), r["steps"].cpu().numpy()
    assert np.isfinite(o).all()
    print(f"decode {dtype} packed={packed}: pairs stopped at the floor {(n < 32).mean():.3f}, steps {np.bincount(n.ravel())}")
    ref = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], x["h"], x["g"],
                           max_steps=32, tol=0.0, forced_steps=n)
    assert rel_l2(o, ref["o"]) <= 1e-4


def test_backward_fixed_steps_past_convergence():
    from oracle import mesa_backward
    cfg = small_fwd(B=1, H=2, T=200, d=128, chunk=64, dtype="bf16", max_steps=30, tol=0.0, seed=78,
                    lam=("const", 1.0))
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    a = dev_inputs(x)
    t = {k: torch.from_numpy(v).cuda() for k, v in g.items()}
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=64, max_steps=30, tol=0.0,
                         return_x=True, h0=t["h0"], g0=t["g0"])
    b = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], t["d_o"], chunk=64,
                         max_steps=30, tol=0.0, h0=t["h0"], g0=t["g0"], d_hfinal=t["d_hfinal"],
                         d_gfinal=t["d_gfinal"], state_grads=True, return_steps=True)
    torch.cuda.synchronize()
    gpu = {k: v.cpu().numpy() for k, v in b.items()}
    for k, v in gpu.items():
        assert np.isfinite(v).all(), k
    ref = mesa_backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], g["d_o"], max_steps=30, tol=0.0,
                        h0=g["h0"], g0=g["g0"], dh_final=g["d_hfinal"], dg_final=g["d_gfinal"],
                        forced_steps=f["steps"].cpu().numpy(), adjoint_forced_steps=gpu["adj_steps"], chunk=64)
    errs = {k: rel_l2(gpu[k], ref[k]) for k in ("dq", "dk", "dv", "dgamma", "dbeta", "dlam", "dh0", "dg0")}
    assert all(e <= 2e-2 for e in errs.values()), errs


@pytest.mark.parametrize("d,max_steps,tol", [(128, 30, 0.0), (128, 64, 1e-4), (64, 30, 0.0)])
def test_no_forgetting(d, max_steps, tol):
    """gamma = sigmoid(u), u in (20, 30), is exactly 1.0 in fp32: no decay at all."""
    from oracle import mesa_forward
    cfg = small_fwd(B=1, H=2, T=300, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol, seed=79,
                    gamma_logit=(20.0, 30.0))
    x = make_fwd_inputs(cfg)
    assert np.all(x["gamma"] == 1.0)
    a = dev_inputs(x)
    r = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=64, max_steps=max_steps,
                         tol=tol, return_state=True)
    torch.cuda.synchronize()
    n = r["steps"].cpu().numpy()
    ref = mesa_forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], max_steps=max_steps, tol=tol,
                       forced_steps=n, exact=False)
    assert rel_l2(r["o"].cpu().numpy(), ref["o_cg"]) <= TOL["bf16"]
    assert rel_l2(r["h_final"].cpu().numpy(), ref["H_final"]) < 1e-4
    assert rel_l2(r["g_final"].cpu().numpy(), ref["G_final"]) < 1e-4
