"""Chunked forward with warm-started CG (mesa_fwd_chunked_warm) on the GPU.

Token t starts its CG from token t-16's solution when both lie in one chunk
(MesaNet page, "significance": warm-started optimisation), else from 0.  The
GPU's outputs, solutions and step counts are compared with the fp64 oracle
run with the same start rule (warm_lag = 16, warm_chunk = chunk) at the GPU's
step counts; with a tolerance every stop is checked against the oracle's
residual history.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, oracle_on_slices, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def run(x, cfg, warm):
    d = dev_inputs(x)
    r = mesa.fwd_chunked(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, return_x=True, return_state=True, warm=warm)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in r.items()}


@pytest.mark.parametrize("d,chunk,T,max_steps,tol,decay", [
    (128, 64, 200, 8, 0.0, False),     # three chunks and a ragged one
    (128, 64, 150, 32, 1e-4, False),   # dynamic steps
    (64, 32, 150, 32, 1e-4, False),
    (128, 64, 200, 10, 0.0, True),     # chunks decaying past e^-40: the unscaled kernel
    (64, 64, 130, 32, 1e-4, True),
])
def test_warm_forward_matches_oracle(d, chunk, T, max_steps, tol, decay):
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=chunk, dtype="bf16", max_steps=max_steps, tol=tol)
    x = make_fwd_inputs(cfg)
    if decay:
        g = x["gamma"].copy()
        g[:, :, chunk:2 * chunk] = np.float32(0.3)
        x = dict(x, gamma=g)
    gpu = run(x, cfg, True)
    steps = gpu["steps"].reshape(2, T)
    refs = oracle_on_slices(x, [0, 1], steps_gpu=steps, warm_start=True, warm_lag=16, warm_chunk=chunk,
                            residual_history=tol > 0)
    assert np.array_equal(np.stack([r["steps"][0, 0] for r in refs]), steps)
    o_ref = np.stack([r["o_cg"][0, 0] for r in refs])
    x_ref = np.stack([r["x_cg"][0, 0] for r in refs])
    eo = rel_l2(gpu["o"].reshape(2, T, d), o_ref)
    ex = rel_l2(gpu["x"].reshape(2, T, d), x_ref)
    assert eo <= 2e-2 and ex <= 2e-2, (eo, ex)
    if tol > 0:
        rep = [check_stops(steps[i], refs[i]["res_hist"][0, 0], max_steps, tol, "bf16") for i in range(2)]
        print(f"warm d={d} C={chunk}: rel L2 {eo:.2e}, stops {rep}")
    # the states do not depend on the start
    cold = run(x, cfg, False)
    assert np.array_equal(gpu["h_final"], cold["h_final"]) and np.array_equal(gpu["g_final"], cold["g_final"])
    # the first tile of every chunk starts cold: identical to the cold call there
    first = (np.arange(T) % chunk) < 16
    assert np.array_equal(gpu["o"][:, :, first], cold["o"][:, :, first])
    assert np.array_equal(gpu["steps"][:, :, first], cold["steps"][:, :, first])


def test_chunk_16_has_no_start_and_equals_the_cold_call():
    cfg = small_fwd(B=1, H=2, T=70, d=128, chunk=16, dtype="bf16", max_steps=20, tol=1e-4)
    x = make_fwd_inputs(cfg)
    w, c = run(x, cfg, True), run(x, cfg, False)
    for key in ("o", "x", "steps"):
        assert np.array_equal(w[key], c[key]), key


def test_slowly_varying_queries_take_fewer_steps():
    """Queries that drift slowly along the sequence (per-dimension AR(1), lag-1
    correlation 0.99): a start from token t-16's solution is close, so the
    warm run stops earlier, at the same outputs within the bf16 bar."""
    from test_regression_sequence_amd.inputs import make_slow_queries
    cfg = small_fwd(B=1, H=2, T=256, d=128, chunk=64, dtype="bf16", max_steps=64, tol=1e-4)
    x = make_slow_queries(make_fwd_inputs(cfg), 0.99)
    w, c = run(x, cfg, True), run(x, cfg, False)
    tiles = (np.arange(cfg.T) % cfg.chunk) >= 16
    nw, nc = w["steps"][:, :, tiles].mean(), c["steps"][:, :, tiles].mean()
    print(f"slow queries: mean steps cold {nc:.2f}, warm {nw:.2f}")
    assert nw < nc
    assert rel_l2(w["o"], c["o"]) < 2e-2
