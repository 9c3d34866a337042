"""Warm-started decode step: CG begins at the pair's previous solution.

Checked against the oracle's warm-started recurrence (token t's CG starts at
token t-1's result) over several steps in a row, at the step counts the GPU
took, plus the cases that pin the start itself: a zero start is the cold
step, the exact solution as the start takes no step, zero steps return the
start.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_decode_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def token_stream(cfg, T):
    """Start states and T new tokens: token 0 and the states from make_decode_inputs(cfg),
    tokens 1.. from the same generator at the next seeds (their states unused); lambda
    is token 0's."""
    x0 = make_decode_inputs(cfg)
    toks = [x0] + [make_decode_inputs(cfg.replace(seed=cfg.seed + 100 + i, prefill=0)) for i in range(1, T)]
    seq = {key: np.stack([t[key] for t in toks], axis=2) for key in ("q", "k", "v", "gamma", "beta")}
    return x0, toks, seq


def step_inputs(tok, lam, cfg):
    d = dev_inputs(dict(tok, cfg=cfg))
    d["lam"] = torch.from_numpy(lam).cuda()
    return d


@pytest.mark.parametrize("dtype,d,packed", [("bf16", 128, False), ("bf16", 128, True), ("f32", 64, False),
                                            ("bf16", 64, True)])
def test_warm_sequence_matches_oracle(dtype, d, packed):
    from oracle import mesa_forward
    cfg = CONFIGS[5].replace(N=8, H=4, d=d, prefill=200, dtype=dtype)
    T = 5
    x0, toks, seq = token_stream(cfg, T)
    h = torch.from_numpy(x0["h"]).cuda()
    g = torch.from_numpy(x0["g"]).cuda()
    hs = mesa.sym_pack(h) if packed else h
    xs = torch.zeros((cfg.N, cfg.H, d), device="cuda")
    os_, ns, xouts = [], [], []
    for t in range(T):
        a = step_inputs(toks[t], x0["lam"], cfg)
        r = mesa.decode_step_warm(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], hs, g, xs,
                                  packed_h=packed, max_steps=cfg.max_steps, tol=cfg.tol)
        torch.cuda.synchronize()
        os_.append(r["o"].cpu().numpy())
        ns.append(r["steps"].cpu().numpy())
        xouts.append(xs.cpu().numpy())
    steps = np.stack(ns, axis=2)
    assert steps.max() > 0
    ref = mesa_forward(seq["q"], seq["k"], seq["v"], seq["gamma"], seq["beta"], x0["lam"],
                       max_steps=cfg.max_steps, tol=cfg.tol, h0=x0["h"], g0=x0["g"], exact=False,
                       warm_start=True, forced_steps=steps, residual_history=True)
    for t in range(T):
        assert rel_l2(os_[t], ref["o_cg"][:, :, t]) <= 1e-4, t
        assert rel_l2(xouts[t], ref["x_cg"][:, :, t]) <= 1e-4, t
    # every stop against the oracle's residuals at the GPU's count (fp32 arithmetic)
    check_stops(steps, ref["res_hist"], cfg.max_steps, cfg.tol, "f32")


@pytest.mark.parametrize("packed", [False, True])
def test_zero_start_is_the_cold_step(packed):
    cfg = CONFIGS[5].replace(N=8, H=4, d=128, prefill=200)
    x = make_decode_inputs(cfg)
    a, b = dev_inputs(x), dev_inputs(x)
    ha = mesa.sym_pack(a["h"]) if packed else a["h"]
    hb = mesa.sym_pack(b["h"]) if packed else b["h"]
    cold = (mesa.decode_step_symh if packed else mesa.decode_step)(
        a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], ha, a["g"],
        max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    xs = torch.zeros((cfg.N, cfg.H, cfg.d), device="cuda")
    warm = mesa.decode_step_warm(b["q"], b["k"], b["v"], b["gamma"], b["beta"], b["lam"], hb, b["g"], xs,
                                 packed_h=packed, max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    assert torch.equal(warm["o"], cold["o"])
    assert torch.equal(warm["steps"], cold["steps"])
    assert torch.equal(xs, cold["x"])
    assert torch.equal(hb, ha) and torch.equal(b["g"], a["g"])


def test_exact_start_takes_no_step_and_zero_steps_return_the_start():
    from oracle import mesa_decode_step
    cfg = CONFIGS[5].replace(N=8, H=4, d=128, prefill=200)
    x = make_decode_inputs(cfg)
    ref = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], x["h"], x["g"],
                           max_steps=cfg.max_steps, tol=cfg.tol, exact=True)
    a = dev_inputs(x)
    # the exact solution (rounded to fp32) as the start: its residual is far below the tolerance
    xs = torch.from_numpy(np.linalg.solve(
        ref["h"] + np.eye(cfg.d) * x["lam"][None, :, None, :], x["q"][..., None])[..., 0].astype(np.float32)).cuda()
    x_start = xs.clone()
    r = mesa.decode_step_warm(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], a["h"], a["g"], xs,
                              max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    assert int(r["steps"].max()) == 0
    assert torch.equal(xs, x_start)
    assert rel_l2(r["o"].cpu().numpy(), ref["o_exact"]) <= 1e-5
    # zero steps: o = G_t x_0 for any start
    b = dev_inputs(x)
    rng = np.random.default_rng(3)
    start = rng.standard_normal((cfg.N, cfg.H, cfg.d)).astype(np.float32)
    xs2 = torch.from_numpy(start).cuda()
    r2 = mesa.decode_step_warm(b["q"], b["k"], b["v"], b["gamma"], b["beta"], b["lam"], b["h"], b["g"], xs2,
                               max_steps=0, tol=cfg.tol)
    torch.cuda.synchronize()
    ref0 = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], x["h"], x["g"],
                            max_steps=0, tol=cfg.tol, x0=start)
    assert int(r2["steps"].max()) == 0
    assert np.array_equal(xs2.cpu().numpy(), start)
    assert rel_l2(r2["o"].cpu().numpy(), ref0["o"]) <= 1e-5
