"""Backward pass (implicit differentiation through the CG solves) on the GPU.

Every gradient is compared with the fp64 oracle's backward on the same
seeded inputs.  The oracle solves both systems by CG at the step counts the
GPU took (fixed steps, or the counts the GPU reports under a tolerance).  The
bar is the bf16 one (relative L2 <= 2e-2): the GPU's products use bf16
operands with fp32 accumulation, like its forward.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_bwd_inputs, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dgamma", "dbeta", "dlam", "dh0", "dg0")


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def run_gpu(cfg, x, g, with_states=True):
    a = dev_inputs(x)
    t = {key: torch.from_numpy(val).cuda() for key, val in g.items()}
    h0 = t["h0"] if with_states else None
    g0 = t["g0"] if with_states else None
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, h0=h0, g0=g0, return_x=True)
    b = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], t["d_o"],
                         chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, h0=h0, g0=g0,
                         d_hfinal=t["d_hfinal"] if with_states else None,
                         d_gfinal=t["d_gfinal"] if with_states else None,
                         state_grads=True, return_steps=True)
    torch.cuda.synchronize()
    out = {key: val.cpu().numpy() for key, val in b.items()}
    out["steps"] = f["steps"].cpu().numpy()
    return out


def run_oracle(cfg, x, g, gpu, with_states=True):
    from oracle import mesa_backward
    return mesa_backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], g["d_o"],
                         max_steps=cfg.max_steps, tol=cfg.tol,
                         h0=g["h0"] if with_states else None, g0=g["g0"] if with_states else None,
                         dh_final=g["d_hfinal"] if with_states else None,
                         dg_final=g["d_gfinal"] if with_states else None,
                         forced_steps=gpu["steps"], adjoint_forced_steps=gpu["adj_steps"], chunk=cfg.chunk)


@pytest.mark.parametrize("d,T,max_steps,tol,with_states", [
    (64, 200, 10, 0.0, True),      # three chunks and a ragged one
    (128, 192, 12, 0.0, True),
    (128, 130, 32, 1e-4, False),   # dynamic steps for both solves
    (64, 64, 8, 0.0, False),       # a single chunk
])
def test_gradients_match_oracle(d, T, max_steps, tol, with_states):
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    gpu = run_gpu(cfg, x, g, with_states)
    ref = run_oracle(cfg, x, g, gpu, with_states)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in NAMES}
    assert all(e <= 2e-2 for e in errs.values()), errs
    if tol > 0:
        assert gpu["adj_steps"].max() <= max_steps and gpu["adj_steps"].min() >= 1


@pytest.mark.parametrize("d,T,max_steps,tol", [(128, 200, 12, 0.0), (64, 150, 32, 1e-4)])
def test_strongly_decaying_gates(d, T, max_steps, tol):
    """gamma = sigmoid(U(-3, 1)) (0.05 to 0.73): every chunk decays past e^-40, so
    every forward and adjoint solve runs in the unscaled kernel, and dgamma_t is
    small-gamma sensitive (it is <Hhat_t, H_{t-1}> + <Ghat_t, G_{t-1}>, formed
    without dividing a cancellation by gamma_t)."""
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol,
                    gamma_logit=(-3.0, 1.0))
    x = make_fwd_inputs(cfg)
    assert float(np.log(x["gamma"][0, 0, :64]).sum()) < -40
    g = make_bwd_inputs(cfg)
    gpu = run_gpu(cfg, x, g, True)
    ref = run_oracle(cfg, x, g, gpu, True)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in NAMES}
    assert all(e <= 2e-2 for e in errs.values()), errs
    # the smallest forget factors, on their own
    small = x["gamma"] < 0.15
    assert small.sum() > 10
    assert rel_l2(gpu["dgamma"][small], ref["dgamma"][small]) <= 2e-2


@pytest.mark.parametrize("H,d", [(2, 64), (1, 128)])
def test_long_sequence_walked_in_segments(H, d):
    """Few sequences, 129 chunks: the adjoint scan splits each sequence into 8
    segments (segment totals, a carry pass, then the walk proper).  Slow decay
    (gamma in (0.99988, 0.999994)) keeps the final-state adjoints and the carries
    between segments far from zero, so a wrong carry shows in every gradient."""
    cfg = small_fwd(B=1, H=H, T=8192 + 100, d=d, chunk=64, dtype="bf16", max_steps=6, tol=0.0,
                    gamma_logit=(9.0, 12.0))
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    gpu = run_gpu(cfg, x, g, True)
    ref = run_oracle(cfg, x, g, gpu, True)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in NAMES}
    assert all(e <= 2e-2 for e in errs.values()), errs


def test_empty_sequence_passes_final_state_gradients_through():
    cfg = small_fwd(B=1, H=2, T=0, d=64, chunk=64, dtype="bf16", max_steps=8, tol=0.0)
    g = make_bwd_inputs(cfg)
    lam = torch.ones((2, 64), device="cuda")
    e = torch.empty((1, 2, 0, 64), device="cuda", dtype=torch.bfloat16)
    z = torch.empty((1, 2, 0), device="cuda")
    f0 = torch.empty((1, 2, 0, 64), device="cuda")
    t = {key: torch.from_numpy(val).cuda() for key, val in g.items() if key != "d_o"}
    b = mesa.bwd_chunked(e, e, e, z, z, lam, f0, f0, max_steps=8, d_hfinal=t["d_hfinal"],
                         d_gfinal=t["d_gfinal"], state_grads=True)
    torch.cuda.synchronize()
    dh = g["d_hfinal"]
    assert np.allclose(b["dh0"].cpu().numpy(), 0.5 * (dh + dh.transpose(0, 1, 3, 2)), atol=1e-6)
    assert np.array_equal(b["dg0"].cpu().numpy(), g["d_gfinal"])
    assert np.array_equal(b["dlam"].cpu().numpy(), np.zeros((2, 64), np.float32))


@pytest.mark.parametrize("d", [64, 128])
def test_whole_state_adjoint_scan(d):
    """128 sequences (B=16, H=8): the adjoint scan walks whole states, two
    workgroups per sequence; two chunks, the second ragged, with initial states and
    final-state gradients.  Every gradient against the oracle, dlambda summed over
    all 16 batch entries."""
    cfg = small_fwd(B=16, H=8, T=70, d=d, chunk=64, dtype="bf16", max_steps=8, tol=0.0)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    gpu = run_gpu(cfg, x, g)
    ref = run_oracle(cfg, x, g, gpu)
    errs = {n: rel_l2(gpu[n], ref[n]) for n in NAMES}
    print(f"whole-state adjoint scan d={d}: " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
    assert all(e <= 2e-2 for e in errs.values()), errs


def test_lm_workload_sampled_slice():
    """B=8, H=16, T=4096, d=128, 30 CG steps: the whole backward on the GPU, one
    (b, h) slice's gradients against the oracle (dlambda sums over the batch and
    is covered at the smaller sizes)."""
    from oracle import mesa_backward
    cfg = CONFIGS[3]
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    a = dev_inputs(x)
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    b = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"],
                         torch.from_numpy(g["d_o"]).cuda(), chunk=cfg.chunk, max_steps=cfg.max_steps,
                         tol=cfg.tol)
    torch.cuda.synchronize()
    bi, hi = 5, 11
    sl = lambda arr: arr[bi:bi + 1, hi:hi + 1]
    ref = mesa_backward(sl(x["q"]), sl(x["k"]), sl(x["v"]), sl(x["gamma"]), sl(x["beta"]), x["lam"][hi:hi + 1],
                        sl(g["d_o"]), max_steps=cfg.max_steps, tol=cfg.tol, chunk=cfg.chunk)
    errs = {n: rel_l2(b[n][bi:bi + 1, hi:hi + 1].cpu().numpy(), ref[n])
            for n in ("dq", "dk", "dv", "dgamma", "dbeta")}
    assert all(e <= 2e-2 for e in errs.values()), errs


def test_states_kept_from_the_forward_match_recomputed_states():
    cfg = small_fwd(B=2, H=2, T=200, d=128, chunk=64, dtype="bf16", max_steps=10)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    a = dev_inputs(x)
    d_o = torch.from_numpy(g["d_o"]).cuda()
    h0, g0 = torch.from_numpy(g["h0"]).cuda(), torch.from_numpy(g["g0"]).cuda()
    ws = torch.empty(mesa.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, cfg.max_steps, cfg.tol),
                     device="cuda", dtype=torch.uint8)
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, h0=h0, g0=g0, return_x=True, workspace=ws)
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, h0=h0, g0=g0, state_grads=True)
    kept = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], d_o,
                            workspace=ws, states_in_workspace=True, **kw)
    fresh = mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], d_o, **kw)
    torch.cuda.synchronize()
    for n in NAMES:
        assert torch.equal(kept[n], fresh[n]), n
