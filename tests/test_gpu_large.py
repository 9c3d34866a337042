"""Maximum sizes: the chunked forward, its backward and the decode step on arrays of more than 2^31 elements.

q, k, v and o of B=272, H=16, T=4096, d=128 hold 2.28e9 elements each (4.6 GB
bf16 inputs, 9.1 GB fp32 output; with the boundary snapshots about 41 GB of
HBM), so every element offset of the last (b, h) slices lies past 2^31 and a
32-bit index anywhere on the path would show.  The inputs are drawn on the GPU
(make_fwd_inputs_device); the highest slice, a middle one and the first are
copied back and run through the fp64 oracle at sampled tokens -- the first
tokens, both sides of chunk boundaries, the last chunk -- at the forward's bf16
bar, and their final states against the oracle's at 1e-4.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_fwd_inputs_device, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


@pytest.fixture(autouse=True)
def _release():
    """Hand the tens of GB these tests hold back to the device afterwards, so
    the tests that follow in the same process start from an empty cache."""
    yield
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def test_forward_beyond_2_31_elements():
    from oracle import mesa_forward
    cfg = small_fwd(B=272, H=16, T=4096, d=128, chunk=64, dtype="bf16", max_steps=6, tol=0.0, seed=31)
    assert cfg.B * cfg.H * cfg.T * cfg.d > 2 ** 31
    x = make_fwd_inputs_device(cfg)
    r = mesa.fwd_chunked(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, return_state=True, return_steps=True)
    torch.cuda.synchronize()
    assert int(r["steps"].min()) == cfg.max_steps and int(r["steps"].max()) == cfg.max_steps
    C = cfg.chunk
    at = np.zeros(cfg.T, bool)
    at[:4] = True
    for c in (1, 17, 40, cfg.T // C - 1):
        at[c * C - 1] = at[c * C] = True
    at[-C:] = True
    for b, h in ((cfg.B - 1, cfg.H - 1), (cfg.B // 2, 7), (0, 0)):
        sl = {n: x[n][b, h][None, None].double().cpu().numpy() for n in ("q", "k", "v", "gamma", "beta")}
        ref = mesa_forward(sl["q"], sl["k"], sl["v"], sl["gamma"], sl["beta"], x["lam"][h:h + 1].double().cpu().numpy(),
                           max_steps=cfg.max_steps, tol=cfg.tol, exact=False, solve_at=at)
        o = r["o"][b, h].cpu().numpy()[at]
        err = rel_l2(o, ref["o_cg"][0, 0][at])
        eh = rel_l2(r["h_final"][b, h].cpu().numpy(), ref["H_final"][0, 0])
        eg = rel_l2(r["g_final"][b, h].cpu().numpy(), ref["G_final"][0, 0])
        offset = ((b * cfg.H + h) * cfg.T + cfg.T - 1) * cfg.d
        print(f"slice ({b}, {h}) last element offset {offset:.3e}: o rel L2 {err:.2e}, final states {eh:.1e} {eg:.1e}")
        assert err <= 2e-2 and eh <= 1e-4 and eg <= 1e-4, (b, h, err, eh, eg)


def test_backward_beyond_2_31_elements():
    """The backward at B=4352, H=16, T=256, d=128: x, d_o and dq, dk, dv hold
    2.28e9 elements each (about 150 GB of HBM with the workspaces).  Gradients of
    three slices against the oracle's backward (dlambda sums over the batch and
    is covered by the smaller backward tests)."""
    from oracle import mesa_backward
    torch.cuda.empty_cache()
    cfg = small_fwd(B=4352, H=16, T=256, d=128, chunk=64, dtype="bf16", max_steps=4, tol=0.0, seed=37)
    assert cfg.B * cfg.H * cfg.T * cfg.d > 2 ** 31
    x = make_fwd_inputs_device(cfg)
    gen = torch.Generator(device="cuda")
    gen.manual_seed(cfg.seed + 1)
    d_o = torch.randn((cfg.B, cfg.H, cfg.T, cfg.d), generator=gen, device="cuda")
    f = mesa.fwd_chunked(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    b = mesa.bwd_chunked(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], f["x"], d_o, chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, state_grads=True, return_steps=True)
    torch.cuda.synchronize()
    names = ("dq", "dk", "dv", "dgamma", "dbeta", "dh0", "dg0")
    for bb, h in ((cfg.B - 1, cfg.H - 1), (cfg.B // 2, 5), (0, 0)):
        sl = {n: x[n][bb, h][None, None].double().cpu().numpy() for n in ("q", "k", "v", "gamma", "beta")}
        ref = mesa_backward(sl["q"], sl["k"], sl["v"], sl["gamma"], sl["beta"], x["lam"][h:h + 1].double().cpu().numpy(),
                            d_o[bb, h][None, None].double().cpu().numpy(), max_steps=cfg.max_steps, tol=cfg.tol,
                            forced_steps=f["steps"][bb, h][None, None].cpu().numpy(),
                            adjoint_forced_steps=b["adj_steps"][bb, h][None, None].cpu().numpy(), chunk=cfg.chunk)
        errs = {n: rel_l2(b[n][bb, h].cpu().numpy(), ref[n][0, 0]) for n in names}
        print(f"backward slice ({bb}, {h}): " + ", ".join(f"{n} {e:.2e}" for n, e in errs.items()))
        assert all(e <= 2e-2 for e in errs.values()), (bb, h, errs)


def test_decode_beyond_2_31_elements():
    """The decode step with 135,168 (sequence, head) pairs at d=128: h and g hold
    2.21e9 elements each.  The highest, a middle and the first pair against the
    oracle's step: output, solution and both updated states."""
    from oracle import mesa_decode_step
    from test_regression_sequence_amd.inputs import DecodeConfig, make_decode_inputs_device
    torch.cuda.empty_cache()
    cfg = DecodeConfig("decode-large", N=8448, H=16, d=128, prefill=0, dtype="bf16", gamma_logit=(2.0, 6.0),
                       beta_dist=("uniform", 0.0, 1.0), lam_dist=("uniform", 0.25, 1.0), max_steps=8, tol=0.0,
                       seed=41)
    assert cfg.N * cfg.H * cfg.d * cfg.d > 2 ** 31
    x = make_decode_inputs_device(cfg)
    picks = ((cfg.N - 1, cfg.H - 1), (cfg.N // 2, 9), (0, 0))
    before = {(n, h): (x["h"][n, h].double().cpu().numpy(), x["g"][n, h].double().cpu().numpy()) for n, h in picks}
    r = mesa.decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], x["h"], x["g"],
                         max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    torch.cuda.synchronize()
    assert int(r["steps"].min()) == cfg.max_steps and int(r["steps"].max()) == cfg.max_steps
    for n, h in picks:
        one = {key: x[key][n, h][None, None].double().cpu().numpy() for key in ("q", "k", "v", "gamma", "beta")}
        h0, g0 = before[(n, h)]
        ref = mesa_decode_step(one["q"], one["k"], one["v"], one["gamma"], one["beta"],
                               x["lam"][h:h + 1].double().cpu().numpy(), h0[None, None], g0[None, None],
                               max_steps=cfg.max_steps, tol=cfg.tol)
        eo = rel_l2(r["o"][n, h].cpu().numpy(), ref["o"][0, 0])
        ex = rel_l2(r["x"][n, h].cpu().numpy(), ref["x"][0, 0])
        eh = rel_l2(x["h"][n, h].cpu().numpy(), ref["h"][0, 0])
        eg = rel_l2(x["g"][n, h].cpu().numpy(), ref["g"][0, 0])
        off = ((n * cfg.H + h) * cfg.d + cfg.d - 1) * cfg.d + cfg.d - 1
        print(f"decode pair ({n}, {h}) last state offset {off:.3e}: o {eo:.2e}, x {ex:.2e}, states {eh:.1e} {eg:.1e}")
        # the bf16-input bar for the solve, fp32 arithmetic for the state updates
        assert eo <= 2e-2 and ex <= 2e-2 and eh < 1e-6 and eg < 1e-6, (n, h, eo, ex, eh, eg)
