"""Chunked forward with the query/key preprocessing fused in (mesa_fwd_chunked_prep).

The fused call takes raw q and k, convolves and normalises them inside the scan
and solve kernels, and must equal the two-call pipeline -- mesa_qk_preprocess
(bf16 outputs) then mesa_fwd_chunked -- bit for bit: outputs, solutions, step
counts, final states and the next call's histories.  Cases cover the three scan
walks (16-row stripes for few sequences, whole states for many, whole states in
segments for few long sequences), ragged last chunks, windows 1-4 with and
without a history, dynamic steps, initial states and chunks decaying past e^-40
(the unscaled solve kernel).  One case per head dim is also compared with the
fp64 oracle (oracle.qk_preprocess then oracle.mesa_forward, at the GPU's step
counts) to the forward's bf16 bar.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_fwd_inputs, make_preprocess_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def bf16(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda().to(torch.bfloat16)


def f32(a):
    return torch.from_numpy(np.ascontiguousarray(a)).cuda().float()


def inputs(cfg, W, decay=False, states=False):
    x = make_fwd_inputs(cfg)
    xp = make_preprocess_inputs(cfg, window=W)
    if decay:
        g = x["gamma"].copy()
        g[:, :, cfg.chunk:2 * cfg.chunk] = np.float32(0.3)
        x = dict(x, gamma=g)
    d = dict(qr=bf16(xp["q"]), kr=bf16(xp["k"]), v=bf16(x["v"]), gamma=f32(x["gamma"]), beta=f32(x["beta"]),
             lam=f32(x["lam"]), wq=f32(xp["wq"]), wk=f32(xp["wk"]), hq=bf16(xp["hq"]), hk=bf16(xp["hk"]))
    if states:
        rng = np.random.default_rng([cfg.seed, 7])
        B, H, D = cfg.B, cfg.H, cfg.d
        M = rng.standard_normal((B, H, D, D))
        d["h0"] = f32(np.matmul(M, M.transpose(0, 1, 3, 2)) / D)
        d["g0"] = f32(0.1 * rng.standard_normal((B, H, D, D)))
    return x, xp, d


def fused(cfg, d, with_hist):
    r = mesa.fwd_chunked_prep(d["qr"], d["kr"], d["v"], d["gamma"], d["beta"], d["lam"], d["wq"], d["wk"],
                              q_hist=d["hq"] if with_hist else None, k_hist=d["hk"] if with_hist else None,
                              chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, h0=d.get("h0"),
                              g0=d.get("g0"), return_state=True, return_x=True,
                              return_history=d["wq"].shape[-1] > 1)
    torch.cuda.synchronize()
    return r


def separate(cfg, d, with_hist):
    p = mesa.qk_preprocess(d["qr"], d["kr"], d["wq"], d["wk"], q_hist=d["hq"] if with_hist else None,
                           k_hist=d["hk"] if with_hist else None, return_history=d["wq"].shape[-1] > 1)
    r = mesa.fwd_chunked(p["q"], p["k"], d["v"], d["gamma"], d["beta"], d["lam"], chunk=cfg.chunk,
                         max_steps=cfg.max_steps, tol=cfg.tol, h0=d.get("h0"), g0=d.get("g0"),
                         return_state=True, return_x=True)
    torch.cuda.synchronize()
    r.update({k: p[k] for k in ("q_hist", "k_hist") if k in p})
    return r


def assert_bitwise(a, b):
    assert a.keys() == b.keys()
    for key in a:
        assert torch.equal(a[key], b[key]), key


CASES = [
    # B, H, T, d, W, hist, max_steps, tol, decay, states
    (1, 2, 200, 128, 4, True, 8, 0.0, False, False),     # stripes; three chunks and a ragged one
    (1, 2, 200, 128, 4, False, 8, 0.0, False, False),
    (1, 2, 150, 128, 1, False, 32, 1e-4, False, False),  # window 1: normalisation only
    (1, 3, 77, 64, 2, True, 32, 1e-4, False, True),
    (2, 1, 130, 64, 3, True, 10, 0.0, True, False),      # a chunk left to the unscaled kernel
    (1, 2, 200, 128, 4, True, 32, 1e-4, True, True),
    (1, 1, 5, 128, 4, True, 8, 0.0, False, False),       # shorter than the window
    (16, 8, 100, 128, 3, True, 8, 0.0, False, True),     # whole-state scan (2BH = 256)
    (16, 8, 64, 64, 4, False, 32, 1e-4, False, False),
]


@pytest.mark.parametrize("B,H,T,d,W,hist,max_steps,tol,decay,states", CASES)
def test_fused_equals_preprocess_then_forward(B, H, T, d, W, hist, max_steps, tol, decay, states):
    cfg = small_fwd(B=B, H=H, T=T, d=d, chunk=64, dtype="bf16", max_steps=max_steps, tol=tol)
    _, _, dv = inputs(cfg, W, decay, states)
    assert_bitwise(fused(cfg, dv, hist), separate(cfg, dv, hist))


@pytest.mark.parametrize("d", [64, 128])
def test_segmented_scan(d):
    """Two sequences of 131 chunks: the whole-state scan walks 16 segments
    (segment totals, a carry pass, then the walk proper)."""
    cfg = small_fwd(B=1, H=2, T=130 * 64 + 9, d=d, chunk=64, dtype="bf16", max_steps=6, tol=0.0)
    _, _, dv = inputs(cfg, 4, states=True)
    assert_bitwise(fused(cfg, dv, True), separate(cfg, dv, True))


@pytest.mark.parametrize("d,W,tol,decay", [(128, 4, 1e-4, False), (64, 3, 0.0, True)])
def test_fused_matches_oracle(d, W, tol, decay):
    from oracle import mesa_forward, qk_preprocess
    T = 150
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=64, dtype="bf16", max_steps=32 if tol else 10, tol=tol)
    x, xp, dv = inputs(cfg, W, decay)
    gpu = {k: v.float().cpu().numpy() if v.dtype == torch.bfloat16 else v.cpu().numpy()
           for k, v in fused(cfg, dv, True).items()}
    q, _ = qk_preprocess(xp["q"], xp["wq"], xp["hq"])
    k, _ = qk_preprocess(xp["k"], xp["wk"], xp["hk"])
    steps = gpu["steps"].reshape(2, T)
    for i in range(2):
        b, h = divmod(i, cfg.H)
        sl = lambda a: a[b:b + 1, h:h + 1]
        r = mesa_forward(sl(q), sl(k), sl(x["v"]), sl(x["gamma"]), sl(x["beta"]), x["lam"][h:h + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=steps[i][None, None],
                         residual_history=tol > 0)
        assert np.array_equal(r["steps"][0, 0], steps[i])
        eo = rel_l2(gpu["o"][b, h], r["o_cg"][0, 0])
        ex = rel_l2(gpu["x"][b, h], r["x_cg"][0, 0])
        assert eo <= 2e-2 and ex <= 2e-2, (eo, ex)
        if tol > 0:
            print(f"fused d={d} slice {i}: rel L2 {eo:.2e}, stops {check_stops(steps[i], r['res_hist'][0, 0], cfg.max_steps, tol, 'bf16')}")


def test_rejected_arguments_launch_nothing():
    cfg = small_fwd(B=1, H=2, T=70, d=128, chunk=64, dtype="bf16", max_steps=4)
    _, _, dv = inputs(cfg, 4)
    with pytest.raises(mesa.MesaError) as e:
        mesa.fwd_chunked_prep(dv["qr"], dv["kr"], dv["v"], dv["gamma"], dv["beta"], dv["lam"], dv["wq"],
                              dv["wk"], chunk=32)
    assert e.value.status == 2
    with pytest.raises(mesa.MesaError) as e:
        mesa.fwd_chunked_prep(dv["qr"], dv["kr"], dv["v"], dv["gamma"], dv["beta"], dv["lam"], dv["wq"],
                              dv["wk"], eps=0.0)
    assert e.value.status == 1
