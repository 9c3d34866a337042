"""HIP path vs the fp64 oracle on the same seeded inputs (needs an MI355X).

Bars (relative L2 over the compared outputs, fp64):
  * fp32 inputs: <= 1e-4 against the oracle's CG at the GPU's per-token step counts;
  * bf16 inputs (bf16 MFMA, fp32 accumulation): <= 2e-2.
Dynamic-CG step counts are compared to the oracle run with the GPU's counts
(several counts are correct near the threshold); the stopping decision itself
is checked for validity against the oracle's residuals.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, oracle_on_slices, rel_l2, true_residual
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import (
    CONFIGS, make_bwd_inputs, make_decode_inputs, make_fwd_inputs, select_slices, small_fwd,
)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def run_fwd(x, cfg=None, **kw):
    cfg = cfg or x["cfg"]
    d = dev_inputs(x)
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_steps=True)
    args.update(kw)
    res = mesa.fwd_chunked(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **args)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def check_against_oracle(x, gpu, idx, tol):
    """Compare GPU outputs of slices idx with the oracle at the GPU's step counts."""
    cfg = x["cfg"]
    steps = gpu["steps"].reshape(cfg.B * cfg.H, cfg.T)[idx]
    refs = oracle_on_slices(x, idx, steps_gpu=steps, residual_history=cfg.tol > 0)
    o_gpu = gpu["o"].reshape(cfg.B * cfg.H, cfg.T, cfg.d)[idx]
    o_ref = np.stack([r["o_cg"][0, 0] for r in refs])
    err = rel_l2(o_gpu, o_ref)
    # forced mode reproduces the GPU's counts unless the oracle hit a breakdown earlier
    s_ref = np.stack([r["steps"][0, 0] for r in refs])
    assert np.array_equal(s_ref, steps), "oracle could not run the GPU's step counts"
    assert err <= tol, f"rel L2 {err:.3e} > {tol}"
    return err, refs


# ---------------------------------------------------------------------------
# the five workloads
# ---------------------------------------------------------------------------

def test_config1_tiny_fp32_dynamic():
    cfg = CONFIGS[1]
    x = make_fwd_inputs(cfg)
    gpu = run_fwd(x, return_x=True)
    err, refs = check_against_oracle(x, gpu, [0], TOL["f32"])
    n = gpu["steps"][0, 0]
    assert n.max() <= 16 and n.min() >= 1
    # every stop against the oracle's residuals at the same count
    rep = check_stops(n, refs[0]["res_hist"][0, 0], cfg.max_steps, cfg.tol, "f32")
    # true residual of the GPU's solutions against the fp64 systems
    st = oracle_on_slices(x, [0], solve_at=np.zeros(cfg.T, bool), record_every=1)[0]["states"]
    A = np.stack([Ht[0, 0] for _, Ht, _ in st]) + np.diag(x["lam"][0].astype(np.float64))
    tr = true_residual(A, gpu["x"][0, 0], x["q"][0, 0])
    print(f"config1 rel L2 {err:.3e}; stops {rep}; true residual median {np.median(tr):.2e} max {tr.max():.2e}")


def check_final_states(x, gpu, idx, tol):
    """h_final / g_final of slices idx against the oracle's recurrence (no solves)."""
    cfg = x["cfg"]
    refs = oracle_on_slices(x, idx, solve_at=np.zeros(cfg.T, bool))
    d = cfg.d
    Hg = gpu["h_final"].reshape(-1, d, d)[idx]
    Gg = gpu["g_final"].reshape(-1, d, d)[idx]
    eh = rel_l2(Hg, np.stack([r["H_final"][0, 0] for r in refs]))
    eg = rel_l2(Gg, np.stack([r["G_final"][0, 0] for r in refs]))
    assert eh < tol and eg < tol, (eh, eg)
    return eh, eg


def test_config2_mid_bf16_fixed15():
    x = make_fwd_inputs(CONFIGS[2])
    gpu = run_fwd(x, return_state=True)
    assert np.all(gpu["steps"] == 15)
    idx = select_slices(4, 8, 3)
    err, _ = check_against_oracle(x, gpu, idx, TOL["bf16"])
    eh, eg = check_final_states(x, gpu, idx, 1e-4)
    print(f"config2 rel L2 {err:.3e}; final states {eh:.1e} {eg:.1e}")


def test_config3_lm1b_bf16_fixed30():
    x = make_fwd_inputs(CONFIGS[3])
    gpu = run_fwd(x, return_state=True)
    assert np.all(gpu["steps"] == 30)
    idx = select_slices(8, 16, 2)
    err, _ = check_against_oracle(x, gpu, idx, TOL["bf16"])
    assert np.all(np.isfinite(gpu["o"]))
    eh, eg = check_final_states(x, gpu, idx, 1e-4)
    print(f"config3 rel L2 {err:.3e}; final states {eh:.1e} {eg:.1e}")


def test_config4_long_dynamic_sampled_tokens():
    """Long-context dynamic CG on 4 of the 16 sequences: outputs at sampled tokens
    (random, the first tokens, both sides of chunk boundaries, the last chunk) at
    the GPU's step counts, every sampled token's stopping decision, and the true
    residual of x at chunk ends."""
    cfg = CONFIGS[4]
    x = make_fwd_inputs(cfg)
    gpu = run_fwd(x, return_state=True, return_x=True)
    n = gpu["steps"]
    assert n.min() >= 1 and n.max() <= cfg.max_steps
    idx = select_slices(1, 16, 4)
    rng = np.random.default_rng(4)
    C = cfg.chunk
    at = np.zeros(cfg.T, bool)
    at[rng.choice(cfg.T, 96, replace=False)] = True
    at[:8] = True
    for c in rng.choice(np.arange(1, cfg.T // C), 12, replace=False):
        at[c * C - 1] = at[c * C] = True
    at[-C:] = True
    ends = np.flatnonzero(at & (np.arange(cfg.T) % C == C - 1))
    steps = n.reshape(16, cfg.T)[idx]
    refs = oracle_on_slices(x, idx, steps_gpu=steps, solve_at=at, residual_history=True, record_every=C)
    o_gpu = gpu["o"].reshape(16, cfg.T, cfg.d)[idx][:, at]
    err = rel_l2(o_gpu, np.stack([r["o_cg"][0, 0][at] for r in refs]))
    assert err <= TOL["bf16"], err
    reports, tres = [], []
    for i, r in enumerate(refs):
        reports.append(check_stops(steps[i][at], r["res_hist"][0, 0][at], cfg.max_steps, cfg.tol, "bf16"))
        Hs = {t: Ht[0, 0] for t, Ht, _ in r["states"]}
        A = np.stack([Hs[t + 1] for t in ends]) + np.diag(x["lam"][idx[i] % 16].astype(np.float64))
        xg = gpu["x"].reshape(16, cfg.T, cfg.d)[idx[i]][ends]
        tres.append(true_residual(A, xg, x["q"].reshape(16, cfg.T, cfg.d)[idx[i]][ends]))
    tres = np.concatenate(tres)
    eh, eg = check_final_states(x, gpu, idx[:1], 1e-4)
    hist = {}
    for rep in reports:
        for k_, v_ in rep["n_minus_oracle"].items():
            hist[k_] = hist.get(k_, 0) + v_
    print(f"config4 rel L2 {err:.3e}, steps mean {n.mean():.2f} max {n.max()}; final states {eh:.1e} {eg:.1e}; "
          f"n_gpu - n_oracle {hist}; stop ratio max {max(r_['max_stop_ratio'] for r_ in reports):.3f}, "
          f"previous min {min(r_['min_prev_ratio'] for r_ in reports):.3f}; "
          f"true residual at chunk ends median {np.median(tres):.2e} max {tres.max():.2e}")


def test_config5_decode_step():
    cfg = CONFIGS[5]
    x = make_decode_inputs(cfg)
    d = dev_inputs(x)
    res = mesa.decode_step(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], d["h"], d["g"],
                           max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    torch.cuda.synchronize()
    o = res["o"].cpu().numpy()
    n = res["steps"].cpu().numpy()
    xg = res["x"].cpu().numpy()
    h1 = d["h"].cpu().numpy()
    g1 = d["g"].cpu().numpy()
    assert n.min() >= 1 and n.max() <= cfg.max_steps
    from oracle import mesa_decode_step
    rng = np.random.default_rng(5)
    pick = rng.choice(cfg.N * cfg.H, 64, replace=False)
    sel = lambda a: a.reshape(cfg.N * cfg.H, *a.shape[2:])[pick]
    heads = pick % cfg.H
    ref_o, ref_h, ref_g, hist, A = [], [], [], [], []
    for i, p in enumerate(pick):
        hh = heads[i]
        r = mesa_decode_step(sel(x["q"])[i][None, None], sel(x["k"])[i][None, None],
                             sel(x["v"])[i][None, None], sel(x["gamma"])[i][None, None],
                             sel(x["beta"])[i][None, None], x["lam"][hh:hh + 1],
                             sel(x["h"])[i][None, None], sel(x["g"])[i][None, None],
                             max_steps=cfg.max_steps, tol=cfg.tol,
                             forced_steps=sel(n)[i].reshape(1, 1))
        ref_o.append(r["o"][0, 0]); ref_h.append(r["h"][0, 0]); ref_g.append(r["g"][0, 0])
        hist.append(r["res_hist"][0, 0])
        A.append(r["h"][0, 0] + np.diag(x["lam"][hh].astype(np.float64)))
    err = rel_l2(sel(o), np.stack(ref_o))
    assert err <= TOL["bf16"], err
    assert rel_l2(sel(h1), np.stack(ref_h)) < 1e-6
    assert rel_l2(sel(g1), np.stack(ref_g)) < 1e-6
    hs = h1.reshape(-1, cfg.d, cfg.d)
    assert np.array_equal(hs, hs.transpose(0, 2, 1)), "H lost exact symmetry"
    # the decode CG runs in fp32: every stop within the fp32 band
    rep = check_stops(sel(n), np.stack(hist), cfg.max_steps, cfg.tol, "f32")
    tr = true_residual(np.stack(A), sel(xg), sel(x["q"]))
    print(f"config5 rel L2 {err:.3e}, steps mean {n.mean():.2f}; stops {rep}; "
          f"true residual median {np.median(tr):.2e} max {tr.max():.2e}")


# ---------------------------------------------------------------------------
# small cases across dtypes, head dims, chunk sizes and ragged sequence ends
# ---------------------------------------------------------------------------

SMALL = [
    ("f32", 16, 64, 200), ("f32", 32, 16, 77), ("f32", 64, 32, 150), ("f32", 128, 64, 130),
    ("bf16", 32, 32, 100), ("bf16", 64, 64, 200), ("bf16", 64, 16, 70), ("bf16", 128, 64, 200),
    ("bf16", 128, 32, 96), ("bf16", 128, 16, 33),
]


@pytest.mark.parametrize("dtype,d,chunk,T", SMALL)
def test_small_fixed_steps(dtype, d, chunk, T):
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=chunk, dtype=dtype, max_steps=8)
    x = make_fwd_inputs(cfg)
    gpu = run_fwd(x, return_state=True, return_x=True)
    err, refs = check_against_oracle(x, gpu, [0, 1], TOL[dtype])
    # carried states after the last token
    Hr = np.stack([r["H_final"][0, 0] for r in refs])
    Gr = np.stack([r["G_final"][0, 0] for r in refs])
    st_tol = 1e-5 if dtype == "f32" else 1e-4
    assert rel_l2(gpu["h_final"].reshape(2, d, d), Hr) < st_tol
    assert rel_l2(gpu["g_final"].reshape(2, d, d), Gr) < st_tol
    assert rel_l2(gpu["x"].reshape(2, T, d), np.stack([r["x_cg"][0, 0] for r in refs])) < TOL[dtype]


# ---------------------------------------------------------------------------
# the state scan with a whole state per workgroup (B*H >= 128), every slice
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("d,T", [(64, 200), (128, 130)])
def test_whole_state_scan_every_slice(d, T):
    """B*H = 128 (two whole-state workgroups per (b, h)): every slice's final
    states against the oracle's recurrence, from given initial states, and the
    outputs of the first and last slices (they read every boundary snapshot of
    their sequence)."""
    cfg = small_fwd(B=4, H=32, T=T, d=d, chunk=64, dtype="bf16", max_steps=6)
    x = make_fwd_inputs(cfg)
    init = make_bwd_inputs(cfg)  # initial states: h0 = M M^T / d (valid, PSD), g0 ~ N(0, 0.1^2)
    h0, g0 = init["h0"], init["g0"]
    gpu = run_fwd(x, return_state=True, h0=torch.from_numpy(h0).cuda(), g0=torch.from_numpy(g0).cuda())
    from oracle import mesa_forward
    S = cfg.B * cfg.H
    Hg, Gg = gpu["h_final"].reshape(S, d, d), gpu["g_final"].reshape(S, d, d)
    eh, eg = [], []
    for i in range(S):
        b, hh = divmod(i, cfg.H)
        r = mesa_forward(x["q"][b:b + 1, hh:hh + 1], x["k"][b:b + 1, hh:hh + 1], x["v"][b:b + 1, hh:hh + 1],
                         x["gamma"][b:b + 1, hh:hh + 1], x["beta"][b:b + 1, hh:hh + 1], x["lam"][hh:hh + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, h0=h0[b:b + 1, hh:hh + 1],
                         g0=g0[b:b + 1, hh:hh + 1], exact=False, solve_at=np.zeros(T, bool))
        eh.append(rel_l2(Hg[i], r["H_final"][0, 0]))
        eg.append(rel_l2(Gg[i], r["G_final"][0, 0]))
    assert max(eh) < 1e-4 and max(eg) < 1e-4, (max(eh), max(eg))
    for i in (0, S - 1):
        b, hh = divmod(i, cfg.H)
        r = mesa_forward(x["q"][b:b + 1, hh:hh + 1], x["k"][b:b + 1, hh:hh + 1], x["v"][b:b + 1, hh:hh + 1],
                         x["gamma"][b:b + 1, hh:hh + 1], x["beta"][b:b + 1, hh:hh + 1], x["lam"][hh:hh + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, h0=h0[b:b + 1, hh:hh + 1],
                         g0=g0[b:b + 1, hh:hh + 1], exact=False, forced_steps=gpu["steps"][b:b + 1, hh:hh + 1])
        assert rel_l2(gpu["o"][b, hh], r["o_cg"][0, 0]) <= TOL["bf16"]


def test_whole_state_scan_ragged_group_of_sequences():
    """B*H = 131 (not a multiple of the 8 XCDs the scan groups sequences by):
    the padded group's workgroups must leave every real slice's states right."""
    cfg = small_fwd(B=1, H=131, T=70, d=64, chunk=64, dtype="bf16", max_steps=5)
    x = make_fwd_inputs(cfg)
    gpu = run_fwd(x, return_state=True)
    from oracle import mesa_forward
    d, S = cfg.d, cfg.H
    Hg, Gg = gpu["h_final"].reshape(S, d, d), gpu["g_final"].reshape(S, d, d)
    for hh in (0, 7, 8, 127, 128, 130):
        r = mesa_forward(x["q"][:, hh:hh + 1], x["k"][:, hh:hh + 1], x["v"][:, hh:hh + 1],
                         x["gamma"][:, hh:hh + 1], x["beta"][:, hh:hh + 1], x["lam"][hh:hh + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, exact=False,
                         forced_steps=gpu["steps"][:, hh:hh + 1])
        assert rel_l2(Hg[hh], r["H_final"][0, 0]) < 1e-4, hh
        assert rel_l2(Gg[hh], r["G_final"][0, 0]) < 1e-4, hh
        assert rel_l2(gpu["o"][0, hh], r["o_cg"][0, 0]) <= TOL["bf16"], hh
