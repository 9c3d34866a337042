"""Seeded sweep over mixed configurations: the forward (plain, warm-started,
full Lambda), the backward and the decode step against the oracle.

The other GPU tests vary one thing at a time around the workloads; here every
case draws all of its settings at once from a fixed seed: input dtype, head
dim, chunk size, sequence length (ragged ends, a single token, one token short
of or past a chunk), batch and heads, CG step cap, tolerance (fixed and
dynamic steps), gate decay (language-model gates, or strong decay that sends
chunks to the unscaled kernels), initial states and the variant.  The bars are
those of the parity tests: relative L2 <= 1e-4 (fp32 inputs) or 2e-2 (bf16)
against the oracle at the GPU's step counts, every dynamic stop checked
against the oracle's residuals, carried states <= 1e-5 / 1e-4.  Needs an
MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import (
    CONFIGS, make_bwd_inputs, make_decode_inputs, make_full_lambda, make_fwd_inputs, small_fwd,
)

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}
GATES = {"lm": (2.0, 6.0), "strong": (-3.0, 1.0)}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def _pick(rng, edges, probs, lo, hi):
    """One of the edge values with the given probabilities, else uniform in [lo, hi)."""
    u, acc = rng.random(), 0.0
    for val, pr in zip(edges, probs):
        acc += pr
        if u < acc:
            return int(val)
    return int(rng.integers(lo, hi))


def _length(rng, chunk, hi):
    # a single token, one short of a chunk, one chunk, one past it, else ragged
    return _pick(rng, [1, chunk - 1, chunk, chunk + 1], [0.1] * 4, 2, hi)


def _steps(rng, hi):
    return _pick(rng, [0, 1], [0.08, 0.12], 2, hi + 1)


def _fwd_cases(n=40, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        variant = str(rng.choice(["plain", "plain", "warm", "lfull"]))
        dtype = "f32" if variant == "plain" and rng.random() < 0.4 else "bf16"
        if variant == "lfull":
            d, chunk = int(rng.choice([64, 128])), 64
        else:
            d = int(rng.choice([16, 32, 64, 128] if dtype == "f32" else [32, 64, 128]))
            chunk = int(rng.choice([16, 32, 64]))
        T = _length(rng, chunk, 260)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 4))
        max_steps = _steps(rng, 12)
        tol = float(rng.choice([0.0, 1e-2, 1e-3, 1e-4]))
        gates = str(rng.choice(["lm", "lm", "strong"]))
        states = bool(rng.random() < 0.5)
        out.append(dict(variant=variant, dtype=dtype, d=d, chunk=chunk, T=T, B=B, H=H, max_steps=max_steps,
                        tol=tol, gates=gates, states=states, seed=1000 + i))
    return out


def _case_id(c):
    return "-".join(f"{k}{v}" for k, v in c.items() if k != "seed")


FWD_CASES = _fwd_cases()


@pytest.mark.parametrize("c", FWD_CASES, ids=[_case_id(c) for c in FWD_CASES])
def test_forward_sweep(c):
    from oracle import mesa_forward
    cfg = small_fwd(B=c["B"], H=c["H"], T=c["T"], d=c["d"], chunk=c["chunk"], dtype=c["dtype"],
                    max_steps=c["max_steps"], tol=c["tol"], seed=c["seed"], gamma_logit=GATES[c["gates"]])
    print(f"forward case {_case_id(c)}", flush=True)
    x = make_fwd_inputs(cfg)
    init = make_bwd_inputs(cfg) if c["states"] else None
    lam = make_full_lambda(cfg.H, cfg.d, cfg.seed) if c["variant"] == "lfull" else x["lam"]
    a = dev_inputs(x)
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_state=True, return_x=True)
    if init is not None:
        kw.update(h0=torch.from_numpy(init["h0"]).cuda(), g0=torch.from_numpy(init["g0"]).cuda())
    if c["variant"] == "lfull":
        gpu = mesa.fwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], torch.from_numpy(lam).cuda(), **kw)
    else:
        gpu = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"],
                               warm=c["variant"] == "warm", **kw)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in gpu.items()}
    n = gpu["steps"]
    assert n.min() >= 0 and n.max() <= cfg.max_steps
    warm = dict(warm_start=True, warm_lag=16, warm_chunk=cfg.chunk) if c["variant"] == "warm" else {}
    ref = mesa_forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, max_steps=cfg.max_steps, tol=cfg.tol,
                       h0=None if init is None else init["h0"], g0=None if init is None else init["g0"],
                       forced_steps=n, exact=False, residual_history=cfg.tol > 0, **warm)
    assert np.array_equal(ref["steps"], n), "oracle could not run the GPU's step counts"
    bar = TOL[cfg.dtype]
    assert rel_l2(gpu["o"], ref["o_cg"]) <= bar
    assert rel_l2(gpu["x"], ref["x_cg"]) <= bar
    st = 1e-5 if cfg.dtype == "f32" else 1e-4
    assert rel_l2(gpu["h_final"], ref["H_final"]) < st
    assert rel_l2(gpu["g_final"], ref["G_final"]) < st
    if cfg.tol > 0 and cfg.T > 0:
        check_stops(n.ravel(), ref["res_hist"].reshape(-1, cfg.max_steps + 1), cfg.max_steps, cfg.tol, cfg.dtype)
    elif cfg.tol <= 0:
        assert (n == cfg.max_steps).mean() > 0.95  # fixed steps (a few systems may break down early)


def _bwd_cases(n=16, seed=2028):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        lfull = bool(rng.random() < 0.3)
        d = int(rng.choice([64, 128]))
        T = _length(rng, 64, 200)
        B, H = int(rng.integers(1, 3)), int(rng.integers(1, 3))
        max_steps = _pick(rng, [1], [0.1], 2, 13)
        tol = float(rng.choice([0.0, 0.0, 1e-3, 1e-4]))
        gates = str(rng.choice(["lm", "lm", "strong"]))
        states = bool(rng.random() < 0.5)
        out.append(dict(lfull=lfull, d=d, T=T, B=B, H=H, max_steps=max_steps, tol=tol, gates=gates,
                        states=states, seed=2000 + i))
    return out


BWD_CASES = _bwd_cases()
NAMES = ("dq", "dk", "dv", "dgamma", "dbeta", "dlam", "dh0", "dg0")


@pytest.mark.parametrize("c", BWD_CASES, ids=[_case_id(c) for c in BWD_CASES])
def test_backward_sweep(c):
    from oracle import mesa_backward
    cfg = small_fwd(B=c["B"], H=c["H"], T=c["T"], d=c["d"], chunk=64, dtype="bf16", max_steps=c["max_steps"],
                    tol=c["tol"], seed=c["seed"], gamma_logit=GATES[c["gates"]])
    print(f"backward case {_case_id(c)}", flush=True)
    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    lam = make_full_lambda(cfg.H, cfg.d, cfg.seed) if c["lfull"] else x["lam"]
    a = dev_inputs(x)
    t = {key: torch.from_numpy(val).cuda() for key, val in g.items()}
    lam_d = torch.from_numpy(np.ascontiguousarray(lam)).cuda()
    sk = dict(h0=t["h0"], g0=t["g0"]) if c["states"] else {}
    args = dict(chunk=64, max_steps=cfg.max_steps, tol=cfg.tol, **sk)
    f = mesa.fwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_d, return_x=True, **args)
    b = mesa.bwd_chunked_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam_d, f["x"], t["d_o"],
                            d_hfinal=t["d_hfinal"] if c["states"] else None,
                            d_gfinal=t["d_gfinal"] if c["states"] else None,
                            state_grads=True, return_steps=True, **args)
    torch.cuda.synchronize()
    gpu = {key: val.cpu().numpy() for key, val in b.items()}
    steps = f["steps"].cpu().numpy()
    ref = mesa_backward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, g["d_o"],
                        max_steps=cfg.max_steps, tol=cfg.tol,
                        h0=g["h0"] if c["states"] else None, g0=g["g0"] if c["states"] else None,
                        dh_final=g["d_hfinal"] if c["states"] else None,
                        dg_final=g["d_gfinal"] if c["states"] else None,
                        forced_steps=steps, adjoint_forced_steps=gpu["adj_steps"], chunk=64)
    errs = {name: rel_l2(gpu[name], ref[name]) for name in NAMES}
    assert all(e <= 2e-2 for e in errs.values()), errs
    assert gpu["adj_steps"].min() >= 0 and gpu["adj_steps"].max() <= cfg.max_steps


def _dec_cases(n=24, seed=2029):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        out.append(dict(dtype=str(rng.choice(["f32", "bf16"])), d=int(rng.choice([64, 128])),
                        N=_pick(rng, [1], [0.2], 2, 40), H=int(rng.integers(1, 4)),
                        prefill=_pick(rng, [0, 1], [0.15, 0.1], 2, 300),
                        max_steps=_pick(rng, [0, 1, 32], [0.08, 0.08, 0.2], 2, 33),
                        tol=float(rng.choice([0.0, 1e-3, 1e-4, 1e-6])),
                        packed=bool(rng.random() < 0.4), warm=bool(rng.random() < 0.4),
                        lfull=bool(rng.random() < 0.4), gates=str(rng.choice(["lm", "strong"])),
                        seed=3000 + i))
    return out


DEC_CASES = _dec_cases()


@pytest.mark.parametrize("c", DEC_CASES, ids=[_case_id(c) for c in DEC_CASES])
def test_decode_sweep(c):
    from oracle import mesa_decode_step
    cfg = CONFIGS[5].replace(N=c["N"], H=c["H"], d=c["d"], prefill=c["prefill"], dtype=c["dtype"],
                             max_steps=c["max_steps"], tol=c["tol"], seed=c["seed"],
                             gamma_logit=GATES[c["gates"]])
    print(f"decode case {_case_id(c)}", flush=True)
    x = make_decode_inputs(cfg)
    d = cfg.d
    lam = make_full_lambda(cfg.H, d, cfg.seed) if c["lfull"] else x["lam"]
    a = dev_inputs(x)
    h = mesa.sym_pack(a["h"]) if c["packed"] else a["h"]
    x0 = (np.random.default_rng([cfg.seed, 7]).standard_normal((cfg.N, cfg.H, d)) * 0.3).astype(np.float32) \
        if c["warm"] else None
    xs = torch.from_numpy(x0).cuda() if c["warm"] else None
    r = mesa.decode_step_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], torch.from_numpy(lam).cuda(), h, a["g"],
                            x_state=xs, packed_h=c["packed"], max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    steps = r["steps"].cpu().numpy()
    assert steps.min() >= 0 and steps.max() <= cfg.max_steps
    ref = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, x["h"], x["g"],
                           max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=steps, x0=x0)
    assert np.array_equal(ref["steps"], steps), "oracle could not run the GPU's step counts"
    assert rel_l2(r["o"].cpu().numpy(), ref["o"]) <= 1e-4
    if cfg.tol > 0:
        check_stops(steps, ref["res_hist"], cfg.max_steps, cfg.tol, "f32")
    if c["warm"]:
        assert rel_l2(xs.cpu().numpy(), ref["x"]) <= 1e-4
    hf = mesa.sym_unpack(h, d) if c["packed"] else h
    assert rel_l2(hf.cpu().numpy(), ref["h"]) <= 1e-6
    assert rel_l2(a["g"].cpu().numpy(), ref["g"]) <= 1e-6
