"""Properties of the HIP path that hold at any size (needs an MI355X).

Each test also checks against the fp64 oracle where a reference exists:
chunk-size invariance, continuation of a sequence through h0/g0, a decode step
continuing a forward pass, special cases (zero steps, one step, no writes,
empty sequence), causality, run-to-run determinism and decode at other head
dims and input dtypes.  Bars as in test_gpu_parity: relative L2 <= 1e-4 for
fp32 inputs, <= 2e-2 for bf16 inputs.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, oracle_on_slices, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_decode_inputs, make_fwd_inputs, small_fwd, CONFIGS

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def fwd(d, cfg, **kw):
    args = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_steps=True)
    args.update(kw)
    res = mesa.fwd_chunked(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **args)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def oracle_all(x, steps=None, **kw):
    cfg = x["cfg"]
    idx = list(range(cfg.B * cfg.H))
    st = None if steps is None else steps.reshape(cfg.B * cfg.H, -1)
    return oracle_on_slices(x, idx, steps_gpu=st, **kw)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128), ("bf16", 64)])
def test_chunk_size_invariance(dtype, d):
    """The chunked form is exact: every chunk size gives the oracle's output."""
    cfg = small_fwd(B=1, H=2, T=160, d=d, chunk=64, dtype=dtype, max_steps=10)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    outs = {}
    for C in (16, 32, 64):
        outs[C] = fwd(dv, cfg, chunk=C)
        assert np.all(outs[C]["steps"] == 10)
    ref = np.stack([r["o_cg"][0, 0] for r in oracle_all(x, outs[64]["steps"])])
    for C, r in outs.items():
        err = rel_l2(r["o"].reshape(2, cfg.T, d), ref)
        assert err <= TOL[dtype], (C, err)
    # chunkings differ only by rounding
    agree = 1e-5 if dtype == "f32" else TOL[dtype]
    assert rel_l2(outs[16]["o"], outs[64]["o"]) <= agree
    assert rel_l2(outs[32]["o"], outs[64]["o"]) <= agree


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 32, 32), ("bf16", 128, 64)])
def test_continuation_through_states(dtype, d, chunk):
    """h_final/g_final of a prefix are valid h0/g0 for the rest of the sequence."""
    cfg = small_fwd(B=1, H=2, T=200, d=d, chunk=chunk, dtype=dtype, max_steps=8)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    whole = fwd(dv, cfg, return_state=True)
    T1 = 137  # not a multiple of the chunk
    a = {k: (t[:, :, :T1].contiguous() if k in ("q", "k", "v", "gamma", "beta") else t) for k, t in dv.items()}
    b = {k: (t[:, :, T1:].contiguous() if k in ("q", "k", "v", "gamma", "beta") else t) for k, t in dv.items()}
    first = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], chunk=chunk,
                             max_steps=8, tol=0.0, return_state=True)
    second = mesa.fwd_chunked(b["q"], b["k"], b["v"], b["gamma"], b["beta"], b["lam"], chunk=chunk,
                              max_steps=8, tol=0.0, h0=first["h_final"], g0=first["g_final"],
                              return_state=True)
    torch.cuda.synchronize()
    o = np.concatenate([first["o"].cpu().numpy(), second["o"].cpu().numpy()], axis=2)
    # the carried states equal the single call's (fp32 states, different chunk grid)
    assert rel_l2(second["h_final"].cpu().numpy(), whole["h_final"]) < 1e-5
    assert rel_l2(second["g_final"].cpu().numpy(), whole["g_final"]) < 1e-5
    # against the oracle run once over the whole sequence
    ref = np.stack([r["o_cg"][0, 0] for r in oracle_all(x, whole["steps"])])
    assert rel_l2(o.reshape(2, cfg.T, d), ref) <= TOL[dtype]
    # and the second call against the oracle started from the oracle's own prefix states
    from oracle import mesa_forward
    pre = mesa_forward(x["q"][:, :, :T1], x["k"][:, :, :T1], x["v"][:, :, :T1], x["gamma"][:, :, :T1],
                       x["beta"][:, :, :T1], x["lam"], max_steps=0, tol=0.0, exact=False,
                       solve_at=np.zeros(T1, bool))
    rest = mesa_forward(x["q"][:, :, T1:], x["k"][:, :, T1:], x["v"][:, :, T1:], x["gamma"][:, :, T1:],
                        x["beta"][:, :, T1:], x["lam"], max_steps=8, tol=0.0, exact=False,
                        h0=pre["H_final"], g0=pre["G_final"])
    assert rel_l2(second["o"].cpu().numpy(), rest["o_cg"]) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_decode_step_continues_forward(dtype, d):
    """A decode step on the forward pass's final states gives the next token's output."""
    cfg = small_fwd(B=2, H=2, T=97, d=d, chunk=32 if d == 64 else 64, dtype=dtype, max_steps=12, tol=1e-5)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    Tp = cfg.T - 1
    pre = {k: (t[:, :, :Tp].contiguous() if k in ("q", "k", "v", "gamma", "beta") else t) for k, t in dv.items()}
    res = mesa.fwd_chunked(pre["q"], pre["k"], pre["v"], pre["gamma"], pre["beta"], pre["lam"],
                           chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_state=True)
    h, g = res["h_final"], res["g_final"]
    last = {k: dv[k][:, :, Tp].contiguous() for k in ("q", "k", "v", "gamma", "beta")}
    dec = mesa.decode_step(last["q"], last["k"], last["v"], last["gamma"], last["beta"], dv["lam"], h, g,
                           max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    whole = mesa.fwd_chunked(dv["q"], dv["k"], dv["v"], dv["gamma"], dv["beta"], dv["lam"],
                             chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_state=True)
    torch.cuda.synchronize()
    # states after the step equal the forward pass's states after all T tokens
    assert rel_l2(h.cpu().numpy(), whole["h_final"].cpu().numpy()) < 1e-5
    assert rel_l2(g.cpu().numpy(), whole["g_final"].cpu().numpy()) < 1e-5
    # the step's output against the oracle's last token (at the decode's step counts)
    n = dec["steps"].cpu().numpy().reshape(-1)
    ref = []
    for s in range(cfg.B * cfg.H):
        st = np.full((1, cfg.T), cfg.max_steps, np.int64)
        st[0, -1] = n[s]
        r = oracle_on_slices(x, [s], steps_gpu=st, solve_at=np.arange(cfg.T) == cfg.T - 1)[0]
        ref.append(r["o_cg"][0, 0, -1])
    o_dec = dec["o"].cpu().numpy().reshape(-1, d)
    # fp32 arithmetic on exact inputs: far inside the bf16 bar
    assert rel_l2(o_dec, np.stack(ref)) <= 1e-4
    # the chunked pass's last output agrees with the step (both are CG approximations)
    o_fwd = whole["o"].cpu().numpy()[:, :, -1].reshape(-1, d)
    assert rel_l2(o_fwd, o_dec) <= TOL["bf16"]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 16)])
def test_special_cases(dtype, d):
    cfg = small_fwd(B=1, H=2, T=90, d=d, chunk=32, dtype=dtype, max_steps=6)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    # zero steps: x = 0, o = 0, no step taken
    r0 = fwd(dv, cfg, max_steps=0, return_x=True)
    assert np.all(r0["o"] == 0) and np.all(r0["steps"] == 0) and np.all(r0["x"] == 0)
    # one step: the scaled gated-linear-attention sum (oracle at one step)
    r1 = fwd(dv, cfg, max_steps=1)
    assert np.all(r1["steps"] == 1)
    ref = np.stack([rr["o_cg"][0, 0] for rr in oracle_all(x.copy() | {"cfg": cfg.replace(max_steps=1)})])
    assert rel_l2(r1["o"].reshape(2, cfg.T, d), ref) <= TOL[dtype]
    # no writes (beta = 0) and no initial state: G stays 0, so o = 0 exactly
    z = dict(dv)
    z["beta"] = torch.zeros_like(dv["beta"])
    rz = fwd(z, cfg, return_state=True)
    assert np.all(rz["o"] == 0) and np.all(rz["h_final"] == 0) and np.all(rz["g_final"] == 0)


def test_empty_sequence_keeps_state():
    """T = 0: nothing to solve; the final states are the initial ones."""
    d = 64
    B, H = 1, 2
    q = torch.zeros((B, H, 0, d), device="cuda", dtype=torch.bfloat16)
    gm = torch.zeros((B, H, 0), device="cuda")
    lam = torch.ones((H, d), device="cuda")
    h0 = torch.randn((B, H, d, d), device="cuda")
    h0 = (h0 + h0.transpose(-1, -2)).contiguous()
    g0 = torch.randn((B, H, d, d), device="cuda")
    res = mesa.fwd_chunked(q, q, q, gm, gm, lam, chunk=64, max_steps=4, tol=0.0, h0=h0, g0=g0,
                           return_state=True)
    torch.cuda.synchronize()
    assert res["o"].numel() == 0
    assert torch.equal(res["h_final"], h0) and torch.equal(res["g_final"], g0)


def test_causality_and_determinism():
    cfg = small_fwd(B=1, H=2, T=192, d=128, chunk=64, dtype="bf16", max_steps=10)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    a = fwd(dv, cfg)
    b = fwd(dv, cfg)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["steps"], b["steps"])
    t0 = 100  # inside the second chunk
    p = {k: t.clone() for k, t in dv.items()}
    for key in ("q", "k", "v"):
        p[key][:, :, t0:] = torch.flip(p[key][:, :, t0:], dims=[-1])
    p["gamma"][:, :, t0:] = 0.5
    p["beta"][:, :, t0:] = 1.0
    c = fwd(p, cfg)
    assert np.array_equal(c["o"][:, :, :t0], a["o"][:, :, :t0]), "an output depends on a later token"
    assert not np.array_equal(c["o"][:, :, t0:], a["o"][:, :, t0:])


@pytest.mark.parametrize("dtype,d", [("bf16", 64), ("f32", 128), ("f32", 64)])
def test_decode_other_dims_and_dtypes(dtype, d):
    cfg = CONFIGS[5].replace(N=8, H=4, d=d, prefill=200, dtype=dtype)
    x = make_decode_inputs(cfg)
    dv = dev_inputs(x)
    res = mesa.decode_step(dv["q"], dv["k"], dv["v"], dv["gamma"], dv["beta"], dv["lam"], dv["h"], dv["g"],
                           max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    from oracle import mesa_decode_step
    n = res["steps"].cpu().numpy()
    r = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], x["h"], x["g"],
                         max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=n)
    assert np.array_equal(r["steps"], n)
    check_stops(n, r["res_hist"], cfg.max_steps, cfg.tol, "f32")
    assert rel_l2(res["o"].cpu().numpy(), r["o"]) <= 1e-4
    assert rel_l2(dv["h"].cpu().numpy(), r["h"]) < 1e-6
    assert rel_l2(dv["g"].cpu().numpy(), r["g"]) < 1e-6


@pytest.mark.parametrize("d,chunk", [(128, 64), (64, 32)])
def test_strong_decay_chunks(d, chunk):
    """Chunks whose total decay exceeds e^-40 take the unscaled kernel; mixed with normal chunks."""
    cfg = small_fwd(B=1, H=2, T=5 * chunk - 7, d=d, chunk=chunk, dtype="bf16", max_steps=8)
    x = make_fwd_inputs(cfg)
    g = x["gamma"].copy()
    # chunks 1 and 3 forget fast (gamma = 0.3: about e^-77 over 64 tokens), the others as drawn
    for c in (1, 3):
        g[:, :, c * chunk:(c + 1) * chunk] = np.float32(0.3)
    g[:, 1, 4 * chunk:] = np.float32(0.05)  # the ragged last chunk of head 1 as well
    x = dict(x, gamma=g)
    dv = dev_inputs(x)
    r = fwd(dv, cfg, return_x=True, return_state=True)
    refs = oracle_all(x, r["steps"])
    o_ref = np.stack([rr["o_cg"][0, 0] for rr in refs])
    x_ref = np.stack([rr["x_cg"][0, 0] for rr in refs])
    assert rel_l2(r["o"].reshape(2, cfg.T, d), o_ref) <= TOL["bf16"]
    assert rel_l2(r["x"].reshape(2, cfg.T, d), x_ref) <= TOL["bf16"]
    for c in range(5):
        sl = slice(c * chunk, min((c + 1) * chunk, cfg.T))
        e = rel_l2(r["o"].reshape(2, cfg.T, d)[:, sl], o_ref[:, sl])
        assert e <= TOL["bf16"], (c, e)


@pytest.mark.parametrize("dtype,d,chunk", [("bf16", 128, 64), ("f32", 64, 32)])
def test_segmented_scan_with_initial_state(dtype, d, chunk):
    """Few (b, h) and many chunks: the scan walks segments (totals, carry, walk).

    Final states and sampled outputs against the oracle, starting from h0/g0.
    """
    T = 130 * chunk + 9  # 131 chunks (the last one ragged): long enough to be walked in segments
    cfg = small_fwd(B=1, H=2, T=T, d=d, chunk=chunk, dtype=dtype, max_steps=6)
    x = make_fwd_inputs(cfg)
    rng = np.random.default_rng(11)
    m = rng.standard_normal((1, 2, d, d)) / np.sqrt(d)
    h0 = (m @ m.transpose(0, 1, 3, 2)).astype(np.float32)
    h0 = (0.5 * (h0 + h0.transpose(0, 1, 3, 2))).astype(np.float32)
    g0 = (rng.standard_normal((1, 2, d, d)) / np.sqrt(d)).astype(np.float32)
    dv = dev_inputs(x)
    r = fwd(dv, cfg, h0=torch.from_numpy(h0).cuda(), g0=torch.from_numpy(g0).cuda(), return_state=True)
    from oracle import mesa_forward
    at = np.zeros(T, bool)
    at[np.random.default_rng(12).choice(T, 40, replace=False)] = True
    at[-3:] = True
    steps = r["steps"]
    ref = mesa_forward(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], max_steps=6, tol=0.0,
                       h0=h0, g0=g0, forced_steps=steps, exact=False, solve_at=at)
    assert rel_l2(r["h_final"], ref["H_final"]) < 1e-4
    assert rel_l2(r["g_final"], ref["G_final"]) < 1e-4
    assert rel_l2(r["o"][:, :, at], ref["o_cg"][:, :, at]) <= TOL[dtype]


@pytest.mark.parametrize("dtype,d,chunk", [("f32", 32, 32), ("f32", 16, 16), ("bf16", 64, 64), ("bf16", 32, 16)])
def test_many_heads_whole_state_scan(dtype, d, chunk):
    """B*H >= 128: the scan gives each state a whole workgroup; sampled slices vs the oracle."""
    cfg = small_fwd(B=2, H=64, T=3 * chunk + 5, d=d, chunk=chunk, dtype=dtype, max_steps=6)
    x = make_fwd_inputs(cfg)
    dv = dev_inputs(x)
    r = fwd(dv, cfg, return_state=True)
    idx = [0, 37, 64, 127]
    refs = oracle_on_slices(x, idx, steps_gpu=r["steps"].reshape(128, -1)[idx])
    o = r["o"].reshape(128, cfg.T, d)[idx]
    assert rel_l2(o, np.stack([rr["o_cg"][0, 0] for rr in refs])) <= TOL[dtype]
    hf = r["h_final"].reshape(128, d, d)[idx]
    gf = r["g_final"].reshape(128, d, d)[idx]
    assert rel_l2(hf, np.stack([rr["H_final"][0, 0] for rr in refs])) < 1e-5
    assert rel_l2(gf, np.stack([rr["G_final"][0, 0] for rr in refs])) < 1e-5


@pytest.mark.parametrize("d,chunk,tol", [(128, 64, 0.0), (64, 64, 1e-4), (64, 32, 0.0), (128, 32, 1e-4)])
def test_shared_chunks_match_one_wave_per_chunk(d, chunk, tol):
    """A grid of few chunks shares each chunk's token tiles out over 2 or 4
    waves; a large grid gives each chunk one wave.  Every tile runs the same
    arithmetic either way, so a slice's outputs must be bitwise equal whether
    it is solved in a small call or inside a large batch."""
    cfg = small_fwd(B=1, H=2, T=250, d=d, chunk=chunk, dtype="bf16", max_steps=16, tol=tol, seed=404)
    x = make_fwd_inputs(cfg)
    a = dev_inputs(x)
    rep = 320  # 320 x 2 heads x 4-8 chunks: one wave per chunk
    big = {k: (a[k].repeat(rep, *([1] * (a[k].dim() - 1))) if k not in ("lam",) else a[k]) for k in a}
    kw = dict(chunk=chunk, max_steps=16, tol=tol, return_x=True)
    r1 = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], **kw)
    r2 = mesa.fwd_chunked(big["q"], big["k"], big["v"], big["gamma"], big["beta"], big["lam"], **kw)
    torch.cuda.synchronize()
    for key in ("o", "x", "steps"):
        assert torch.equal(r1[key], r2[key][:1]), key
        assert torch.equal(r2[key][:1], r2[key][-1:]), key
