#!/usr/bin/env python3
"""Throughput of the chunked Mesa forward (and the decode step) on one MI355X.

One *step* is one call of ``mesa_fwd_chunked`` -- the state scan plus the
chunked CG solve and read-out -- over the 1B-LM-shaped layer workload
(B=8, H=16, T=4096, d=128, chunk 64, bf16 q/k/v with fp32 accumulation,
30 fixed CG steps), inputs resident in HBM.  The JSON line reports:

* value: tokens/s = B*H*T / (time per step);
* roofline: the CG kernel (the dominant kernel) -- counted flops per launch
  over its average duration, measured with HIP events on the stream it runs
  on, against the bf16 dense MFMA peak;
* decode: the recurrent decode step (256 sequences x 16 heads, d=128, fp32
  states, CG tolerance 1e-4 / at most 32 steps): HBM bytes moved per step
  over its duration, against the HBM peak, with H stored full and packed
  (blocked upper triangle); successive calls rotate over three copies of the
  states so that none is served from the last-level cache;
* cpu_baseline: the fp64 oracle on a bounded sample of the same workload.

Counted flops per token follow the chunkwise algorithm (causal half of the
intra-chunk products, nbar = (C+1)/2 keys on average):
  scan  F_s = 2 dk^2 + 2 dv dk
  CG    F_c = 2 dk^2 + 4 dk nbar + 10 dk   per iteration
  out   F_o = 2 dv dk + 2 dk nbar + 2 dv nbar
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
NOMINAL_CLOCK_MHZ = 2400.0  # MI355X peak engine clock, the one the MFMA peak is quoted at
DECODE_STATE_COPIES = 3     # decode calls rotate over this many state copies


def flops_per_token(d: int, C: int, n_steps: float) -> dict:
    nbar = (C + 1) / 2.0
    f_s = 2 * d * d + 2 * d * d
    f_c = 2 * d * d + 4 * d * nbar + 10 * d
    f_o = 2 * d * d + 2 * d * nbar + 2 * d * nbar
    return {"scan": f_s, "cg_iter": f_c, "out": f_o, "cg_kernel": n_steps * f_c + f_o,
            "total": f_s + n_steps * f_c + f_o}


def decode_bytes_per_pair(d: int, in_bytes: int = 2, h_floats: int | None = None) -> int:
    # H and G read + written (fp32), q/k/v in, gamma/beta in, o out, steps out;
    # h_floats: floats of a packed H state (default: full d x d)
    hf = d * d if h_floats is None else h_floats
    return 2 * 4 * (hf + d * d) + 3 * in_bytes * d + 2 * 4 + 4 * d + 4


def time_events(fn, iters):
    import torch
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(iters):
        fn()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / iters


def bench_forward(cfg, steps, warmup, x=None, clock=False):
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs

    x = make_fwd_inputs(cfg) if x is None else x
    dev = "cuda"
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(x["q"]).to(dev).to(dt)
    k = torch.from_numpy(x["k"]).to(dev).to(dt)
    v = torch.from_numpy(x["v"]).to(dev).to(dt)
    gamma = torch.from_numpy(x["gamma"]).to(dev)
    beta = torch.from_numpy(x["beta"]).to(dev)
    lam = torch.from_numpy(x["lam"]).to(dev)
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    need = mesa.workspace_bytes(B, H, T, d, cfg.chunk, dtype=dt)
    ws = torch.empty(need, device=dev, dtype=torch.uint8)
    o = torch.empty((B, H, T, d), device=dev, dtype=torch.float32)
    st = torch.empty((B, H, T), device=dev, dtype=torch.int32)
    out = {"o": o, "steps": st}
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, workspace=ws, out=out)

    # One step is the forward's two entry points back to back on the current
    # stream -- the state scan, then the CG solve and read-out -- which are the
    # kernels one mesa_fwd_chunked call launches.  An event between the two, in
    # every timed step, gives each kernel's duration over the timed region
    # itself (the solve's pair also brackets its 4.5 us strong-decay check).
    def step(ev=None):
        if ev is not None:
            ev[0].record()
        mesa.fwd_scan(k, v, gamma, beta, chunk=cfg.chunk, workspace=ws)
        if ev is not None:
            ev[1].record()
        mesa.fwd_solve(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps,
                       tol=cfg.tol, workspace=ws, o=o, steps=st)
        if ev is not None:
            ev[2].record()

    for _ in range(warmup):
        step()
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(steps):
        step(evs[i])
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps * 1e3
    ms = evs[0][0].elapsed_time(evs[-1][2]) / steps
    scan_ms = [e[0].elapsed_time(e[1]) for e in evs]
    cg_ms = [e[1].elapsed_time(e[2]) for e in evs]
    step_ms = [e[0].elapsed_time(e[2]) for e in evs]
    n = st.cpu().numpy()
    clock = sample_gfx_clock(step, ms) if clock else None
    return dict(ms=ms, wall_ms=wall, scan_ms=float(np.mean(scan_ms)), cg_ms=float(np.mean(cg_ms)),
                step_ms=step_ms, cg_ms_each=cg_ms,
                steps_mean=float(n.mean()), steps_max=int(n.max()), steps=n, x=x, clock=clock)


def sample_gfx_clock(step, ms_per_step: float, seconds: float = 2.5, period: float = 0.1):
    """The GFX clock (MHz) under the timed work, as the SMI library reports it:
    after the timed region the step runs back to back for about `seconds`
    while the host reads the GPU metrics every `period` seconds.  A sample is
    the mean of the per-XCD current GFX clocks; only samples taken while the
    GFX engine reports itself at least half busy count (the metrics table is
    refreshed about once a second, so the first reads still show the idle
    GPU).  None where the SMI library cannot be read."""
    import torch
    try:
        handle = torch.cuda._get_amdsmi_handler(0)
        import amdsmi
        amdsmi.amdsmi_get_gpu_metrics_info(handle)
    except Exception:
        return None

    def read():
        m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
        clks = [c for c in m.get("current_gfxclks", []) if isinstance(c, (int, float)) and 0 < c < 0xFFFF]
        act = m.get("average_gfx_activity")
        if not clks or not isinstance(act, (int, float)) or act < 50:
            return None
        return float(sum(clks)) / len(clks)

    n = max(1, int(seconds * 1e3 / max(ms_per_step, 1e-3)))
    torch.cuda.synchronize()
    done = torch.cuda.Event()
    for _ in range(n):
        step()
    done.record()
    samples = []
    while not done.query():
        try:
            c = read()
        except Exception:
            break
        if c is not None:
            samples.append(c)
        time.sleep(period)
    torch.cuda.synchronize()
    if not samples:
        return None
    return {"gfx_mhz_median": round(float(np.median(samples)), 1), "gfx_mhz_min": round(min(samples), 1),
            "gfx_mhz_max": round(max(samples), 1), "samples": len(samples), "steps_run": n}


def clock_report(clock, cg_tflops: float):
    """The sustained GFX clock beside the CG kernel's fraction of the nominal
    peak, and that fraction rescaled to the clock measured (the nominal peak
    assumes 2.4 GHz)."""
    if clock is None:
        return None
    r = dict(clock)
    r["source"] = ("SMI GPU metrics (mean of the per-XCD current GFX clocks, samples at >= 50 % GFX "
                   "activity) read from the host every 0.1 s while the forward step ran back to back for "
                   "2.5 s after the timed region")
    r["nominal_mhz"] = NOMINAL_CLOCK_MHZ
    peak_at_clock = PEAK_BF16_TFLOPS * clock["gfx_mhz_median"] / NOMINAL_CLOCK_MHZ
    r["cg_frac_of_peak_at_that_clock"] = round(cg_tflops / peak_at_clock, 4)
    return r


def spread(ms: list) -> dict:
    """Median and interquartile range of per-step times (ms)."""
    q1, med, q3 = np.percentile(np.asarray(ms, dtype=np.float64), [25, 50, 75])
    return {"median": round(float(med), 4), "p25": round(float(q1), 4), "p75": round(float(q3), 4),
            "iqr": round(float(q3 - q1), 4), "n": len(ms)}


def recurrent_flops_per_token(d: int, n_steps: float) -> float:
    """The token-by-token recurrence's own count: the two state updates, the
    CG iterations on an explicit H and the read-out; a lower bound on the
    flops of any form of the layer, reported for context."""
    return 3 * d * d + 3 * d * d + n_steps * (2 * d * d + 10 * d) + 2 * d * d


def cg_kernel_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one CG launch (bf16 inputs): per chunk the two
    bf16 boundary snapshots, q, k, v, gamma, beta read; o and steps written."""
    chunks = cfg.B * cfg.H * ((cfg.T + cfg.chunk - 1) // cfg.chunk)
    esz = 2 if cfg.dtype == "bf16" else 4
    tok = cfg.B * cfg.H * cfg.T
    return int(chunks * 2 * cfg.d * cfg.d * esz + tok * (3 * cfg.d * esz + 2 * 4 + cfg.d * 4 + 4))


def scan_kernel_bytes(cfg) -> int:
    """Algorithmic HBM bytes of one scan launch: k, v and gates read, the two
    boundary snapshots of every chunk written."""
    chunks = cfg.B * cfg.H * ((cfg.T + cfg.chunk - 1) // cfg.chunk)
    esz = 2 if cfg.dtype == "bf16" else 4
    tok = cfg.B * cfg.H * cfg.T
    return int(chunks * 2 * cfg.d * cfg.d * esz + tok * (2 * cfg.d * esz + 2 * 4))


def forward_report(cfg, fw) -> dict:
    """Times, counted TFLOP/s and HBM rates of one forward workload."""
    tokens = cfg.B * cfg.H * cfg.T
    f = flops_per_token(cfg.d, cfg.chunk, fw["steps_mean"])
    cg_tf = f["cg_kernel"] * tokens / (fw["cg_ms"] * 1e-3) / 1e12
    tot_tf = f["total"] * tokens / (fw["ms"] * 1e-3) / 1e12
    cg_b, sc_b = cg_kernel_bytes(cfg), scan_kernel_bytes(cfg)
    n = fw["steps"].reshape(cfg.B * cfg.H, -1)
    T = n.shape[1]
    pad = (-T) % cfg.chunk
    nc = np.pad(n, ((0, 0), (0, pad)), constant_values=0).reshape(n.shape[0], -1, cfg.chunk)
    nt = nc.reshape(n.shape[0], nc.shape[1], cfg.chunk // 16, 16)
    return {
        "workload": f"{cfg.name}: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} chunk={cfg.chunk} {cfg.dtype}, "
                    + (f"fixed {cfg.max_steps}" if cfg.tol <= 0 else f"tol {cfg.tol:g} max {cfg.max_steps}")
                    + " CG steps",
        "ms_per_call": round(fw["ms"], 4),
        "tokens_per_s": round(tokens / (fw["ms"] * 1e-3), 1),
        "kernels_ms": {"scan": round(fw["scan_ms"], 4), "cg": round(fw["cg_ms"], 4)},
        "cg_counted_TFLOPs": round(cg_tf, 2),
        "cg_frac_of_mfma_peak": round(cg_tf / PEAK_BF16_TFLOPS, 4),
        "fwd_frac_of_mfma_peak": round(tot_tf / PEAK_BF16_TFLOPS, 4),
        "cg_hbm_GBs": round(cg_b / (fw["cg_ms"] * 1e-3) / 1e9, 1),
        "cg_frac_of_hbm_peak": round(cg_b / (fw["cg_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "scan_hbm_GBs": round(sc_b / (fw["scan_ms"] * 1e-3) / 1e9, 1),
        "scan_frac_of_hbm_peak": round(sc_b / (fw["scan_ms"] * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
        "step_ms": spread(fw["step_ms"]),
        "cg_ms": spread(fw["cg_ms_each"]),
        "recurrent_form_flops_per_token": recurrent_flops_per_token(cfg.d, fw["steps_mean"]),
        "recurrent_form_TFLOPs": round(recurrent_flops_per_token(cfg.d, fw["steps_mean"]) * tokens
                                       / (fw["ms"] * 1e-3) / 1e12, 2),
        "cg_steps_mean": round(fw["steps_mean"], 3),
        "cg_steps_max": fw["steps_max"],
        # the work a chunk's wave does follows its tiles' slowest tokens
        "chunk_max_over_mean": round(float(nc.max(axis=2).mean() / max(fw["steps_mean"], 1e-9)), 4),
        "tile_max_over_mean": round(float(nt.max(axis=3).mean() / max(fw["steps_mean"], 1e-9)), 4),
    }


def bench_warm_forward(cfg, steps, warmup) -> dict:
    """Cold against warm-started CG in the chunked forward (mesa_fwd_chunked_warm:
    token t starts from token t-16's solution within its chunk), on the
    workload's own queries and on slowly varying ones (per-dimension AR(1),
    lag-1 correlation 0.99).  Whole calls, alternating cold and warm, HIP
    events, medians; mean CG steps over the tokens a warm start applies to
    (tiles 1.. of every chunk) and over all, and the mean over 16-token tiles
    of a tile's slowest token (the wave iterates until it stops)."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs, make_slow_queries
    base = make_fwd_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    ws = torch.empty(mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, dtype=dt), device="cuda",
                     dtype=torch.uint8)
    later = (np.arange(cfg.T) % cfg.chunk) >= 16
    out = {"rule": "token t starts from token t-16's solution when both lie in one chunk, else from 0"}
    for name, x in (("workload_queries", base), ("slow_queries_ar1_0.99", make_slow_queries(base, 0.99))):
        q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
        gamma, beta, lam = (torch.from_numpy(x[n]).cuda() for n in ("gamma", "beta", "lam"))
        rec = {}
        res = {w: mesa.fwd_chunked(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps,
                                   tol=cfg.tol, workspace=ws, warm=w) for w in (False, True)}
        ev = {w: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                  for _ in range(steps)] for w in (False, True)}

        def call(w, e=None):
            if e is not None:
                e[0].record()
            mesa.fwd_chunked(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                             workspace=ws, out=res[w], warm=w)
            if e is not None:
                e[1].record()

        # cold and warm calls alternate, so that neither profits from the clock
        # or cache state the other leaves
        for _ in range(warmup):
            call(False)
            call(True)
        torch.cuda.synchronize()
        for i in range(steps):
            call(False, ev[False][i])
            call(True, ev[True][i])
        torch.cuda.synchronize()
        for w in (False, True):
            ms = float(np.median([a.elapsed_time(b) for a, b in ev[w]]))
            n = res[w]["steps"].cpu().numpy()
            rec["warm" if w else "cold"] = {"ms_per_call_median": round(ms, 4),
                                            "cg_steps_mean": round(float(n.mean()), 3),
                                            "cg_steps_mean_tiles_1_on": round(float(n[:, :, later].mean()), 3),
                                            "tile_max_steps_mean": round(float(n.reshape(
                                                cfg.B * cfg.H, -1, 16).max(axis=2).mean()), 3)}
        out[name] = rec
        del q, k, v, gamma, beta, lam
    return out


def bench_prep_forward(cfg, steps, warmup, window=4) -> dict:
    """The layer forward on raw queries and keys: the preprocessing kernel then
    the forward (two calls) against mesa_fwd_chunked_prep (preprocessing fused
    into the scan and solve loads), with raw histories.  Whole calls, the two
    forms alternating, HIP events, medians; the outputs are checked equal."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs, make_preprocess_inputs
    x = make_fwd_inputs(cfg)
    xp = make_preprocess_inputs(cfg, window)
    qr, kr, hq, hk = (torch.from_numpy(xp[n]).cuda().to(torch.bfloat16) for n in ("q", "k", "hq", "hk"))
    wq, wk = (torch.from_numpy(xp[n]).cuda() for n in ("wq", "wk"))
    v = torch.from_numpy(x["v"]).cuda().to(torch.bfloat16)
    gamma, beta, lam = (torch.from_numpy(x[n]).cuda() for n in ("gamma", "beta", "lam"))
    del x, xp
    ws = torch.empty(mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk), device="cuda", dtype=torch.uint8)
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, workspace=ws)
    pre = mesa.qk_preprocess(qr, kr, wq, wk, q_hist=hq, k_hist=hk)
    res = {"separate": mesa.fwd_chunked(pre["q"], pre["k"], v, gamma, beta, lam, **kw),
           "fused": mesa.fwd_chunked_prep(qr, kr, v, gamma, beta, lam, wq, wk, q_hist=hq, k_hist=hk, **kw)}

    def call(form, e=None):
        if e is not None:
            e[0].record()
        if form == "separate":
            mesa.qk_preprocess(qr, kr, wq, wk, q_hist=hq, k_hist=hk, out=pre)
            mesa.fwd_chunked(pre["q"], pre["k"], v, gamma, beta, lam, out=res[form], **kw)
        else:
            mesa.fwd_chunked_prep(qr, kr, v, gamma, beta, lam, wq, wk, q_hist=hq, k_hist=hk, out=res[form], **kw)
        if e is not None:
            e[1].record()

    ev = {f: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
          for f in res}
    for _ in range(warmup):
        for f in res:
            call(f)
    torch.cuda.synchronize()
    for i in range(steps):
        for f in res:
            call(f, ev[f][i])
    torch.cuda.synchronize()
    same = all(torch.equal(res["separate"][k], res["fused"][k]) for k in res["separate"])
    ms = {f: float(np.median([a.elapsed_time(b) for a, b in ev[f]])) for f in res}
    tokens = cfg.B * cfg.H * cfg.T
    return {"workload": f"{cfg.name} shape, raw q/k with window {window} and histories",
            "separate_ms_median": round(ms["separate"], 4), "fused_ms_median": round(ms["fused"], 4),
            "saved_ms": round(ms["separate"] - ms["fused"], 4),
            "fused_tokens_per_s": round(tokens / (ms["fused"] * 1e-3), 1),
            "outputs_bitwise_equal": bool(same)}


def bench_latency(cfg, steps, warmup) -> dict:
    """One whole mesa_fwd_chunked call on a tiny workload: latency."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs
    x = make_fwd_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
    gamma, beta, lam = (torch.from_numpy(x[n]).cuda() for n in ("gamma", "beta", "lam"))
    ws = torch.empty(max(1, mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, dtype=dt)),
                     device="cuda", dtype=torch.uint8)
    res = mesa.fwd_chunked(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                           workspace=ws)

    def step():
        mesa.fwd_chunked(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                         workspace=ws, out=res)

    for _ in range(warmup):
        step()
    ms = time_events(step, steps)
    n = res["steps"].cpu().numpy()
    return {"workload": f"{cfg.name}: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} chunk={cfg.chunk} {cfg.dtype}, "
                        f"tol {cfg.tol:g} max {cfg.max_steps} CG steps",
            "us_per_call": round(ms * 1e3, 2), "cg_steps_mean": round(float(n.mean()), 3),
            "cg_steps_max": int(n.max())}


def bench_decode(cfg, steps, warmup):
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_decode_inputs

    x = make_decode_inputs(cfg)
    dev = "cuda"
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(x["q"]).to(dev).to(dt)
    k = torch.from_numpy(x["k"]).to(dev).to(dt)
    v = torch.from_numpy(x["v"]).to(dev).to(dt)
    gamma = torch.from_numpy(x["gamma"]).to(dev)
    beta = torch.from_numpy(x["beta"]).to(dev)
    lam = torch.from_numpy(x["lam"]).to(dev)
    # Successive calls take the next of DECODE_STATE_COPIES copies of the
    # states: a model streams every other layer's states between two steps of
    # one layer, so no step finds its states in the 256 MB last-level cache
    # (one state of this workload, 268 MB, nearly fits, and timing a single
    # copy over and over would count those cache hits as HBM bandwidth).
    hs_full = [torch.from_numpy(x["h"]).to(dev) for _ in range(DECODE_STATE_COPIES)]
    gs = [torch.from_numpy(x["g"]).to(dev) for _ in range(DECODE_STATE_COPIES)]
    o = torch.empty((cfg.N, cfg.H, cfg.d), device=dev, dtype=torch.float32)
    st = torch.empty((cfg.N, cfg.H), device=dev, dtype=torch.int32)
    h_host, g_host = x["h"], x["g"]
    del x
    turn = [0]

    def next_copy():
        i = turn[0] % DECODE_STATE_COPIES
        turn[0] += 1
        return i

    def step():
        i = next_copy()
        mesa.decode_step(q, k, v, gamma, beta, lam, hs_full[i], gs[i], max_steps=cfg.max_steps, tol=cfg.tol,
                         out={"o": o, "steps": st})

    # the first call measures the step count on the generated state
    step()
    torch.cuda.synchronize()
    n_first = st.cpu().numpy()
    for _ in range(warmup):
        step()
    ms = time_events(step, steps)
    n = st.cpu().numpy()
    pairs = cfg.N * cfg.H
    in_bytes = 2 if cfg.dtype == "bf16" else 4
    nbytes = pairs * decode_bytes_per_pair(cfg.d, in_bytes) + cfg.H * cfg.d * 4
    gbs = nbytes / (ms * 1e-3) / 1e9

    # the same step with a full symmetric positive definite Lambda per head
    from test_regression_sequence_amd.inputs import make_full_lambda
    lam_full = torch.from_numpy(make_full_lambda(cfg.H, cfg.d, cfg.seed)).to(dev)

    def step_lfull():
        i = next_copy()
        mesa.decode_step_ex(q, k, v, gamma, beta, lam_full, hs_full[i], gs[i], max_steps=cfg.max_steps,
                            tol=cfg.tol, out={"o": o, "steps": st})

    for _ in range(max(1, warmup)):
        step_lfull()
    ms_lf = time_events(step_lfull, steps)
    n_lf = st.cpu().numpy()

    # the same step with H in the packed-symmetric layout (blocked upper triangle)
    hs_sym = [mesa.sym_pack(h) for h in hs_full]
    del hs_full
    torch.cuda.empty_cache()

    def step_symh():
        i = next_copy()
        mesa.decode_step_symh(q, k, v, gamma, beta, lam, hs_sym[i], gs[i], max_steps=cfg.max_steps, tol=cfg.tol,
                              out={"o": o, "steps": st})

    for _ in range(max(1, warmup)):
        step_symh()
    ms_s = time_events(step_symh, steps)
    nbytes_s = pairs * decode_bytes_per_pair(cfg.d, in_bytes, mesa.sym_state_floats(cfg.d)) + cfg.H * cfg.d * 4
    gbs_s = nbytes_s / (ms_s * 1e-3) / 1e9
    del hs_sym, gs
    torch.cuda.empty_cache()
    warm = bench_decode_warm(cfg, h_host, g_host, lam, in_bytes)
    return {
        "workload": f"decode step: {cfg.N} seqs x {cfg.H} heads, d={cfg.d}, fp32 states, "
                    f"{cfg.dtype} q/k/v, CG tol {cfg.tol:g} max {cfg.max_steps}",
        "us_per_step": round(ms * 1e3, 2),
        "pairs_per_s": round(pairs / (ms * 1e-3), 1),
        "seq_tokens_per_s": round(cfg.N / (ms * 1e-3), 1),
        "bytes_per_step": int(nbytes),
        "achieved_GBs": round(gbs, 1),
        "peak_GBs": PEAK_HBM_GBS,
        "frac": round(gbs / PEAK_HBM_GBS, 4),
        "cg_steps_first_call_mean": round(float(n_first.mean()), 2),
        "cg_steps_mean": round(float(n.mean()), 2),
        "state_copies": DECODE_STATE_COPIES,
        "full_lambda": {
            "lambda": "full symmetric positive definite per head (read through the cache, shared by the sequences)",
            "us_per_step": round(ms_lf * 1e3, 2),
            "achieved_GBs": round(nbytes / (ms_lf * 1e-3) / 1e9, 1),
            "frac": round(nbytes / (ms_lf * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "cg_steps_mean": round(float(n_lf.mean()), 2),
        },
        "packed_h": {
            "layout": "H as 16x16 blocks on and above the block diagonal (36 of 64 at d=128)",
            "us_per_step": round(ms_s * 1e3, 2),
            "pairs_per_s": round(pairs / (ms_s * 1e-3), 1),
            "bytes_per_step": int(nbytes_s),
            "achieved_GBs": round(gbs_s, 1),
            "frac": round(gbs_s / PEAK_HBM_GBS, 4),
        },
        "warm_start": warm,
    }


def bench_decode_warm(cfg, h_host, g_host, lam, in_bytes, T=8):
    """Cold against warm-started CG over T consecutive tokens of related queries.

    Both runs decode the same stream from the same states (full-layout H,
    rotating over the state copies); the warm run starts every pair's CG at
    its previous solution.  Step counts are averaged over tokens 1..T-1
    (token 0 starts from zero in both)."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_decode_stream

    dev = "cuda"
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    x = make_decode_stream(cfg, T)
    tok = [{key: torch.from_numpy(np.ascontiguousarray(x[key][:, :, t])).to(dev).to(dt if key in ("q", "k", "v") else torch.float32)
            for key in ("q", "k", "v", "gamma", "beta")} for t in range(T)]
    del x
    nc = DECODE_STATE_COPIES
    o = torch.empty((cfg.N, cfg.H, cfg.d), device=dev, dtype=torch.float32)
    st = torch.empty((nc, T, cfg.N, cfg.H), device=dev, dtype=torch.int32)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)

    def run(warm):
        hs = [torch.from_numpy(h_host).to(dev) for _ in range(nc)]
        gs = [torch.from_numpy(g_host).to(dev) for _ in range(nc)]
        xs = [torch.zeros((cfg.N, cfg.H, cfg.d), device=dev) for _ in range(nc)]
        torch.cuda.synchronize()
        e0.record()
        for t in range(T):
            a = tok[t]
            for c in range(nc):
                if warm:
                    mesa.decode_step_warm(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam, hs[c], gs[c], xs[c],
                                          max_steps=cfg.max_steps, tol=cfg.tol, out={"o": o, "steps": st[c, t]})
                else:
                    mesa.decode_step(a["q"], a["k"], a["v"], a["gamma"], a["beta"], lam, hs[c], gs[c],
                                     max_steps=cfg.max_steps, tol=cfg.tol, out={"o": o, "steps": st[c, t]})
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / (T * nc)
        n = st[:, 1:].float().mean().item()
        del hs, gs, xs
        torch.cuda.empty_cache()
        return ms, n

    run(True)  # warm-up
    ms_c, n_c = run(False)
    ms_w, n_w = run(True)
    pairs = cfg.N * cfg.H
    nbytes = pairs * (decode_bytes_per_pair(cfg.d, in_bytes) + 2 * 4 * cfg.d) + cfg.H * cfg.d * 4
    gbs = nbytes / (ms_w * 1e-3) / 1e9
    return {
        "stream": f"{T} tokens per pair; q, k per-dim AR(1) with lag-1 correlation 0.75, L2-normalised",
        "cold": {"us_per_step": round(ms_c * 1e3, 2), "cg_steps_mean": round(n_c, 2)},
        "warm": {"us_per_step": round(ms_w * 1e3, 2), "cg_steps_mean": round(n_w, 2),
                 "bytes_per_step": int(nbytes), "achieved_GBs": round(gbs, 1),
                 "frac": round(gbs / PEAK_HBM_GBS, 4)},
    }


def bench_backward(cfg, steps, warmup):
    """The backward pass (implicit differentiation through both CG solves) at the
    layer workload: one mesa_bwd_chunked call, the forward's x and o resident."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs, make_bwd_inputs

    x = make_fwd_inputs(cfg)
    g = make_bwd_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
    gamma, beta, lam = (torch.from_numpy(x[n]).cuda() for n in ("gamma", "beta", "lam"))
    d_o = torch.from_numpy(g["d_o"]).cuda()
    del x, g
    ws = torch.empty(mesa.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, cfg.max_steps, cfg.tol),
                     device="cuda", dtype=torch.uint8)
    # the forward runs with the backward's workspace and leaves its boundary states there
    f = mesa.fwd_chunked(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                         return_x=True, workspace=ws)
    res = mesa.bwd_chunked(q, k, v, gamma, beta, lam, f["x"], d_o, chunk=cfg.chunk,
                           max_steps=cfg.max_steps, tol=cfg.tol, workspace=ws, states_in_workspace=True)

    def step(kept):
        mesa.bwd_chunked(q, k, v, gamma, beta, lam, f["x"], d_o, chunk=cfg.chunk, max_steps=cfg.max_steps,
                         tol=cfg.tol, out=res, workspace=ws, states_in_workspace=kept)

    for _ in range(warmup):
        step(True)
    ms_kept = time_events(lambda: step(True), steps)
    ms = time_events(lambda: step(False), steps)
    tokens = cfg.B * cfg.H * cfg.T
    return {
        "workload": f"backward: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} {cfg.dtype}, "
                    f"{cfg.max_steps} CG steps per solve",
        "ms_per_call": round(ms, 4),
        "ms_per_call_states_kept": round(ms_kept, 4),
        "token_heads_per_s": round(tokens / (ms * 1e-3), 1),
    }


def bench_forward_full_lambda(cfg, steps, warmup):
    """The forward with a full symmetric positive definite Lambda per head: one
    mesa_fwd_chunked_ex call (scan, CG solve with the extra d x d product, read-out)."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_fwd_inputs, make_full_lambda

    x = make_fwd_inputs(cfg)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q, k, v = (torch.from_numpy(x[n]).cuda().to(dt) for n in ("q", "k", "v"))
    gamma, beta = (torch.from_numpy(x[n]).cuda() for n in ("gamma", "beta"))
    lam = torch.from_numpy(make_full_lambda(cfg.H, cfg.d, cfg.seed)).cuda()
    del x
    ws = torch.empty(mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, dtype=dt), device="cuda",
                     dtype=torch.uint8)
    res = mesa.fwd_chunked_ex(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                              workspace=ws)

    def step():
        mesa.fwd_chunked_ex(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                            workspace=ws, out=res)

    for _ in range(warmup):
        step()
    ms = time_events(step, steps)
    n_avg = float(res["steps"].float().mean().item())
    tokens = cfg.B * cfg.H * cfg.T
    # counted flops: the diagonal forward's plus the full Lambda's product per CG iteration
    f = flops_per_token(cfg.d, cfg.chunk, n_avg)["total"] + n_avg * 2 * cfg.d * cfg.d
    tflops = f * tokens / (ms * 1e-3) / 1e12
    # the backward with the same Lambda (adjoint solves with the full matrix, dLambda [H, d, d])
    x = mesa.fwd_chunked_ex(q, k, v, gamma, beta, lam, chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol,
                            return_x=True)["x"]
    d_o = torch.randn(x.shape, device="cuda", generator=torch.Generator(device="cuda").manual_seed(cfg.seed))
    wsb = torch.empty(mesa.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, cfg.max_steps, cfg.tol),
                      device="cuda", dtype=torch.uint8)
    gres = mesa.bwd_chunked_ex(q, k, v, gamma, beta, lam, x, d_o, chunk=cfg.chunk, max_steps=cfg.max_steps,
                               tol=cfg.tol, workspace=wsb)

    def bstep():
        mesa.bwd_chunked_ex(q, k, v, gamma, beta, lam, x, d_o, chunk=cfg.chunk, max_steps=cfg.max_steps,
                            tol=cfg.tol, workspace=wsb, out=gres)

    for _ in range(warmup):
        bstep()
    ms_b = time_events(bstep, steps)
    return {
        "workload": f"forward with a full SPD Lambda per head: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} "
                    f"{cfg.dtype}, chunk {cfg.chunk}, cg_steps_mean {n_avg:.1f}",
        "ms_per_call": round(ms, 4),
        "tokens_per_s": round(tokens / (ms * 1e-3), 1),
        "counted_TFLOPs": round(tflops, 2),
        "frac_of_mfma_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "backward_ms_per_call": round(ms_b, 4),
    }


def bench_preprocess(cfg, steps, warmup, window=4):
    """Query/key preprocessing (causal depthwise convolution + L2 norm) at the layer
    workload's shape: raw q, k read once, processed q, k written once."""
    import torch
    from test_regression_sequence_amd import mesa
    from test_regression_sequence_amd.inputs import make_preprocess_inputs

    x = make_preprocess_inputs(cfg, window)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    q = torch.from_numpy(x["q"]).cuda().to(dt)
    k = torch.from_numpy(x["k"]).cuda().to(dt)
    wq = torch.from_numpy(x["wq"]).cuda()
    wk = torch.from_numpy(x["wk"]).cuda()
    del x
    out = {"q": torch.empty_like(q), "k": torch.empty_like(k)}

    def step():
        mesa.qk_preprocess(q, k, wq, wk, out=out)

    for _ in range(warmup):
        step()
    ms = time_events(step, steps)
    esz = 2 if cfg.dtype == "bf16" else 4
    nbytes = 4 * cfg.B * cfg.H * cfg.T * cfg.d * esz + 2 * cfg.H * cfg.d * window * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    return {
        "workload": f"q/k preprocessing: B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} {cfg.dtype}, window {window}",
        "us_per_call": round(ms * 1e3, 2),
        "bytes_per_call": int(nbytes),
        "achieved_GBs": round(gbs, 1),
        "frac": round(gbs / PEAK_HBM_GBS, 4),
    }


def kernel_source_digest(names=("mesa_cg_bf16.hip", "mesa_common.h")) -> str:
    """sha256 over the sources of the CG kernel (ties a traffic record to one kernel version)."""
    import hashlib
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "test_regression_sequence_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def recorded_traffic(digest: str):
    """HBM bytes per CG launch from the committed counter summary, or None.

    The summary holds one line ``traffic_json: {...}`` with the FETCH_SIZE and
    WRITE_SIZE readings per dispatch, each already scaled by the factor a plain
    copy of known size gives for the same counter.  A record taken on another
    version of the kernel's sources does not count.
    """
    path = os.path.join(ROOT, "profiles", "cg_bf16_lm1b_d128_hbm_traffic.md")
    try:
        with open(path) as f:
            for line in f:
                if line.startswith("traffic_json:"):
                    rec = json.loads(line.split(":", 1)[1])
                    if rec.get("source_sha256") == digest:
                        return rec
    except OSError:
        pass
    return None


def calibrate_copy(mib: int, reps: int):
    """A plain device copy of known size, for scaling the HBM byte counters."""
    import torch
    n = mib * (1 << 20) // 4
    a = torch.ones(n, device="cuda")
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(reps):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calibration": "copy", "bytes_read_per_launch": 4 * n,
                      "bytes_written_per_launch": 4 * n, "launches": reps}), flush=True)


def measure_copy_bw(mib: int = 512, copies: int = 3, reps: int = 10) -> float:
    """Read + write rate (GB/s) of a plain device copy, over three rotating
    buffer pairs so that no copy finds its source in the last-level cache: the
    practical HBM rate the memory-bound kernels are compared with."""
    import itertools
    import torch
    n = mib * (1 << 20) // 4
    src = [torch.ones(n, device="cuda") for _ in range(copies)]
    dst = [torch.empty(n, device="cuda") for _ in range(copies)]
    ctr = itertools.count()

    def one():
        i = next(ctr) % copies
        dst[i].copy_(src[i])

    for _ in range(copies):
        one()
    ms = time_events(one, reps)
    del src, dst
    return 2 * 4 * n / (ms * 1e-3) / 1e9


def _oracle_slice(args):
    """One (b, h) slice of the oracle's forward (CG schedule only), in a worker."""
    from threadpoolctl import threadpool_limits
    from oracle import mesa_forward
    q, k, v, gamma, beta, lam, max_steps, tol = args
    with threadpool_limits(1):
        mesa_forward(q, k, v, gamma, beta, lam, max_steps=max_steps, tol=tol, exact=False)
    return q.shape[2]


def host_workers() -> int:
    """Host cores this process may use, at most 16 (one GPU's share of its host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def cpu_baseline(x, per_worker: int, tokens: int):
    """The fp64 oracle, untuned, over the host's cores: one worker process per
    core, each running whole (b, h) slices with one BLAS thread.  Runs before
    the GPU is initialised, so the workers are plain forks."""
    import multiprocessing as mp
    cfg = x["cfg"]
    workers = host_workers()
    slices = min(cfg.B * cfg.H, workers * per_worker)
    rng = np.random.default_rng(7)
    flat = rng.choice(cfg.B * cfg.H, size=slices, replace=False)
    b, h = flat // cfg.H, flat % cfg.H
    T = min(tokens, cfg.T)
    jobs = [(x["q"][b[i], h[i]][None, None, :T], x["k"][b[i], h[i]][None, None, :T],
             x["v"][b[i], h[i]][None, None, :T], x["gamma"][b[i], h[i]][None, None, :T],
             x["beta"][b[i], h[i]][None, None, :T], x["lam"][h[i]][None], cfg.max_steps, cfg.tol)
            for i in range(slices)]
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        pool.map(_oracle_slice, jobs[:workers])          # warm: imports in every worker
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_slice, jobs, chunksize=1))
        dt = time.perf_counter() - t0
    return {
        "value": round(done / dt, 2),
        "unit": "tokens/s",
        "cores": workers,
        "kind": "oracle",
        "sample": f"{slices} (b,h) slices x first {T} tokens of the same workload, fp64 NumPy, CG schedule "
                  f"only (no exact solve), {workers} worker processes with one BLAS thread each; {dt:.1f} s wall, "
                  f"{dt * workers:.0f} core-s",
        "host": cpu_model(),
        "host_cpus": os.cpu_count(),
    }


def _oracle_decode(args):
    """One block of (sequence, head) pairs of the oracle's decode step, in a worker."""
    from threadpoolctl import threadpool_limits
    from oracle import mesa_decode_step
    q, k, v, gamma, beta, lam, h, g, max_steps, tol = args
    with threadpool_limits(1):
        mesa_decode_step(q, k, v, gamma, beta, lam, h, g, max_steps=max_steps, tol=tol)
    return q.shape[0] * q.shape[1]


def cpu_other_workloads() -> dict:
    """The oracle (CG schedule, fp64) on the other workloads, over the host's
    cores like the main baseline: workloads 1 and 2 in full (every slice), the
    decode step on 32 sequences x 16 heads drawn with workload 5's
    distributions.  A reported baseline, not a target."""
    import multiprocessing as mp
    from test_regression_sequence_amd.inputs import CONFIGS, make_decode_inputs, make_fwd_inputs
    workers = host_workers()
    out = {}
    ctx = mp.get_context("fork")
    with ctx.Pool(workers) as pool:
        for key, c in (("tiny_fp32", 1), ("mid_d64", 2)):
            cfg = CONFIGS[c]
            x = make_fwd_inputs(cfg)
            jobs = [(x["q"][b, h][None, None].astype(np.float64), x["k"][b, h][None, None].astype(np.float64),
                     x["v"][b, h][None, None].astype(np.float64), x["gamma"][b, h][None, None],
                     x["beta"][b, h][None, None], x["lam"][h][None], cfg.max_steps, cfg.tol)
                    for b in range(cfg.B) for h in range(cfg.H)]
            pool.map(_oracle_slice, jobs[:1])
            t0 = time.perf_counter()
            done = sum(pool.map(_oracle_slice, jobs, chunksize=1))
            dt = time.perf_counter() - t0
            out[key] = {"value": round(done / dt, 2), "unit": "tokens/s", "cores": workers, "kind": "oracle",
                        "sample": f"the whole workload ({len(jobs)} (b,h) slices x {cfg.T} tokens), CG schedule; "
                                  f"{dt:.2f} s wall"}
        cfg = CONFIGS[5].replace(N=32)
        x = make_decode_inputs(cfg)
        P = 4  # pairs per job, all of one head (the oracle takes one lambda per head of its batch)
        jobs = []
        for h in range(cfg.H):
            for n0 in range(0, cfg.N, P):
                ns = np.arange(n0, min(n0 + P, cfg.N))
                jobs.append(tuple(x[key_][ns, h][:, None] for key_ in ("q", "k", "v", "gamma", "beta"))
                            + (x["lam"][h][None], x["h"][ns, h][:, None], x["g"][ns, h][:, None],
                               cfg.max_steps, cfg.tol))
        pool.map(_oracle_decode, jobs[:1])
        t0 = time.perf_counter()
        done = sum(pool.map(_oracle_decode, jobs, chunksize=1))
        dt = time.perf_counter() - t0
        out["decode"] = {"value": round(done / dt, 2), "unit": "pairs/s", "cores": workers, "kind": "oracle",
                         "sample": f"{done} (sequence, head) pairs of workload 5's distributions (32 sequences), "
                                   f"one decode step each, CG schedule; {dt:.2f} s wall"}
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", type=int, default=3, choices=[2, 3, 4],
                    help="forward workload: 2 (d=64), 3 (d=128, default), 4 (T=32768, dynamic CG)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--forward-only", action="store_true",
                    help="time the chosen forward workload only (profiling runs)")
    ap.add_argument("--prep-forward", action="store_true",
                    help="also time the forward on raw q/k: preprocessing kernel + forward against the fused call")
    ap.add_argument("--backward", action="store_true",
                    help="with --forward-only: also time the backward pass")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-slices-per-core", type=int, default=4)
    ap.add_argument("--cpu-tokens", type=int, default=4096)
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device copy of MIB MiB (counter calibration) and exit")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: the Mesa layer's (b, h) slices shard across GPUs "
              "with no communication, and this benchmark runs and reports a single MI355X. "
              "Run with --gpus 1.", file=sys.stderr)
        sys.exit(2)

    from test_regression_sequence_amd.inputs import CONFIGS, make_fwd_inputs

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    cfg = CONFIGS[args.workload]
    x_main = None
    cpu = None
    cpu_other = None
    if not args.no_cpu_baseline and not args.calibrate_copy:
        # before any HIP call: the oracle's worker processes are plain forks
        x_main = make_fwd_inputs(cfg)
        cpu = cpu_baseline(x_main, args.cpu_slices_per_core, args.cpu_tokens)
        log(f"cpu baseline: {cpu['value']} tokens/s on {cpu['cores']} cores")
        if not args.forward_only:
            cpu_other = cpu_other_workloads()
            log(f"cpu baseline, other workloads: {cpu_other}")

    import torch
    from test_regression_sequence_amd import mesa

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.calibrate_copy:
        calibrate_copy(args.calibrate_copy, max(1, args.steps))
        return
    mesa.lib()

    fw = bench_forward(cfg, args.steps, args.warmup, x_main, clock=True)
    x_main = None
    log(f"forward: {fw['ms']:.4f} ms per call")
    tokens = cfg.B * cfg.H * cfg.T
    n_avg = fw["steps_mean"]
    f = flops_per_token(cfg.d, cfg.chunk, n_avg)
    cg_flops = f["cg_kernel"] * tokens
    cg_tflops = cg_flops / (fw["cg_ms"] * 1e-3) / 1e12
    total_tflops = f["total"] * tokens / (fw["ms"] * 1e-3) / 1e12
    traffic = None
    rec = recorded_traffic(kernel_source_digest()) if cfg.name == "lm1b-d128-bf16" else None
    if rec is not None:
        traffic = int(rec["fetch_bytes_per_launch"] + rec["write_bytes_per_launch"])

    line = {
        "metric": f"Mesa fwd tokens/s (B*H*T/s) at d={cfg.d}",
        "value": round(tokens / (fw["ms"] * 1e-3), 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(fw["ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if cfg.dtype == "bf16" else "f32",
        "data": "synthetic (seeded; q,k L2-normalised Gaussian, v Gaussian, gamma=sigmoid(U), beta~U(0,1))",
        "config": {
            "workload": f"{cfg.name}: chunked Mesa forward B={cfg.B} H={cfg.H} T={cfg.T} d={cfg.d} "
                        f"chunk={cfg.chunk}, {'fixed %d' % cfg.max_steps if cfg.tol <= 0 else 'tol %g max %d' % (cfg.tol, cfg.max_steps)} CG steps",
            "B": cfg.B, "H": cfg.H, "T": cfg.T, "d": cfg.d, "chunk": cfg.chunk,
            "cg_steps_mean": round(n_avg, 3),
        },
        "roofline": {
            "kernel": "cg_kernel (chunked CG solve + read-out)",
            "bound": "mfma",
            "achieved": round(cg_tflops, 2),
            "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s",
            "frac": round(cg_tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "flops_per_launch": cg_flops,
            "avg_launch_ms": round(fw["cg_ms"], 4),
        },
        "clock": clock_report(fw["clock"], cg_tflops),
        "kernels_ms": {"scan": round(fw["scan_ms"], 4), "cg": round(fw["cg_ms"], 4)},
        "fwd_counted_TFLOPs": round(total_tflops, 2),
        "fwd_frac_of_mfma_peak": round(total_tflops / PEAK_BF16_TFLOPS, 4),
        "wall_ms_per_step": round(fw["wall_ms"], 4),
    }
    if args.prep_forward:
        line["forward_with_preprocessing"] = bench_prep_forward(cfg, args.steps, args.warmup)
        log(f"forward with preprocessing: {line['forward_with_preprocessing']}")
    if args.backward and args.forward_only:
        line["backward"] = bench_backward(cfg, args.steps, args.warmup)
        log(f"backward: {line['backward']['ms_per_call']} ms per call")
    if args.forward_only:
        line["forward_detail"] = forward_report(cfg, fw)
        if cpu is not None:
            line["cpu_baseline"] = cpu
        print(json.dumps(line), flush=True)
        return
    copy_gbs = measure_copy_bw()
    line["measured_peaks"] = {"torch_copy_GBs": round(copy_gbs, 1),
                              "note": "torch device copy of 512 MiB (read + write bytes), three rotating "
                                      "buffer pairs: a reference rate, not a ceiling"}
    log(f"device copy: {copy_gbs:.0f} GB/s")
    if not args.no_decode:
        line["decode"] = bench_decode(CONFIGS[5], args.steps, args.warmup)
        line["decode"]["vs_torch_copy"] = round(line["decode"]["achieved_GBs"] / copy_gbs, 4)
        log(f"decode: {line['decode']['us_per_step']} us per step")
    line["preprocess"] = bench_preprocess(CONFIGS[args.workload], args.steps, args.warmup)
    line["preprocess"]["vs_torch_copy"] = round(line["preprocess"]["achieved_GBs"] / copy_gbs, 4)
    log(f"preprocess: {line['preprocess']['us_per_call']} us per call")
    if "forward_with_preprocessing" not in line:
        line["forward_with_preprocessing"] = bench_prep_forward(cfg, args.steps, args.warmup)
        log(f"forward with preprocessing: {line['forward_with_preprocessing']}")
    line["backward"] = bench_backward(CONFIGS[args.workload], args.steps, args.warmup)
    log(f"backward: {line['backward']['ms_per_call']} ms per call")
    cfg_w = CONFIGS[args.workload]
    if cfg_w.dtype == "bf16" and cfg_w.chunk == 64 and cfg_w.d in (64, 128):
        line["forward_full_lambda"] = bench_forward_full_lambda(cfg_w, args.steps, args.warmup)
        log(f"forward, full Lambda: {line['forward_full_lambda']['ms_per_call']} ms per call")
    # the other forward workloads: latency (1), mid size (2), long context with dynamic CG (4)
    others = {}
    others["tiny_fp32"] = bench_latency(CONFIGS[1], args.steps, args.warmup)
    log(f"tiny fp32: {others['tiny_fp32']['us_per_call']} us per call")
    for key, c in (("mid_d64", 2), ("long_dynamic", 4)):
        if c == args.workload:
            continue
        fwc = bench_forward(CONFIGS[c], args.steps, args.warmup)
        fwc.pop("x")
        others[key] = forward_report(CONFIGS[c], fwc)
        log(f"workload {c}: {others[key]['ms_per_call']} ms per call")
    line["other_workloads"] = others
    line["warm_start_forward"] = bench_warm_forward(CONFIGS[4], args.steps, args.warmup)
    log(f"warm-start forward: {line['warm_start_forward']['workload_queries']}")
    line["forward_detail"] = forward_report(cfg, fw)
    if cpu is not None:
        line["cpu_baseline"] = cpu
    if cpu_other is not None:
        line["cpu_baseline_other_workloads"] = cpu_other
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
