"""Seeded synthetic inputs for the Mesa layer forward and decode step.

This module only draws random numbers and shapes them.  It performs none of
the layer's own arithmetic on the values it hands out (no state update, no
solve, no output), so both the HIP path and the fp64 oracle can consume the
same draws without sharing any of the method's code.  The one exception is
documented at :func:`make_decode_inputs`: a pre-filled decode state is a
weighted Gram matrix of random tokens, which is how such a state is
distributed; it is an input to the decode step, never a result compared by a
test.

Workloads (method: MesaNet, "Sequence Modeling by Locally Optimal Test-Time
Training", technical summary, Mesa layer section):

* q, k ~ N(0, 1), then each token vector L2-normalised (the architecture
  section normalises queries and keys before the layer);
* v ~ N(0, 1);
* gamma_t = sigmoid(u), u ~ U(lo, hi) -- the forget factor of each token;
* beta_t  ~ U(0, 1) or Beta(a, b) -- the write strength of each token;
* Lambda  = diag(lambda), either a constant or drawn per (head, dim).

bf16 inputs are produced as: draw in fp64 -> normalise -> cast to fp32 ->
round to nearest even bf16.  Arrays returned here always hold float32 values;
for bf16 configurations those values are exactly representable in bf16, and
``*_bits`` holds the raw uint16 encodings.
"""
from __future__ import annotations

import concurrent.futures
import dataclasses
import os
from typing import Optional

import numpy as np

__all__ = [
    "FwdConfig", "DecodeConfig", "CONFIGS", "make_fwd_inputs", "make_fwd_inputs_device",
    "make_decode_inputs_device",
    "make_decode_inputs", "make_decode_stream", "make_preprocess_inputs", "make_bwd_inputs",
    "make_full_lambda", "make_slow_queries", "round_to_bf16",
    "bf16_bits", "bits_to_f32",
]


@dataclasses.dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    T: int
    d: int
    chunk: int
    dtype: str                  # "f32" or "bf16": dtype of q, k, v
    gamma_logit: tuple          # (lo, hi) of u, gamma = sigmoid(u)
    beta_dist: tuple            # ("uniform", lo, hi) or ("beta", a, b)
    lam_dist: tuple             # ("const", c) or ("uniform", lo, hi) per (head, dim)
    max_steps: int
    tol: float                  # <= 0: fixed max_steps
    seed: int

    @property
    def tokens(self) -> int:
        return self.B * self.H * self.T

    def replace(self, **kw) -> "FwdConfig":
        return dataclasses.replace(self, **kw)


@dataclasses.dataclass(frozen=True)
class DecodeConfig:
    name: str
    N: int                      # sequences
    H: int
    d: int
    prefill: int                # tokens folded into the starting state
    dtype: str
    gamma_logit: tuple
    beta_dist: tuple
    lam_dist: tuple
    max_steps: int
    tol: float
    seed: int

    def replace(self, **kw) -> "DecodeConfig":
        return dataclasses.replace(self, **kw)


_LM_GATES = dict(gamma_logit=(2.0, 6.0), beta_dist=("uniform", 0.0, 1.0))

CONFIGS = {
    1: FwdConfig("tiny-f32", B=1, H=1, T=256, d=16, chunk=64, dtype="f32",
                 lam_dist=("const", 1.0), max_steps=16, tol=1e-6, seed=0, **_LM_GATES),
    2: FwdConfig("mid-d64-bf16", B=4, H=8, T=2048, d=64, chunk=64, dtype="bf16",
                 lam_dist=("uniform", 0.25, 1.0), max_steps=15, tol=0.0, seed=1, **_LM_GATES),
    3: FwdConfig("lm1b-d128-bf16", B=8, H=16, T=4096, d=128, chunk=64, dtype="bf16",
                 lam_dist=("uniform", 0.25, 1.0), max_steps=30, tol=0.0, seed=2, **_LM_GATES),
    4: FwdConfig("long-dynamic-d128-bf16", B=1, H=16, T=32768, d=128, chunk=64, dtype="bf16",
                 gamma_logit=(4.0, 9.0), beta_dist=("beta", 5.0, 1.0),
                 lam_dist=("const", 0.25), max_steps=64, tol=1e-4, seed=3),
    5: DecodeConfig("decode-d128", N=256, H=16, d=128, prefill=1024, dtype="bf16",
                    lam_dist=("uniform", 0.25, 1.0), max_steps=32, tol=1e-4, seed=4,
                    **_LM_GATES),
}


# ----------------------------------------------------------------------------
# bf16 helpers (round to nearest, ties to even, on the fp32 bit pattern)
# ----------------------------------------------------------------------------

def bf16_bits(x32: np.ndarray) -> np.ndarray:
    """uint16 bf16 encodings of fp32 values, rounded to nearest even."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    r = u + np.uint32(0x7FFF) + lsb
    bits = (r >> np.uint32(16)).astype(np.uint16)
    nan = np.isnan(x32)
    if nan.any():
        bits[nan] = np.uint16(0x7FC0)
    return bits


def bits_to_f32(bits: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def round_to_bf16(x32: np.ndarray) -> np.ndarray:
    """fp32 values rounded to the nearest bf16, returned as fp32."""
    return bits_to_f32(bf16_bits(x32))


# ----------------------------------------------------------------------------
# draws
# ----------------------------------------------------------------------------

def _unit_gauss(rng: np.random.Generator, shape) -> np.ndarray:
    x = rng.standard_normal(shape)
    x /= np.linalg.norm(x, axis=-1, keepdims=True)
    return x


def _beta(rng, dist, shape):
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], shape)
    if dist[0] == "beta":
        return rng.beta(dist[1], dist[2], shape)
    raise ValueError(dist)


def _lam(rng, dist, H, d):
    if dist[0] == "const":
        return np.full((H, d), float(dist[1]))
    if dist[0] == "uniform":
        return rng.uniform(dist[1], dist[2], (H, d))
    raise ValueError(dist)


def _finish(x64: np.ndarray, dtype: str):
    x32 = x64.astype(np.float32)
    if dtype == "bf16":
        bits = bf16_bits(x32)
        return bits_to_f32(bits), bits
    return x32, None


def make_fwd_inputs(cfg: FwdConfig) -> dict:
    """Inputs of one chunked-forward workload.

    Draw order (one ``numpy.random.default_rng(seed)`` stream): q, k, v, u,
    beta, lambda.  Shapes: q, k, v ``[B, H, T, d]``; gamma, beta ``[B, H, T]``;
    lam ``[H, d]`` (the diagonal of Lambda per head).
    """
    rng = np.random.default_rng(cfg.seed)
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    q, qb = _finish(_unit_gauss(rng, shp), cfg.dtype)
    k, kb = _finish(_unit_gauss(rng, shp), cfg.dtype)
    v, vb = _finish(rng.standard_normal(shp), cfg.dtype)
    u = rng.uniform(cfg.gamma_logit[0], cfg.gamma_logit[1], shp[:3])
    gamma = (1.0 / (1.0 + np.exp(-u))).astype(np.float32)
    beta = _beta(rng, cfg.beta_dist, shp[:3]).astype(np.float32)
    lam = _lam(rng, cfg.lam_dist, cfg.H, cfg.d).astype(np.float32)
    out = dict(q=q, k=k, v=v, gamma=gamma, beta=beta, lam=lam, cfg=cfg)
    if cfg.dtype == "bf16":
        out.update(q_bits=qb, k_bits=kb, v_bits=vb)
    return out


def make_fwd_inputs_device(cfg: FwdConfig, device="cuda") -> dict:
    """The inputs of a forward workload drawn on the device, for sizes whose host
    copies would not fit (billions of elements): the distributions of
    :func:`make_fwd_inputs`, drawn in the same order from torch's seeded
    generator on ``device`` instead of NumPy's.  q, k, v come back in the
    config's dtype (bf16 or fp32), gamma, beta, lam in fp32; every value is
    exactly representable in its dtype, so a slice copied to the host (as
    float64) is the same input for the oracle."""
    import torch

    if cfg.beta_dist[0] != "uniform":
        raise ValueError("device generator: uniform beta only")
    g = torch.Generator(device=device)
    g.manual_seed(cfg.seed)
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def unit_gauss():
        x = torch.randn(shp, generator=g, device=device)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dt)

    q = unit_gauss()
    k = unit_gauss()
    v = torch.randn(shp, generator=g, device=device).to(dt)
    lo, hi = cfg.gamma_logit
    gamma = torch.sigmoid(torch.rand(shp[:3], generator=g, device=device) * (hi - lo) + lo)
    blo, bhi = cfg.beta_dist[1], cfg.beta_dist[2]
    beta = torch.rand(shp[:3], generator=g, device=device) * (bhi - blo) + blo
    lam = torch.from_numpy(_lam(np.random.default_rng(cfg.seed), cfg.lam_dist, cfg.H, cfg.d).astype(np.float32))
    return dict(q=q, k=k, v=v, gamma=gamma, beta=beta, lam=lam.to(device), cfg=cfg)


def make_decode_inputs_device(cfg: DecodeConfig, device="cuda", rank: int = 8) -> dict:
    """A decode step's inputs drawn on the device, for state arrays of billions
    of elements: q, k, v, gamma, beta, lambda as in :func:`make_decode_inputs`
    (torch's seeded generator in place of NumPy's), and starting states of the
    same scale without a prefill pass: h = W W^T / rank + 0.05 I with W
    [d, rank] Gaussian per pair (symmetric positive semidefinite plus a ridge),
    g Gaussian times 0.1.  Every value is exact in its dtype."""
    import torch

    if cfg.beta_dist[0] != "uniform":
        raise ValueError("device generator: uniform beta only")
    gen = torch.Generator(device=device)
    gen.manual_seed(cfg.seed)
    shp = (cfg.N, cfg.H, cfg.d)
    dt = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32

    def unit_gauss():
        x = torch.randn(shp, generator=gen, device=device)
        x /= torch.linalg.vector_norm(x, dim=-1, keepdim=True)
        return x.to(dt)

    q = unit_gauss()
    k = unit_gauss()
    v = torch.randn(shp, generator=gen, device=device).to(dt)
    lo, hi = cfg.gamma_logit
    gamma = torch.sigmoid(torch.rand(shp[:2], generator=gen, device=device) * (hi - lo) + lo)
    blo, bhi = cfg.beta_dist[1], cfg.beta_dist[2]
    beta = torch.rand(shp[:2], generator=gen, device=device) * (bhi - blo) + blo
    lam = torch.from_numpy(_lam(np.random.default_rng(cfg.seed), cfg.lam_dist, cfg.H, cfg.d).astype(np.float32))
    pairs = cfg.N * cfg.H
    w = torch.randn((pairs, cfg.d, rank), generator=gen, device=device)
    h = torch.bmm(w, w.transpose(1, 2).contiguous()) / rank
    del w
    h.diagonal(dim1=1, dim2=2).add_(0.05)
    g = torch.randn((pairs, cfg.d, cfg.d), generator=gen, device=device) * 0.1
    return dict(q=q, k=k, v=v, gamma=gamma, beta=beta, lam=lam.to(device),
                h=h.view(cfg.N, cfg.H, cfg.d, cfg.d), g=g.view(cfg.N, cfg.H, cfg.d, cfg.d), cfg=cfg)


def make_slow_queries(x: dict, rho1: float) -> dict:
    """A forward workload whose queries drift slowly along each sequence.

    q_t = rho1 q_{t-1} + sqrt(1 - rho1^2) e_t per dimension (e ~ N(0, 1),
    q_0 = e_0), then L2-normalised per token and rounded like the workload's
    other q (stream ``default_rng([seed, 6])``).  Keys, values, gates and
    Lambda are the workload's.  A stand-in for queries that change smoothly
    from token to token; the pages say nothing about query statistics.
    """
    cfg = x["cfg"]
    rng = np.random.default_rng([cfg.seed, 6])
    e = rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.d))
    q = np.empty_like(e)
    q[:, :, 0] = e[:, :, 0]
    c = np.sqrt(1.0 - rho1 * rho1)
    for t in range(1, cfg.T):
        q[:, :, t] = rho1 * q[:, :, t - 1] + c * e[:, :, t]
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    q32, qb = _finish(q, cfg.dtype)
    out = dict(x, q=q32)
    if cfg.dtype == "bf16":
        out["q_bits"] = qb
    return out


def _prefill_block(seed: int, block: int, P: int, prefill: int, d: int,
                   gamma_logit, beta_dist, dtype: str):
    """Random prefix tokens for P (sequence, head) pairs and their state.

    The state is the weighted Gram matrix of the prefix: H = sum_j w_j k_j k_j^T,
    G = sum_j w_j v_j k_j^T with w_j = beta_j * prod_{i>j} gamma_i, i.e. what a
    zero state becomes after absorbing the prefix.  It is drawn here as an
    *input* of the decode step (a structured random SPD matrix), in fp64, then
    symmetrised and cast to fp32.
    """
    rng = np.random.default_rng([seed, 1, block])
    k, _ = _finish(_unit_gauss(rng, (P, prefill, d)), dtype)
    v, _ = _finish(rng.standard_normal((P, prefill, d)), dtype)
    u = rng.uniform(gamma_logit[0], gamma_logit[1], (P, prefill))
    gamma = (1.0 / (1.0 + np.exp(-u))).astype(np.float32).astype(np.float64)
    beta = _beta(rng, beta_dist, (P, prefill)).astype(np.float32).astype(np.float64)
    # survival of token j to the end of the prefix: prod_{i=j+1}^{L-1} gamma_i
    logg = np.log(gamma)
    surv = np.exp(np.cumsum(logg[:, ::-1], axis=1)[:, ::-1] - logg)
    w = beta * surv
    k64 = k.astype(np.float64)
    v64 = v.astype(np.float64)
    kw = k64 * w[:, :, None]
    Hs = np.matmul(kw.transpose(0, 2, 1), k64)
    Gs = np.matmul(v64.transpose(0, 2, 1), kw)
    Hs = 0.5 * (Hs + Hs.transpose(0, 2, 1))
    return Hs.astype(np.float32), Gs.astype(np.float32)


def make_decode_inputs(cfg: DecodeConfig, block: int = 64) -> dict:
    """Inputs of one recurrent decode step.

    The new token's q, k, v, u, beta and lambda come from
    ``default_rng(seed)`` in that order; the starting states of the pairs come
    from independent streams ``default_rng([seed, 1, b])`` per block ``b`` of
    ``block`` consecutive (sequence, head) pairs, so memory stays bounded.
    Shapes: q, k, v ``[N, H, d]``; gamma, beta ``[N, H]``; lam ``[H, d]``;
    h, g ``[N, H, d, d]`` fp32 (row-major, ``g[n][k]`` = value dim n, key dim k).
    """
    rng = np.random.default_rng(cfg.seed)
    shp = (cfg.N, cfg.H, cfg.d)
    q, qb = _finish(_unit_gauss(rng, shp), cfg.dtype)
    k, kb = _finish(_unit_gauss(rng, shp), cfg.dtype)
    v, vb = _finish(rng.standard_normal(shp), cfg.dtype)
    u = rng.uniform(cfg.gamma_logit[0], cfg.gamma_logit[1], shp[:2])
    gamma = (1.0 / (1.0 + np.exp(-u))).astype(np.float32)
    beta = _beta(rng, cfg.beta_dist, shp[:2]).astype(np.float32)
    lam = _lam(rng, cfg.lam_dist, cfg.H, cfg.d).astype(np.float32)
    pairs = cfg.N * cfg.H
    h = np.empty((pairs, cfg.d, cfg.d), np.float32)
    g = np.empty((pairs, cfg.d, cfg.d), np.float32)
    if cfg.prefill > 0:
        def work(b0):
            P = min(block, pairs - b0)
            hb, gb = _prefill_block(cfg.seed, b0 // block, P, cfg.prefill, cfg.d,
                                    cfg.gamma_logit, cfg.beta_dist, cfg.dtype)
            h[b0:b0 + P] = hb
            g[b0:b0 + P] = gb
        # blocks draw from independent streams, so the thread count does not change the result
        workers = max(1, min(16, os.cpu_count() or 1))
        try:
            from threadpoolctl import threadpool_limits
            limit = threadpool_limits(1)
        except ImportError:  # pragma: no cover
            limit = None
        try:
            with concurrent.futures.ThreadPoolExecutor(workers) as ex:
                list(ex.map(work, range(0, pairs, block)))
        finally:
            if limit is not None:
                limit.restore_original_limits()
    else:
        h[:] = 0
        g[:] = 0
    out = dict(q=q, k=k, v=v, gamma=gamma, beta=beta, lam=lam,
               h=h.reshape(cfg.N, cfg.H, cfg.d, cfg.d),
               g=g.reshape(cfg.N, cfg.H, cfg.d, cfg.d), cfg=cfg)
    if cfg.dtype == "bf16":
        out.update(q_bits=qb, k_bits=kb, v_bits=vb)
    return out


def make_decode_stream(cfg: DecodeConfig, T: int, rho: float = 0.75) -> dict:
    """T consecutive new tokens for the decode step, neighbouring queries and keys related.

    Queries and keys follow a Gaussian AR(1) process per (pair, dim),
    z_t = rho z_{t-1} + sqrt(1 - rho^2) eps_t, each token then L2-normalised:
    consecutive tokens correlate like the outputs of a short causal filter
    (rho = 0.75 is the lag-1 correlation of a 4-tap moving average of
    independent vectors).  v ~ N(0, 1), gamma and beta as in
    :func:`make_decode_inputs`, independent per token.  Stream:
    ``default_rng([seed, 2])`` drawing z_0 and eps for q, then for k, then v,
    u, beta.  Shapes: q, k, v ``[N, H, T, d]``; gamma, beta ``[N, H, T]``.
    Lambda and the starting states are those of ``make_decode_inputs(cfg)``.
    """
    rng = np.random.default_rng([cfg.seed, 2])
    shp = (cfg.N, cfg.H, T, cfg.d)

    def ar1():
        z = np.empty(shp)
        z[:, :, 0] = rng.standard_normal(shp[:2] + (cfg.d,))
        eps = rng.standard_normal((cfg.N, cfg.H, T - 1, cfg.d)) if T > 1 else None
        for t in range(1, T):
            z[:, :, t] = rho * z[:, :, t - 1] + np.sqrt(1.0 - rho * rho) * eps[:, :, t - 1]
        return z / np.linalg.norm(z, axis=-1, keepdims=True)

    q, _ = _finish(ar1(), cfg.dtype)
    k, _ = _finish(ar1(), cfg.dtype)
    v, _ = _finish(rng.standard_normal(shp), cfg.dtype)
    u = rng.uniform(cfg.gamma_logit[0], cfg.gamma_logit[1], shp[:3])
    gamma = (1.0 / (1.0 + np.exp(-u))).astype(np.float32)
    beta = _beta(rng, cfg.beta_dist, shp[:3]).astype(np.float32)
    return dict(q=q, k=k, v=v, gamma=gamma, beta=beta, cfg=cfg)


def make_preprocess_inputs(cfg: FwdConfig, window: int = 4) -> dict:
    """Raw queries and keys, and convolution taps, for the query/key preprocessing.

    Raw q, k ~ N(0, 1) (not normalised: the preprocessing normalises),
    ``[B, H, T, d]`` in the configuration's dtype; taps wq, wk ``[H, d, window]``
    fp32 ~ U(-1/sqrt(window), 1/sqrt(window)) (the usual initialisation of a
    depthwise convolution); raw histories hq, hk ``[B, H, window-1, d]`` ~ N(0, 1)
    for calls that continue a sequence.  Stream: ``default_rng([seed, 3])``
    in the order q, k, wq, wk, hq, hk, drawn in fp32.
    """
    rng = np.random.default_rng([cfg.seed, 3])
    shp = (cfg.B, cfg.H, cfg.T, cfg.d)
    q, _ = _finish(rng.standard_normal(shp, dtype=np.float32), cfg.dtype)
    k, _ = _finish(rng.standard_normal(shp, dtype=np.float32), cfg.dtype)
    a = 1.0 / np.sqrt(window)
    wq = rng.uniform(-a, a, (cfg.H, cfg.d, window)).astype(np.float32)
    wk = rng.uniform(-a, a, (cfg.H, cfg.d, window)).astype(np.float32)
    hshp = (cfg.B, cfg.H, window - 1, cfg.d)
    hq, _ = _finish(rng.standard_normal(hshp, dtype=np.float32), cfg.dtype)
    hk, _ = _finish(rng.standard_normal(hshp, dtype=np.float32), cfg.dtype)
    return dict(q=q, k=k, wq=wq, wk=wk, hq=hq, hk=hk, window=window, cfg=cfg)


def make_bwd_inputs(cfg: FwdConfig) -> dict:
    """Upstream gradients and initial states for the backward pass.

    d_o ~ N(0, 1) ``[B, H, T, d]``; d_hfinal, d_gfinal ~ N(0, 0.1^2)
    ``[B, H, d, d]``; initial states h0 = M M^T / d (M ~ N(0, 1), symmetric
    positive semi-definite) and g0 ~ N(0, 0.1^2).  All fp32.  Stream:
    ``default_rng([seed, 4])`` in the order d_o, d_hfinal, d_gfinal, M, g0.
    """
    rng = np.random.default_rng([cfg.seed, 4])
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    d_o = rng.standard_normal((B, H, T, d), dtype=np.float32)
    d_hfinal = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    d_gfinal = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    M = rng.standard_normal((B, H, d, d))
    h0 = np.matmul(M, M.transpose(0, 1, 3, 2)) / d
    h0 = (0.5 * (h0 + h0.transpose(0, 1, 3, 2))).astype(np.float32)
    g0 = (0.1 * rng.standard_normal((B, H, d, d))).astype(np.float32)
    return dict(d_o=d_o, d_hfinal=d_hfinal, d_gfinal=d_gfinal, h0=h0, g0=g0)


def make_full_lambda(H: int, d: int, seed: int) -> np.ndarray:
    """A full symmetric positive definite Lambda per head, ``[H, d, d]`` fp32.

    Lambda = 0.5 M M^T / d + diag(u), M ~ N(0, 1), u ~ U(0.25, 1): the
    diagonal distribution of the workloads plus a random positive semi-definite
    coupling, symmetrised after the fp32 cast.  Stream ``default_rng([seed, 5])``
    in the order M, u.
    """
    rng = np.random.default_rng([seed, 5])
    M = rng.standard_normal((H, d, d))
    u = rng.uniform(0.25, 1.0, (H, d))
    lam = 0.5 * np.matmul(M, M.transpose(0, 2, 1)) / d
    idx = np.arange(d)
    lam[:, idx, idx] += u
    lam = lam.astype(np.float32)
    return (0.5 * (lam + lam.transpose(0, 2, 1))).astype(np.float32)


def small_fwd(B=1, H=2, T=200, d=64, chunk=64, dtype="bf16", max_steps=8, tol=0.0,
              seed=123, lam=("uniform", 0.25, 1.0), gamma_logit=(2.0, 6.0),
              beta=("uniform", 0.0, 1.0)) -> FwdConfig:
    """A small workload with the language-model distributions (parity sizes)."""
    return FwdConfig(f"small-B{B}H{H}T{T}d{d}c{chunk}-{dtype}", B=B, H=H, T=T, d=d,
                     chunk=chunk, dtype=dtype, gamma_logit=gamma_logit, beta_dist=beta,
                     lam_dist=lam, max_steps=max_steps, tol=tol, seed=seed)


def select_slices(B: int, H: int, count: int, seed: int = 99) -> np.ndarray:
    """A fixed random subset of (b, h) slice indices (flattened b*H + h)."""
    rng = np.random.default_rng([seed, B, H])
    n = min(count, B * H)
    return np.sort(rng.choice(B * H, size=n, replace=False))
