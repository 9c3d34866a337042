"""Shared test utilities: moving seeded inputs to the GPU and error metrics."""
import numpy as np
import torch


def rel_l2(a, b) -> float:
    """||a - b||_F / ||b||_F in fp64 (1.0 denominator when b == 0)."""
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    den = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / (den if den > 0 else 1.0))


def dev_inputs(x: dict, device="cuda") -> dict:
    """torch device tensors of a generator dict (bf16 q/k/v when the config is bf16)."""
    cfg = x["cfg"]
    qkv_dtype = torch.bfloat16 if cfg.dtype == "bf16" else torch.float32
    out = {}
    for key in ("q", "k", "v"):
        out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device).to(qkv_dtype).contiguous()
    for key in ("gamma", "beta", "lam"):
        out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device, dtype=torch.float32)
    for key in ("h", "g"):
        if key in x:
            out[key] = torch.from_numpy(np.ascontiguousarray(x[key])).to(device=device, dtype=torch.float32)
    if cfg.dtype == "bf16":
        # the device values must be exactly the generator's (bf16-representable) values
        for key in ("q", "k", "v"):
            assert torch.equal(out[key].float().cpu(), torch.from_numpy(x[key]))
    return out


def slice_inputs(x: dict, idx) -> dict:
    """The (b, h) slices idx (flattened b*H + h) of a forward workload, as a B=len(idx), H=1 batch."""
    cfg = x["cfg"]
    B, H = cfg.B, cfg.H
    b = np.asarray(idx) // H
    h = np.asarray(idx) % H
    out = {}
    for key in ("q", "k", "v"):
        out[key] = x[key][b, h][:, None]
    for key in ("gamma", "beta"):
        out[key] = x[key][b, h][:, None]
    return out, h


def oracle_on_slices(x: dict, idx, steps_gpu=None, exact=False, solve_at=None):
    """Run the oracle on selected (b, h) slices; lambda follows each slice's head."""
    from oracle import mesa_forward
    sl, heads = slice_inputs(x, idx)
    cfg = x["cfg"]
    res = []
    for i, hh in enumerate(heads):
        fs = None if steps_gpu is None else steps_gpu[i][None, None]
        r = mesa_forward(sl["q"][i:i + 1], sl["k"][i:i + 1], sl["v"][i:i + 1],
                         sl["gamma"][i:i + 1], sl["beta"][i:i + 1], x["lam"][hh:hh + 1],
                         max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=fs, exact=exact,
                         solve_at=solve_at)
        res.append(r)
    return res
