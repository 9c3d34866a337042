"""The allocation-free forward (mesa_fwd_chunked_noalloc) against mesa_fwd_chunked.

For callers that cannot allocate device memory.  Both calls run the same
kernels on the same inputs, so every output must be bit-identical; two calls
in a row, the second smaller, show that the shared static scratch carries
nothing from one call into the next.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs, oracle_on_slices, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def both(x, cfg):
    d = dev_inputs(x)
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_state=True, return_steps=True,
              return_x=True)
    ref = mesa.fwd_chunked(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], **kw)
    # outputs preallocated: the call under test allocates nothing, here or in the library
    out = {key: torch.full_like(t, float("nan")) if t.is_floating_point() else torch.full_like(t, -1)
           for key, t in ref.items()}
    torch.cuda.synchronize()
    res = mesa.fwd_chunked_noalloc(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], out=out, **kw)
    torch.cuda.synchronize()
    for key in ref:
        assert res[key] is out[key]
        assert torch.equal(res[key], ref[key]), key
    return {k: v.cpu().numpy() for k, v in res.items()}


def test_noalloc_matches_the_workspace_forward_on_two_calls_in_a_row():
    # first call: the mid-size workload with dynamic CG (16 MiB of scratch)
    c1 = CONFIGS[2].replace(max_steps=20, tol=1e-4)
    x1 = make_fwd_inputs(c1)
    r1 = both(x1, c1)
    assert mesa.workspace_bytes(c1.B, c1.H, c1.T, c1.d, c1.chunk) > 8 << 20
    # second call, smaller: d = 128, a ragged last chunk, a chunk with decay past e^-40
    c2 = small_fwd(B=1, H=2, T=150, d=128, chunk=64, dtype="bf16", max_steps=10)
    x2 = make_fwd_inputs(c2)
    g = x2["gamma"].copy()
    g[:, 1, 64:128] = np.float32(0.3)
    x2 = dict(x2, gamma=g)
    r2 = both(x2, c2)
    # and both against the oracle at the GPU's step counts
    for x, r, cfg, idx in ((x1, r1, c1, [0, 17]), (x2, r2, c2, [0, 1])):
        steps = r["steps"].reshape(cfg.B * cfg.H, cfg.T)[idx]
        refs = oracle_on_slices(x, idx, steps_gpu=steps)
        o = r["o"].reshape(cfg.B * cfg.H, cfg.T, cfg.d)[idx]
        assert rel_l2(o, np.stack([rr["o_cg"][0, 0] for rr in refs])) <= 2e-2


def test_noalloc_rejects_a_workload_beyond_its_scratch():
    cfg = CONFIGS[3].replace(B=1, H=16, T=8192)  # 2048 chunks x 64 KB of snapshots: 128 MiB
    assert mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk) > mesa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros((cfg.B, cfg.H, cfg.T, cfg.d), device="cuda", dtype=torch.bfloat16)
    ga = torch.zeros((cfg.B, cfg.H, cfg.T), device="cuda")
    lam = torch.ones((cfg.H, cfg.d), device="cuda")
    with pytest.raises(mesa.MesaError) as e:
        mesa.fwd_chunked_noalloc(q, q, q, ga, ga, lam, chunk=cfg.chunk, max_steps=2)
    assert e.value.status == 2
