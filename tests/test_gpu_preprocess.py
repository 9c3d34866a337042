"""Query/key preprocessing (causal depthwise convolution, then L2 norm) on the GPU.

Compared element by element with the fp64 oracle.  fp32 outputs agree to
fp32 rounding; bf16 outputs are the kernel's fp32 result rounded once to
nearest even, so each element lies within half a bf16 unit in the last place
of the oracle's value (2^-8 relative) plus fp32 rounding.  The history
outputs are raw copies and must match exactly.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_preprocess_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def to_dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(torch.bfloat16) if dtype == "bf16" else t.float()


def check(gpu, ref, dtype):
    gpu = gpu.float().cpu().numpy().astype(np.float64)
    if dtype == "bf16":
        assert np.all(np.abs(gpu - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    else:
        assert np.abs(gpu - ref).max() <= 2e-6


def run(x, dtype, with_hist):
    qh = to_dev(x["hq"], dtype) if with_hist else None
    kh = to_dev(x["hk"], dtype) if with_hist else None
    return mesa.qk_preprocess(to_dev(x["q"], dtype), to_dev(x["k"], dtype),
                              torch.from_numpy(x["wq"]).cuda(), torch.from_numpy(x["wk"]).cuda(),
                              q_hist=qh, k_hist=kh, return_history=True)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("d,T,W", [(128, 300, 4), (128, 77, 2), (64, 600, 3), (64, 5, 4), (16, 40, 1), (16, 2100, 4)])
@pytest.mark.parametrize("with_hist", [False, True])
def test_matches_oracle(dtype, d, T, W, with_hist):
    from oracle import qk_preprocess
    cfg = small_fwd(B=2, H=3, T=T, d=d, dtype=dtype)
    x = make_preprocess_inputs(cfg, window=W)
    r = run(x, dtype, with_hist)
    torch.cuda.synchronize()
    for key, hk in (("q", "hq"), ("k", "hk")):
        ref, href = qk_preprocess(x[key], x["w" + key], x[hk] if with_hist else None)
        check(r[key], ref, dtype)
        assert np.array_equal(r[key + "_hist"].float().cpu().numpy(), href)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_split_call_equals_one_call_and_decode_steps(dtype):
    cfg = small_fwd(B=2, H=2, T=700, d=128, dtype=dtype)
    x = make_preprocess_inputs(cfg, window=4)
    wq, wk = torch.from_numpy(x["wq"]).cuda(), torch.from_numpy(x["wk"]).cuda()
    q, k = to_dev(x["q"], dtype), to_dev(x["k"], dtype)
    whole = mesa.qk_preprocess(q, k, wq, wk)
    a = mesa.qk_preprocess(q[:, :, :333].contiguous(), k[:, :, :333].contiguous(), wq, wk, return_history=True)
    b = mesa.qk_preprocess(q[:, :, 333:].contiguous(), k[:, :, 333:].contiguous(), wq, wk,
                           q_hist=a["q_hist"], k_hist=a["k_hist"], return_history=True)
    torch.cuda.synchronize()
    for key in ("q", "k"):
        assert torch.equal(torch.cat([a[key], b[key]], dim=2), whole[key])
    # one token at a time, as a decode step would call it
    qh, kh = b["q_hist"], b["k_hist"]
    rng = np.random.default_rng(5)
    nq = to_dev(rng.standard_normal((2, 2, 3, 128), dtype=np.float32), dtype)
    nk = to_dev(rng.standard_normal((2, 2, 3, 128), dtype=np.float32), dtype)
    full = mesa.qk_preprocess(torch.cat([q, nq], 2), torch.cat([k, nk], 2), wq, wk)
    for t in range(3):
        s = mesa.qk_preprocess(nq[:, :, t:t + 1].contiguous(), nk[:, :, t:t + 1].contiguous(), wq, wk,
                               q_hist=qh, k_hist=kh, return_history=True)
        torch.cuda.synchronize()
        assert torch.equal(s["q"][:, :, 0], full["q"][:, :, 700 + t])
        assert torch.equal(s["k"][:, :, 0], full["k"][:, :, 700 + t])
        qh, kh = s["q_hist"], s["k_hist"]


def test_empty_sequence_passes_history_through():
    cfg = small_fwd(B=1, H=2, T=0, d=64, dtype="bf16")
    x = make_preprocess_inputs(cfg, window=4)
    r = run(x, "bf16", True)
    torch.cuda.synchronize()
    assert np.array_equal(r["q_hist"].float().cpu().numpy(), x["hq"])
    assert np.array_equal(r["k_hist"].float().cpu().numpy(), x["hk"])


def test_lm_workload_sampled_slices():
    """The layer workload's shape (B=8, H=16, T=4096, d=128, bf16), checked on sampled slices."""
    from oracle import qk_preprocess
    cfg = CONFIGS[3]
    x = make_preprocess_inputs(cfg, window=4)
    r = run(x, "bf16", False)
    torch.cuda.synchronize()
    rng = np.random.default_rng(11)
    for b, h in zip(rng.integers(0, cfg.B, 4), rng.integers(0, cfg.H, 4)):
        for key in ("q", "k"):
            ref, _ = qk_preprocess(x[key][b:b + 1, h:h + 1], x["w" + key][h:h + 1])
            check(r[key][b:b + 1, h:h + 1], ref, "bf16")
