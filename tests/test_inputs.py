"""The seeded input generator: determinism, rounding and distributions."""
import numpy as np
import pytest
import torch

from test_regression_sequence_amd.inputs import (
    CONFIGS, bf16_bits, bits_to_f32, make_decode_inputs, make_fwd_inputs, round_to_bf16,
    small_fwd,
)


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(100000).astype(np.float32),
                        np.array([0.0, -0.0, 1.0, 1.00390625, 1.01171875, 3.4e38, -1e-40], np.float32)])
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    assert np.array_equal(bits_to_f32(ours), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_fwd_inputs_deterministic_and_shaped():
    cfg = small_fwd(B=2, H=3, T=70, d=64, dtype="bf16")
    a = make_fwd_inputs(cfg)
    b = make_fwd_inputs(cfg)
    for key in ("q", "k", "v", "gamma", "beta", "lam", "q_bits"):
        assert np.array_equal(a[key], b[key])
    assert a["q"].shape == (2, 3, 70, 64) and a["gamma"].shape == (2, 3, 70)
    assert a["lam"].shape == (3, 64)
    assert np.array_equal(round_to_bf16(a["k"]), a["k"])
    nrm = np.linalg.norm(a["q"].astype(np.float64), axis=-1)
    assert np.all(np.abs(nrm - 1) < 1e-2)
    sig = lambda z: 1 / (1 + np.exp(-z))
    assert a["gamma"].min() >= np.float32(sig(2.0)) * (1 - 1e-6)
    assert a["gamma"].max() <= np.float32(sig(6.0)) * (1 + 1e-6)
    assert 0 <= a["beta"].min() and a["beta"].max() <= 1
    assert 0.25 <= a["lam"].min() and a["lam"].max() <= 1.0


def test_config1_is_fp32_and_seed0():
    x = make_fwd_inputs(CONFIGS[1])
    assert "q_bits" not in x
    assert x["q"].dtype == np.float32 and x["q"].shape == (1, 1, 256, 16)
    assert np.all(x["lam"] == 1.0)
    # seed 0 draws q first
    rng = np.random.default_rng(0)
    q0 = rng.standard_normal((1, 1, 256, 16))
    q0 /= np.linalg.norm(q0, axis=-1, keepdims=True)
    assert np.array_equal(x["q"], q0.astype(np.float32))


def test_decode_inputs_small():
    cfg = CONFIGS[5].replace(N=3, H=2, prefill=40)
    a = make_decode_inputs(cfg, block=4)
    b = make_decode_inputs(cfg, block=4)
    assert np.array_equal(a["h"], b["h"]) and np.array_equal(a["g"], b["g"])
    h = a["h"].reshape(-1, 128, 128)
    assert np.array_equal(h, h.transpose(0, 2, 1))
    assert np.linalg.eigvalsh(h.astype(np.float64)).min() > -1e-5
    assert a["q"].shape == (3, 2, 128) and a["gamma"].shape == (3, 2)
