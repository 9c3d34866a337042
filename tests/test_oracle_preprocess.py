"""Pins of the oracle's query/key preprocessing (causal depthwise convolution,
then L2 normalisation per token) against library routines.

The convolution is checked channel by channel against ``numpy.convolve`` over
the history followed by the sequence, the normalisation against
``sklearn.preprocessing.normalize``; neither shares code with the oracle.
"""
import numpy as np
import pytest
from sklearn.preprocessing import normalize

from oracle import qk_preprocess


def reference(x, w, hist):
    """Per channel: full linear convolution of [hist, x] with the taps, the T
    outputs aligned with x; then each token vector to unit L2 norm."""
    B, H, T, d = x.shape
    W = w.shape[-1]
    y = np.zeros((B, H, T, d))
    for b in range(B):
        for h in range(H):
            for j in range(d):
                seq = np.concatenate([hist[b, h, :, j], x[b, h, :, j]])
                y[b, h, :, j] = np.convolve(seq, w[h, j])[W - 1:W - 1 + T]
    return normalize(y.reshape(-1, d), norm="l2").reshape(B, H, T, d)


def draw(seed, B=2, H=3, T=11, d=8, W=4):
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((B, H, T, d))
    w = rng.uniform(-0.5, 0.5, (H, d, W))
    hist = rng.standard_normal((B, H, W - 1, d))
    return x, w, hist


@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_matches_library_convolution_and_normalisation(W):
    x, w, hist = draw(W, W=W)
    out, hist_out = qk_preprocess(x, w, hist)
    assert np.abs(out - reference(x, w, hist)).max() < 1e-13
    # the next call's history: the last W-1 raw vectors, oldest first
    assert np.array_equal(hist_out, np.concatenate([hist, x], axis=2)[:, :, x.shape[2]:])


def test_zero_history_is_the_default():
    x, w, hist = draw(7)
    out, _ = qk_preprocess(x, w)
    assert np.abs(out - reference(x, w, np.zeros_like(hist))).max() < 1e-13


def test_window_one_with_unit_tap_is_plain_normalisation():
    x, _, _ = draw(8, W=1)
    out, hist_out = qk_preprocess(x, np.ones((x.shape[1], x.shape[3], 1)))
    assert np.abs(out - normalize(x.reshape(-1, x.shape[-1])).reshape(x.shape)).max() < 1e-14
    assert hist_out.shape[2] == 0


def test_short_sequences_carry_history_through():
    x, w, hist = draw(9, T=2, W=4)  # fewer tokens than the window
    out, hist_out = qk_preprocess(x, w, hist)
    assert np.abs(out - reference(x, w, hist)).max() < 1e-13
    assert np.array_equal(hist_out, np.concatenate([hist[:, :, 2:], x], axis=2))


def test_unit_norm_and_positive_scale_invariance():
    x, w, hist = draw(10)
    out, _ = qk_preprocess(x, w, hist)
    assert np.abs(np.linalg.norm(out, axis=-1) - 1.0).max() < 1e-14
    out2, _ = qk_preprocess(3.5 * x, w, 3.5 * hist)
    assert np.abs(out2 - out).max() < 1e-14
