"""Decode step with the packed-symmetric H state (blocked upper triangle).

The packed layout is a storage format of the same state, so the packed step
must reproduce the unpacked one: the updated states exactly (same arithmetic
per element), the outputs up to the order of the matvec sums, and the oracle
at the step counts the GPU took.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_decode_inputs

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def packed_reference(h: np.ndarray) -> np.ndarray:
    """The blocked upper-triangular layout written out directly from its definition."""
    d = h.shape[-1]
    nb = d // 16
    blocks = [h[..., 16 * bi:16 * bi + 16, 16 * bj:16 * bj + 16] for bi in range(nb) for bj in range(bi, nb)]
    return np.stack(blocks, axis=-3).reshape(*h.shape[:-2], -1)


@pytest.mark.parametrize("d", [64, 128])
def test_pack_unpack_round_trip(d):
    rng = np.random.default_rng(d)
    m = rng.standard_normal((3, 2, d, d)).astype(np.float32)
    h = (m + m.transpose(0, 1, 3, 2)).astype(np.float32)
    ht = torch.from_numpy(h).cuda()
    pk = mesa.sym_pack(ht)
    assert pk.shape == (3, 2, mesa.sym_state_floats(d))
    assert np.array_equal(pk.cpu().numpy(), packed_reference(h))
    back = mesa.sym_unpack(pk, d)
    torch.cuda.synchronize()
    assert np.array_equal(back.cpu().numpy(), h)


def oracle_outputs(x, cfg, h, g, steps):
    """The oracle's step from states h, g at the given per-pair step counts; each
    stop is checked against the oracle's residuals (the decode CG is fp32)."""
    from oracle import mesa_decode_step
    r = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], x["lam"], h, g,
                         max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=steps)
    check_stops(steps, r["res_hist"], cfg.max_steps, cfg.tol, "f32")
    return r["o"]


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("f32", 128), ("f32", 64)])
def test_packed_step_matches_full_step(dtype, d):
    cfg = CONFIGS[5].replace(N=8, H=4, d=d, prefill=200, dtype=dtype)
    x = make_decode_inputs(cfg)
    a = dev_inputs(x)
    b = dev_inputs(x)
    hs = mesa.sym_pack(b["h"])
    for step in range(3):  # a few steps in a row: the packed state carries over
        h_in, g_in = a["h"].cpu().numpy(), a["g"].cpu().numpy()
        ra = mesa.decode_step(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], a["h"], a["g"],
                              max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
        rb = mesa.decode_step_symh(b["q"], b["k"], b["v"], b["gamma"], b["beta"], b["lam"], hs, b["g"],
                                   max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
        torch.cuda.synchronize()
        # the state updates are the same arithmetic per element
        assert torch.equal(mesa.sym_unpack(hs, d), a["h"]), "packed H differs from the full update"
        assert torch.equal(b["g"], a["g"])
        # outputs: both within the fp32 bar of the oracle at their own step counts,
        # and of each other (the matvec sums run in another order; a step count
        # may differ by one where the residual sits at the tolerance)
        na, nb = ra["steps"].cpu().numpy(), rb["steps"].cpu().numpy()
        oa, ob = ra["o"].cpu().numpy(), rb["o"].cpu().numpy()
        assert rel_l2(oa, oracle_outputs(x, cfg, h_in, g_in, na)) <= 1e-4
        assert rel_l2(ob, oracle_outputs(x, cfg, h_in, g_in, nb)) <= 1e-4
        assert rel_l2(ob, oa) <= 1e-4
        assert np.mean(na != nb) < 0.1


def test_packed_step_config5_against_oracle():
    cfg = CONFIGS[5]
    x = make_decode_inputs(cfg)
    d = dev_inputs(x)
    hs = mesa.sym_pack(d["h"])
    del d["h"]
    res = mesa.decode_step_symh(d["q"], d["k"], d["v"], d["gamma"], d["beta"], d["lam"], hs, d["g"],
                                max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    o = res["o"].cpu().numpy().reshape(-1, cfg.d)
    n = res["steps"].cpu().numpy().reshape(-1)
    from oracle import mesa_decode_step
    pick = np.random.default_rng(55).choice(cfg.N * cfg.H, 48, replace=False)
    flat = lambda a: a.reshape(cfg.N * cfg.H, *a.shape[2:])
    heads = pick % cfg.H
    ref, hist = [], []
    for i, p in enumerate(pick):
        hh = heads[i]
        r = mesa_decode_step(flat(x["q"])[p][None, None], flat(x["k"])[p][None, None],
                             flat(x["v"])[p][None, None], flat(x["gamma"])[p][None, None],
                             flat(x["beta"])[p][None, None], x["lam"][hh:hh + 1],
                             flat(x["h"])[p][None, None], flat(x["g"])[p][None, None],
                             max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=n[p].reshape(1, 1))
        ref.append(r["o"][0, 0])
        hist.append(r["res_hist"][0, 0])
    assert rel_l2(o[pick], np.stack(ref)) <= 1e-4
    check_stops(n[pick], np.stack(hist), cfg.max_steps, cfg.tol, "f32")
    h_after = mesa.sym_unpack(hs, cfg.d).cpu().numpy().reshape(-1, cfg.d, cfg.d)
    assert np.array_equal(h_after, h_after.transpose(0, 2, 1))
