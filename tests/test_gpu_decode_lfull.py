"""Decode step with a full symmetric positive definite Lambda per head.

The pages' objective regularises with a symmetric positive definite Lambda;
the oracle's decode step takes it as a full matrix.  Checked against the
oracle at the GPU's step counts for both H layouts, cold and warm starts,
bf16 and fp32 inputs, d = 64 and 128; and a diagonal Lambda given as a full
matrix must reproduce the diagonal path.  Needs an MI355X.
"""
import numpy as np
import pytest
import torch

from helpers import check_stops, dev_inputs, rel_l2
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_decode_inputs, make_full_lambda

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


@pytest.mark.parametrize("dtype,d,packed,warm", [("bf16", 128, False, False), ("bf16", 128, True, False),
                                                 ("f32", 64, False, True), ("bf16", 64, True, True)])
def test_full_lambda_matches_oracle(dtype, d, packed, warm):
    from oracle import mesa_decode_step
    cfg = CONFIGS[5].replace(N=8, H=4, d=d, prefill=200, dtype=dtype)
    x = make_decode_inputs(cfg)
    lam = make_full_lambda(cfg.H, d, cfg.seed)
    a = dev_inputs(x)
    h = mesa.sym_pack(a["h"]) if packed else a["h"]
    x0 = np.random.default_rng(9).standard_normal((cfg.N, cfg.H, d)).astype(np.float32) * 0.3 if warm else None
    xs = torch.from_numpy(x0).cuda() if warm else None
    r = mesa.decode_step_ex(a["q"], a["k"], a["v"], a["gamma"], a["beta"], torch.from_numpy(lam).cuda(), h, a["g"],
                            x_state=xs, packed_h=packed, max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    steps = r["steps"].cpu().numpy()
    assert steps.max() > 0
    ref = mesa_decode_step(x["q"], x["k"], x["v"], x["gamma"], x["beta"], lam, x["h"], x["g"],
                           max_steps=cfg.max_steps, tol=cfg.tol, forced_steps=steps, x0=x0)
    assert rel_l2(r["o"].cpu().numpy(), ref["o"]) <= 1e-4
    check_stops(steps, ref["res_hist"], cfg.max_steps, cfg.tol, "f32")
    if warm:
        assert rel_l2(xs.cpu().numpy(), ref["x"]) <= 1e-4
    # the stored state is H alone (Lambda is added only for the solve)
    hf = mesa.sym_unpack(h, d) if packed else h
    assert rel_l2(hf.cpu().numpy(), ref["h"]) <= 1e-6


def test_diagonal_as_full_matrix_matches_diagonal_path():
    cfg = CONFIGS[5].replace(N=8, H=4, d=128, prefill=200)
    x = make_decode_inputs(cfg)
    a, b = dev_inputs(x), dev_inputs(x)
    lam_full = torch.diag_embed(a["lam"]).contiguous()
    r1 = mesa.decode_step(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], a["h"], a["g"],
                          max_steps=cfg.max_steps, tol=cfg.tol)
    r2 = mesa.decode_step_ex(b["q"], b["k"], b["v"], b["gamma"], b["beta"], lam_full, b["h"], b["g"],
                             max_steps=cfg.max_steps, tol=cfg.tol)
    torch.cuda.synchronize()
    assert torch.equal(a["h"], b["h"]) and torch.equal(a["g"], b["g"])
    n1, n2 = r1["steps"].cpu().numpy(), r2["steps"].cpu().numpy()
    assert np.mean(n1 != n2) < 0.1
    same = n1 == n2
    o1, o2 = r1["o"].cpu().numpy(), r2["o"].cpu().numpy()
    assert rel_l2(o2[same], o1[same]) <= 1e-5
