"""Calls on different streams at once (needs an MI355X).

Every entry point is asynchronous on its stream and keeps no global state
(the allocation-free forward aside), so calls on different streams that write
different buffers may run at the same time.  Here two forwards, a backward and
a decode step are launched on three side streams without synchronising in
between, with every buffer allocated beforehand; each result must be bitwise
equal to the same call run alone.
"""
import numpy as np
import pytest
import torch

from helpers import dev_inputs
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import CONFIGS, make_bwd_inputs, make_decode_inputs, make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def _fwd_buffers(a, cfg):
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    dev = a["q"].device
    out = {"o": torch.empty((B, H, T, d), device=dev), "steps": torch.empty((B, H, T), device=dev, dtype=torch.int32),
           "x": torch.empty((B, H, T, d), device=dev), "h_final": torch.empty((B, H, d, d), device=dev),
           "g_final": torch.empty((B, H, d, d), device=dev)}
    ws = torch.empty(mesa.workspace_bytes(B, H, T, d, cfg.chunk, dtype=a["q"].dtype), device=dev, dtype=torch.uint8)
    return out, ws


def test_calls_on_three_streams_match_calls_alone():
    cfg_a = small_fwd(B=2, H=4, T=700, d=128, chunk=64, dtype="bf16", max_steps=20, tol=1e-4, seed=301)
    cfg_b = small_fwd(B=1, H=8, T=333, d=64, chunk=32, dtype="bf16", max_steps=12, tol=0.0, seed=302)
    xa, xb = make_fwd_inputs(cfg_a), make_fwd_inputs(cfg_b)
    aa, ab = dev_inputs(xa), dev_inputs(xb)
    ga = {k: torch.from_numpy(v).cuda() for k, v in make_bwd_inputs(cfg_a).items()}
    dcfg = CONFIGS[5].replace(N=64, H=4, prefill=32)
    xd = make_decode_inputs(dcfg)

    def run_all(streams):
        """Launch every call on its stream (None: the current stream) and return host copies."""
        s_a, s_b, s_d = streams
        out_a, ws_a = _fwd_buffers(aa, cfg_a)
        out_b, ws_b = _fwd_buffers(ab, cfg_b)
        ad = dev_inputs(xd)
        dout = {"o": torch.empty((dcfg.N, dcfg.H, dcfg.d), device="cuda"),
                "steps": torch.empty((dcfg.N, dcfg.H), device="cuda", dtype=torch.int32)}
        torch.cuda.synchronize()
        fa = mesa.fwd_chunked(aa["q"], aa["k"], aa["v"], aa["gamma"], aa["beta"], aa["lam"], chunk=64, max_steps=20,
                              tol=1e-4, return_x=True, return_state=True, out=out_a, workspace=ws_a, stream=s_a)
        fb = mesa.fwd_chunked(ab["q"], ab["k"], ab["v"], ab["gamma"], ab["beta"], ab["lam"], chunk=32, max_steps=12,
                              tol=0.0, return_x=True, return_state=True, out=out_b, workspace=ws_b, stream=s_b)
        rd = mesa.decode_step(ad["q"], ad["k"], ad["v"], ad["gamma"], ad["beta"], ad["lam"], ad["h"], ad["g"],
                              max_steps=dcfg.max_steps, tol=dcfg.tol, out=dout, stream=s_d)
        # the backward of call A on A's stream, after A's forward
        ba = mesa.bwd_chunked(aa["q"], aa["k"], aa["v"], aa["gamma"], aa["beta"], aa["lam"], fa["x"], ga["d_o"],
                              chunk=64, max_steps=20, tol=1e-4, state_grads=True, stream=s_a)
        torch.cuda.synchronize()
        res = {f"a_{k}": v.cpu().numpy() for k, v in fa.items()}
        res.update({f"b_{k}": v.cpu().numpy() for k, v in fb.items()})
        res.update({f"d_{k}": v.cpu().numpy() for k, v in rd.items()})
        res.update({"d_h": ad["h"].cpu().numpy(), "d_g": ad["g"].cpu().numpy()})
        res.update({f"ba_{k}": v.cpu().numpy() for k, v in ba.items()})
        return res

    alone = run_all((None, None, None))
    streams = [torch.cuda.Stream() for _ in range(3)]
    for rep in range(2):
        together = run_all(streams)
        for key, val in alone.items():
            assert np.array_equal(together[key], val), (rep, key)
