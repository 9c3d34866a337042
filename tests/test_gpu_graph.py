"""The forward, the decode step and the backward inside a HIP graph: the calls that allocate nothing when given
their buffers -- mesa_fwd_chunked with a workspace and preallocated outputs,
and mesa_fwd_chunked_noalloc (its scratch is the library's own) -- are
captured once and replayed several times.  Between replays the program runs
eager work of its own (another forward on other inputs, and new contents in
the captured input buffers); every replay must equal an eager call on the same
inputs bit for bit.  Needs an MI355X.
"""
import pytest
import torch

from helpers import dev_inputs
from test_regression_sequence_amd import mesa
from test_regression_sequence_amd.inputs import make_fwd_inputs, small_fwd

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    mesa.lib()


def alloc_out(cfg):
    B, H, T, d = cfg.B, cfg.H, cfg.T, cfg.d
    return {"o": torch.empty((B, H, T, d), device="cuda"),
            "steps": torch.empty((B, H, T), device="cuda", dtype=torch.int32),
            "x": torch.empty((B, H, T, d), device="cuda")}


@pytest.mark.parametrize("form", ["workspace", "noalloc"])
@pytest.mark.parametrize("tol", [0.0, 1e-4])
def test_forward_replays_in_a_graph(form, tol):
    cfg = small_fwd(B=2, H=4, T=300, d=128, chunk=64, dtype="bf16", max_steps=12 if tol == 0 else 32, tol=tol)
    a = dev_inputs(make_fwd_inputs(cfg))
    b = dev_inputs(make_fwd_inputs(cfg.replace(seed=cfg.seed + 1)))
    need = mesa.workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, dtype=torch.bfloat16)
    ws = torch.empty(need, device="cuda", dtype=torch.uint8)
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)

    def call(inp, out, stream=None):
        args = (inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], inp["lam"])
        if form == "noalloc":
            return mesa.fwd_chunked_noalloc(*args, out=out, stream=stream, **kw)
        return mesa.fwd_chunked(*args, out=out, workspace=ws, stream=stream, **kw)

    # the captured input buffers, first holding a's values
    cap = {k: v.clone() for k, v in a.items()}
    out_g = alloc_out(cfg)
    call(cap, out_g)  # eager warm-up (first use initialises the library's scratch)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        call(cap, out_g, stream=s)
    torch.cuda.synchronize()

    def eager(inp):
        out = alloc_out(cfg)
        call(inp, out)
        torch.cuda.synchronize()
        return out

    ref_a, ref_b = eager(a), eager(b)
    for rep, (src, ref) in enumerate([(a, ref_a), (a, ref_a), (b, ref_b), (a, ref_a), (b, ref_b)]):
        for k in cap:
            cap[k].copy_(src[k])
        for key in out_g:
            out_g[key].fill_(float("nan") if out_g[key].is_floating_point() else -1)
        other = eager(b if src is a else a)  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        for key in out_g:
            assert torch.equal(out_g[key], ref[key]), (form, tol, rep, key)
        assert torch.equal(other["o"], (ref_b if src is a else ref_a)["o"])


def test_decode_step_replays_in_a_graph():
    """The decode step updates its states in place: each replay starts from
    states copied into the captured buffers and must equal an eager step."""
    from test_regression_sequence_amd.inputs import CONFIGS, make_decode_inputs
    cfg = CONFIGS[5].replace(N=16)
    srcs = [dev_inputs(make_decode_inputs(cfg.replace(seed=cfg.seed + i))) for i in range(2)]
    cap = {k: v.clone() for k, v in srcs[0].items()}
    kw = dict(max_steps=cfg.max_steps, tol=cfg.tol, return_x=True)
    N, H, d = cfg.N, cfg.H, cfg.d
    out_g = {"o": torch.empty((N, H, d), device="cuda"), "steps": torch.empty((N, H), device="cuda", dtype=torch.int32),
             "x": torch.empty((N, H, d), device="cuda")}

    def step(inp, out, stream=None):
        return mesa.decode_step(inp["q"], inp["k"], inp["v"], inp["gamma"], inp["beta"], inp["lam"], inp["h"],
                                inp["g"], out=out, stream=stream, **kw)

    def eager(src):
        inp = {k: v.clone() for k, v in src.items()}
        out = step(inp, None)
        torch.cuda.synchronize()
        return out, inp["h"], inp["g"]

    step({k: v.clone() for k, v in cap.items()}, None)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        step(cap, out_g, stream=s)
    torch.cuda.synchronize()
    refs = [eager(src) for src in srcs]
    for rep, i in enumerate([0, 1, 1, 0]):
        for k in cap:
            cap[k].copy_(srcs[i][k])
        eager(srcs[1 - i])  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        out, h1, g1 = refs[i]
        for key in out_g:
            assert torch.equal(out_g[key], out[key]), (rep, key)
        assert torch.equal(cap["h"], h1) and torch.equal(cap["g"], g1), rep


def test_backward_replays_in_a_graph():
    """mesa_bwd_chunked with its workspace and preallocated gradients, captured
    once and replayed: every replay equals an eager call."""
    from test_regression_sequence_amd.inputs import make_bwd_inputs
    cfg = small_fwd(B=2, H=4, T=200, d=128, chunk=64, dtype="bf16", max_steps=10, tol=0.0)
    a = dev_inputs(make_fwd_inputs(cfg))
    d_o = torch.from_numpy(make_bwd_inputs(cfg)["d_o"]).cuda()
    kw = dict(chunk=cfg.chunk, max_steps=cfg.max_steps, tol=cfg.tol)
    f = mesa.fwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], return_x=True, **kw)
    ws = torch.empty(mesa.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d, cfg.chunk, cfg.max_steps, cfg.tol),
                     device="cuda", dtype=torch.uint8)

    def bwd(dout, out=None, stream=None):
        return mesa.bwd_chunked(a["q"], a["k"], a["v"], a["gamma"], a["beta"], a["lam"], f["x"], dout, out=out,
                                workspace=ws, stream=stream, **kw)

    out_g = bwd(d_o)  # eager call; its result tensors become the captured outputs
    torch.cuda.synchronize()
    cap = d_o.clone()
    graph = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.graph(graph, stream=s):
        bwd(cap, out=out_g, stream=s)
    torch.cuda.synchronize()
    d_o2 = torch.flip(d_o, dims=[2]).contiguous()
    refs = {}
    for name, src in (("a", d_o), ("b", d_o2)):
        r = bwd(src)
        torch.cuda.synchronize()
        refs[name] = {k: v.clone() for k, v in r.items()}
    for rep, name in enumerate(["a", "b", "a"]):
        cap.copy_(d_o if name == "a" else d_o2)
        for key in out_g:
            out_g[key].fill_(float("nan"))
        bwd(d_o2 if name == "a" else d_o)  # eager work between the replays
        graph.replay()
        torch.cuda.synchronize()
        for key in out_g:
            assert torch.equal(out_g[key], refs[name][key]), (rep, key)
