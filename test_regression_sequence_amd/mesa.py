"""Python binding of libmesa (ctypes).  Argument marshalling only.

Every step of the layer runs in the HIP library; this module passes device
pointers of torch tensors and the current HIP stream through the C ABI
declared in ``include/mesa.h``, and allocates outputs with torch.  There is no
fallback: if the library is missing, every call raises ``MesaError``.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

__all__ = [
    "MesaError", "lib", "library_path", "FwdDesc", "MESA_F32", "MESA_BF16",
    "workspace_bytes", "fwd_chunked", "fwd_chunked_noalloc", "fwd_chunked_prep", "fwd_scan", "fwd_solve", "decode_step", "abi_version",
    "status_string", "sym_state_floats", "sym_pack", "sym_unpack", "decode_step_symh",
]

MESA_F32 = 0
MESA_BF16 = 1
STATUS = {0: "MESA_OK", 1: "MESA_ERR_INVALID_ARG", 2: "MESA_ERR_UNSUPPORTED",
          3: "MESA_ERR_ALIGNMENT", 4: "MESA_ERR_WORKSPACE", 5: "MESA_ERR_HIP"}

_LIB: Optional[ctypes.CDLL] = None


class MesaError(RuntimeError):
    def __init__(self, msg, status: int | None = None):
        super().__init__(msg)
        self.status = status


class FwdDesc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("T", ctypes.c_int32),
                ("dk", ctypes.c_int32), ("dv", ctypes.c_int32), ("chunk", ctypes.c_int32),
                ("max_steps", ctypes.c_int32), ("tol", ctypes.c_float), ("in_dtype", ctypes.c_int)]


def library_path() -> str:
    return os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmesa.so")


def lib() -> ctypes.CDLL:
    global _LIB
    if _LIB is None:
        path = library_path()
        if not os.path.exists(path):
            raise MesaError(f"{path} is not built; run `python -m test_regression_sequence_amd.build`")
        L = ctypes.CDLL(path)
        P, S, I32, F = ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int32, ctypes.c_float
        L.mesa_abi_version.restype = I32
        L.mesa_abi_version.argtypes = []
        L.mesa_status_string.restype = ctypes.c_char_p
        L.mesa_status_string.argtypes = [ctypes.c_int]
        L.mesa_fwd_workspace_bytes.restype = S
        L.mesa_fwd_workspace_bytes.argtypes = [ctypes.POINTER(FwdDesc)]
        L.mesa_fwd_chunked.restype = ctypes.c_int
        L.mesa_fwd_chunked.argtypes = [ctypes.POINTER(FwdDesc), P, P, P, P, P, P, P, P, P, P, P, P, P,
                                       P, S, P]
        L.mesa_fwd_chunked_warm.restype = ctypes.c_int
        L.mesa_fwd_chunked_warm.argtypes = list(L.mesa_fwd_chunked.argtypes)
        L.mesa_fwd_chunked_noalloc.restype = ctypes.c_int
        L.mesa_fwd_chunked_noalloc.argtypes = [ctypes.POINTER(FwdDesc)] + [P] * 13 + [P]
        L.mesa_fwd_chunked_prep.restype = ctypes.c_int
        L.mesa_fwd_chunked_prep.argtypes = [ctypes.POINTER(FwdDesc), P, P, P, P, P, I32, F] + [P] * 15 + [S, P]
        L.mesa_fwd_chunked_ex.restype = ctypes.c_int
        L.mesa_fwd_chunked_ex.argtypes = [ctypes.POINTER(FwdDesc), P, P, P, P, P, P, I32, P, P, P, P, P, P,
                                          P, P, S, P]
        L.mesa_fwd_scan.restype = ctypes.c_int
        L.mesa_fwd_scan.argtypes = [ctypes.POINTER(FwdDesc), P, P, P, P, P, P, P, P, P, S, P]
        L.mesa_fwd_solve.restype = ctypes.c_int
        L.mesa_fwd_solve.argtypes = [ctypes.POINTER(FwdDesc), P, P, P, P, P, P, P, P, P, P, S, P]
        L.mesa_decode_step.restype = ctypes.c_int
        L.mesa_decode_step.argtypes = [I32, I32, I32, I32, P, P, P, ctypes.c_int, P, P, P, P, P, P,
                                       P, P, I32, F, P]
        L.mesa_decode_step_symh.restype = ctypes.c_int
        L.mesa_decode_step_symh.argtypes = list(L.mesa_decode_step.argtypes)
        L.mesa_decode_step_warm.restype = ctypes.c_int
        L.mesa_decode_step_warm.argtypes = [I32, I32, I32, I32, P, P, P, ctypes.c_int, P, P, P, P, I32,
                                            P, P, P, P, I32, F, P]
        L.mesa_decode_step_ex.restype = ctypes.c_int
        L.mesa_decode_step_ex.argtypes = [I32, I32, I32, I32, P, P, P, ctypes.c_int, P, P, P, I32, P, I32,
                                          P, P, P, P, P, I32, F, P]
        L.mesa_bwd_workspace_bytes.restype = S
        L.mesa_bwd_workspace_bytes.argtypes = [ctypes.POINTER(FwdDesc)]
        L.mesa_bwd_chunked.restype = ctypes.c_int
        L.mesa_bwd_chunked.argtypes = [ctypes.POINTER(FwdDesc)] + [P] * 21 + [I32, P, S, P]
        L.mesa_bwd_chunked_ex.restype = ctypes.c_int
        L.mesa_bwd_chunked_ex.argtypes = [ctypes.POINTER(FwdDesc)] + [P] * 6 + [I32] + [P] * 15 + [I32, P, S, P]
        L.mesa_qk_preprocess.restype = ctypes.c_int
        L.mesa_qk_preprocess.argtypes = [I32, I32, I32, I32, I32, ctypes.c_int, P, P, P, P, P, P, F,
                                         P, P, P, P, P]
        L.mesa_sym_state_floats.restype = S
        L.mesa_sym_state_floats.argtypes = [I32]
        L.mesa_sym_pack.restype = ctypes.c_int
        L.mesa_sym_pack.argtypes = [I32, I32, P, P, P]
        L.mesa_sym_unpack.restype = ctypes.c_int
        L.mesa_sym_unpack.argtypes = [I32, I32, P, P, P]
        _LIB = L
    return _LIB


def abi_version() -> int:
    return int(lib().mesa_abi_version())


def status_string(code: int) -> str:
    return lib().mesa_status_string(int(code)).decode()


def _check(code: int, what: str):
    if code != 0:
        raise MesaError(f"{what}: {STATUS.get(code, code)} ({status_string(code)})", code)


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return MESA_F32
    if t.dtype == torch.bfloat16:
        return MESA_BF16
    raise MesaError(f"q/k/v must be float32 or bfloat16, got {t.dtype}")


def _need(t: torch.Tensor, name: str, shape, dtype=None):
    if not t.is_cuda:
        raise MesaError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise MesaError(f"{name} must be contiguous")
    if tuple(t.shape) != tuple(shape):
        raise MesaError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if dtype is not None and t.dtype != dtype:
        raise MesaError(f"{name} must be {dtype}, got {t.dtype}")


def make_desc(B, H, T, d, chunk, max_steps, tol, dtype_code) -> FwdDesc:
    return FwdDesc(B, H, T, d, d, chunk, max_steps, float(tol), dtype_code)


def workspace_bytes(B, H, T, d, chunk, max_steps=0, tol=0.0, dtype=torch.bfloat16) -> int:
    code = MESA_BF16 if dtype == torch.bfloat16 else MESA_F32
    desc = make_desc(B, H, T, d, chunk, max_steps, tol, code)
    return int(lib().mesa_fwd_workspace_bytes(ctypes.byref(desc)))


def fwd_chunked(q, k, v, gamma, beta, lam, *, chunk: int = 64, max_steps: int = 30,
                tol: float = 0.0, h0=None, g0=None, return_state: bool = False,
                return_steps: bool = True, return_x: bool = False, out=None,
                workspace: Optional[torch.Tensor] = None, stream=None, warm: bool = False) -> dict:
    """Chunked Mesa forward; q, k, v [B, H, T, d] (fp32 or bf16) on the GPU.

    gamma, beta [B, H, T] fp32; lam [H, d] fp32; h0, g0 optional [B, H, d, d]
    fp32.  Returns a dict with ``o`` [B, H, T, d] fp32 and, on request,
    ``steps`` [B, H, T] int32, ``x`` [B, H, T, d], ``h_final``, ``g_final``.
    ``out`` may pass preallocated result tensors (same keys).  ``warm`` calls
    ``mesa_fwd_chunked_warm``: token t's CG starts from token t-16's solution
    when both lie in one chunk (bf16 inputs).
    """
    return _fwd("warm" if warm else False, q, k, v, gamma, beta, lam, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, return_state=return_state, return_steps=return_steps, return_x=return_x,
                out=out, workspace=workspace, stream=stream)


NOALLOC_SCRATCH_BYTES = 64 << 20  # MESA_NOALLOC_SCRATCH_BYTES


def fwd_chunked_noalloc(q, k, v, gamma, beta, lam, *, chunk: int = 64, max_steps: int = 30,
                        tol: float = 0.0, h0=None, g0=None, return_state: bool = False,
                        return_steps: bool = True, return_x: bool = False, out=None,
                        stream=None) -> dict:
    """``fwd_chunked`` through ``mesa_fwd_chunked_noalloc``: the library uses its
    static per-GPU scratch (at most ``NOALLOC_SCRATCH_BYTES`` of workspace) and
    allocates nothing; pass ``out`` to allocate nothing here either."""
    return _fwd("noalloc", q, k, v, gamma, beta, lam, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, return_state=return_state, return_steps=return_steps, return_x=return_x,
                out=out, workspace=None, stream=stream)


def fwd_chunked_prep(q_raw, k_raw, v, gamma, beta, lam, w_q, w_k, *, q_hist=None, k_hist=None,
                     eps: float = 1e-6, chunk: int = 64, max_steps: int = 30, tol: float = 0.0,
                     h0=None, g0=None, return_state: bool = False, return_steps: bool = True,
                     return_x: bool = False, return_history: bool = False, out=None,
                     workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """``fwd_chunked`` on raw bf16 q, k [B, H, T, d] with ``qk_preprocess`` fused
    into the forward (``mesa_fwd_chunked_prep``): taps w_q, w_k [H, d, W], raw
    histories q_hist, k_hist [B, H, W-1, d] (None: zeros).  The result equals
    ``qk_preprocess`` followed by ``fwd_chunked`` bit for bit; with
    return_history it also holds the next call's histories ``q_hist``,
    ``k_hist``.  bf16 inputs, chunk 64, d in {64, 128}, W in 1..4."""
    B, H, T, d = q_raw.shape
    W = w_q.shape[-1]
    _need(w_q, "w_q", (H, d, W), torch.float32)
    _need(w_k, "w_k", (H, d, W), torch.float32)
    for name, t in (("q_hist", q_hist), ("k_hist", k_hist)):
        if t is not None:
            _need(t, name, (B, H, W - 1, d), q_raw.dtype)
    prep = {"w_q": w_q, "w_k": w_k, "W": W, "eps": eps, "q_hist": q_hist, "k_hist": k_hist,
            "return_history": return_history}
    return _fwd("prep", q_raw, k_raw, v, gamma, beta, lam, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, return_state=return_state, return_steps=return_steps, return_x=return_x,
                out=out, workspace=workspace, stream=stream, prep=prep)


def fwd_chunked_ex(q, k, v, gamma, beta, lam, *, chunk: int = 64, max_steps: int = 30,
                   tol: float = 0.0, h0=None, g0=None, return_state: bool = False,
                   return_steps: bool = True, return_x: bool = False, out=None,
                   workspace: Optional[torch.Tensor] = None, stream=None) -> dict:
    """``fwd_chunked`` with ``lam`` either the diagonal [H, d] or a full
    symmetric positive definite matrix per head [H, d, d] (fp32, row-major);
    the full form needs bf16 inputs, chunk 64 and d in {64, 128}."""
    return _fwd(True, q, k, v, gamma, beta, lam, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, return_state=return_state, return_steps=return_steps, return_x=return_x,
                out=out, workspace=workspace, stream=stream)


def _fwd(ex: bool, q, k, v, gamma, beta, lam, *, chunk, max_steps, tol, h0, g0, return_state,
         return_steps, return_x, out, workspace, stream, prep=None) -> dict:
    B, H, T, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (B, H, T, d), q.dtype)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(beta, "beta", (B, H, T), torch.float32)
    noalloc = ex == "noalloc"
    lam_full = ex is True and lam.dim() == 3
    _need(lam, "lam", (H, d, d) if lam_full else (H, d), torch.float32)
    for name, t in (("h0", h0), ("g0", g0)):
        if t is not None:
            _need(t, name, (B, H, d, d), torch.float32)
    desc = make_desc(B, H, T, d, chunk, max_steps, tol, code)
    L = lib()
    need = int(L.mesa_fwd_workspace_bytes(ctypes.byref(desc)))
    dev = q.device
    out = dict(out or {})
    res = {}
    res["o"] = out.get("o") if out.get("o") is not None else torch.empty((B, H, T, d), device=dev, dtype=torch.float32)
    if return_steps:
        res["steps"] = out.get("steps") if out.get("steps") is not None else torch.empty((B, H, T), device=dev, dtype=torch.int32)
    if return_x:
        res["x"] = out.get("x") if out.get("x") is not None else torch.empty((B, H, T, d), device=dev, dtype=torch.float32)
    if return_state:
        res["h_final"] = out.get("h_final") if out.get("h_final") is not None else torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
        res["g_final"] = out.get("g_final") if out.get("g_final") is not None else torch.empty((B, H, d, d), device=dev, dtype=torch.float32)
    if prep is not None and prep["return_history"]:
        for key in ("q_hist", "k_hist"):
            res[key] = out.get(key) if out.get(key) is not None else torch.empty((B, H, prep["W"] - 1, d), device=dev, dtype=q.dtype)
    if noalloc:
        code_ = L.mesa_fwd_chunked_noalloc(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta),
                                           _ptr(lam), _ptr(h0), _ptr(g0), _ptr(res["o"]), _ptr(res.get("h_final")),
                                           _ptr(res.get("g_final")), _ptr(res.get("steps")), _ptr(res.get("x")),
                                           _stream(stream))
        _check(code_, "mesa_fwd_chunked_noalloc")
        return res
    if workspace is None and need > 0:
        workspace = torch.empty(need, device=dev, dtype=torch.uint8)
    wbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    rest = (_ptr(h0), _ptr(g0), _ptr(res["o"]), _ptr(res.get("h_final")), _ptr(res.get("g_final")),
            _ptr(res.get("steps")), _ptr(res.get("x")), _ptr(workspace), ctypes.c_size_t(wbytes),
            _stream(stream))
    head = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(lam))
    if ex == "prep":
        code_ = L.mesa_fwd_chunked_prep(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(prep["w_q"]),
                                        _ptr(prep["w_k"]), int(prep["W"]), float(prep["eps"]), _ptr(prep["q_hist"]),
                                        _ptr(prep["k_hist"]), _ptr(gamma), _ptr(beta), _ptr(lam), *rest[:7],
                                        _ptr(res.get("q_hist")), _ptr(res.get("k_hist")), *rest[7:])
        _check(code_, "mesa_fwd_chunked_prep")
    elif ex == "warm":
        code_ = L.mesa_fwd_chunked_warm(*head, *rest)
        _check(code_, "mesa_fwd_chunked_warm")
    elif ex:
        code_ = L.mesa_fwd_chunked_ex(*head, 1 if lam_full else 0, *rest)
        _check(code_, "mesa_fwd_chunked_ex")
    else:
        code_ = L.mesa_fwd_chunked(*head, *rest)
        _check(code_, "mesa_fwd_chunked")
    return res


def fwd_scan(k, v, gamma, beta, *, chunk: int, workspace: torch.Tensor, h0=None, g0=None,
             h_final=None, g_final=None, stream=None):
    """State scan only: boundary states into ``workspace``, optional final states."""
    B, H, T, d = k.shape
    desc = make_desc(B, H, T, d, chunk, 0, 0.0, _dtype_code(k))
    wbytes = workspace.numel() * workspace.element_size()
    code_ = lib().mesa_fwd_scan(ctypes.byref(desc), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta),
                                _ptr(h0), _ptr(g0), _ptr(h_final), _ptr(g_final), _ptr(workspace),
                                ctypes.c_size_t(wbytes), _stream(stream))
    _check(code_, "mesa_fwd_scan")


def fwd_solve(q, k, v, gamma, beta, lam, *, chunk: int, max_steps: int, tol: float,
              workspace: torch.Tensor, o: torch.Tensor, steps=None, x=None, stream=None):
    """CG solve + read-out only, from the boundary states a preceding fwd_scan left in ``workspace``."""
    B, H, T, d = q.shape
    desc = make_desc(B, H, T, d, chunk, max_steps, tol, _dtype_code(q))
    wbytes = workspace.numel() * workspace.element_size()
    code_ = lib().mesa_fwd_solve(ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta),
                                 _ptr(lam), _ptr(o), _ptr(steps), _ptr(x), _ptr(workspace),
                                 ctypes.c_size_t(wbytes), _stream(stream))
    _check(code_, "mesa_fwd_solve")


def sym_state_floats(d: int) -> int:
    """Floats of one H state in the blocked upper-triangular layout (d in {64, 128})."""
    n = int(lib().mesa_sym_state_floats(int(d)))
    if n == 0:
        raise MesaError(f"no packed layout for d={d}", 2)
    return n


def sym_pack(full: torch.Tensor, stream=None) -> torch.Tensor:
    """[..., d, d] fp32 symmetric states -> [..., sym_state_floats(d)] blocked upper triangle."""
    d = full.shape[-1]
    lead = full.shape[:-2]
    count = int(full.numel() // (d * d))
    _need(full, "full", tuple(lead) + (d, d), torch.float32)
    out = torch.empty(tuple(lead) + (sym_state_floats(d),), device=full.device, dtype=torch.float32)
    _check(lib().mesa_sym_pack(count, d, _ptr(full), _ptr(out), _stream(stream)), "mesa_sym_pack")
    return out


def sym_unpack(packed: torch.Tensor, d: int, stream=None) -> torch.Tensor:
    """[..., sym_state_floats(d)] -> [..., d, d] fp32 (lower blocks mirrored)."""
    n = sym_state_floats(d)
    lead = packed.shape[:-1]
    _need(packed, "packed", tuple(lead) + (n,), torch.float32)
    count = int(packed.numel() // n)
    out = torch.empty(tuple(lead) + (d, d), device=packed.device, dtype=torch.float32)
    _check(lib().mesa_sym_unpack(count, d, _ptr(packed), _ptr(out), _stream(stream)), "mesa_sym_unpack")
    return out


def decode_step_symh(q, k, v, gamma, beta, lam, h_sym, g_state, *, max_steps: int = 32,
                     tol: float = 1e-4, return_steps: bool = True, return_x: bool = False,
                     out=None, stream=None) -> dict:
    """decode_step with h_sym [N, H, sym_state_floats(d)] in the blocked layout (updated in place)."""
    return decode_step(q, k, v, gamma, beta, lam, h_sym, g_state, max_steps=max_steps, tol=tol,
                       return_steps=return_steps, return_x=return_x, out=out, stream=stream,
                       _symh=True)


def decode_step(q, k, v, gamma, beta, lam, h_state, g_state, *, max_steps: int = 32,
                tol: float = 1e-4, return_steps: bool = True, return_x: bool = False,
                out=None, stream=None, _symh: bool = False) -> dict:
    """One recurrent step; q, k, v [N, H, d]; h_state, g_state [N, H, d, d] fp32, updated in place."""
    N, H, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, H, d), q.dtype)
    _need(gamma, "gamma", (N, H), torch.float32)
    _need(beta, "beta", (N, H), torch.float32)
    _need(lam, "lam", (H, d), torch.float32)
    if _symh:
        _need(h_state, "h_sym", (N, H, sym_state_floats(d)), torch.float32)
    else:
        _need(h_state, "h_state", (N, H, d, d), torch.float32)
    _need(g_state, "g_state", (N, H, d, d), torch.float32)
    dev = q.device
    out = dict(out or {})
    res = {"o": out.get("o") if out.get("o") is not None else torch.empty((N, H, d), device=dev, dtype=torch.float32)}
    if return_steps:
        res["steps"] = out.get("steps") if out.get("steps") is not None else torch.empty((N, H), device=dev, dtype=torch.int32)
    if return_x:
        res["x"] = out.get("x") if out.get("x") is not None else torch.empty((N, H, d), device=dev, dtype=torch.float32)
    fn = lib().mesa_decode_step_symh if _symh else lib().mesa_decode_step
    code_ = fn(N, H, d, d, _ptr(q), _ptr(k), _ptr(v), code, _ptr(gamma), _ptr(beta),
               _ptr(lam), _ptr(h_state), _ptr(g_state), _ptr(res["o"]),
               _ptr(res.get("steps")), _ptr(res.get("x")), int(max_steps),
               float(tol), _stream(stream))
    _check(code_, "mesa_decode_step_symh" if _symh else "mesa_decode_step")
    return res


def decode_step_warm(q, k, v, gamma, beta, lam, h_state, g_state, x_state, *, packed_h: bool = False,
                     max_steps: int = 32, tol: float = 1e-4, return_steps: bool = True,
                     out=None, stream=None) -> dict:
    """decode_step with CG started from x_state [N, H, d] fp32, which is overwritten
    with this token's solution (the next step's start).  h_state is [N, H, d, d], or
    [N, H, sym_state_floats(d)] in the blocked layout when packed_h."""
    N, H, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, H, d), q.dtype)
    _need(gamma, "gamma", (N, H), torch.float32)
    _need(beta, "beta", (N, H), torch.float32)
    _need(lam, "lam", (H, d), torch.float32)
    if packed_h:
        _need(h_state, "h_sym", (N, H, sym_state_floats(d)), torch.float32)
    else:
        _need(h_state, "h_state", (N, H, d, d), torch.float32)
    _need(g_state, "g_state", (N, H, d, d), torch.float32)
    _need(x_state, "x_state", (N, H, d), torch.float32)
    dev = q.device
    out = dict(out or {})
    res = {"o": out.get("o") if out.get("o") is not None else torch.empty((N, H, d), device=dev, dtype=torch.float32)}
    if return_steps:
        res["steps"] = out.get("steps") if out.get("steps") is not None else torch.empty((N, H), device=dev, dtype=torch.int32)
    code_ = lib().mesa_decode_step_warm(N, H, d, d, _ptr(q), _ptr(k), _ptr(v), code, _ptr(gamma), _ptr(beta),
                                        _ptr(lam), _ptr(h_state), 1 if packed_h else 0, _ptr(g_state),
                                        _ptr(x_state), _ptr(res["o"]), _ptr(res.get("steps")),
                                        int(max_steps), float(tol), _stream(stream))
    _check(code_, "mesa_decode_step_warm")
    return res


def qk_preprocess(q_raw, k_raw, w_q, w_k, *, q_hist=None, k_hist=None, eps: float = 1e-6,
                  return_history: bool = False, out=None, stream=None) -> dict:
    """Causal depthwise convolution of raw q, k [B, H, T, d] along time with taps
    w_q, w_k [H, d, W], then L2 normalisation per token.  q_hist, k_hist
    [B, H, W-1, d]: raw vectors before t = 0 (None: zeros).  Returns q, k (and,
    with return_history, the next call's histories q_hist, k_hist)."""
    B, H, T, d = q_raw.shape
    W = w_q.shape[-1]
    code = _dtype_code(q_raw)
    _need(q_raw, "q_raw", (B, H, T, d), q_raw.dtype)
    _need(k_raw, "k_raw", (B, H, T, d), q_raw.dtype)
    _need(w_q, "w_q", (H, d, W), torch.float32)
    _need(w_k, "w_k", (H, d, W), torch.float32)
    for name, t in (("q_hist", q_hist), ("k_hist", k_hist)):
        if t is not None:
            _need(t, name, (B, H, W - 1, d), q_raw.dtype)
    out = dict(out or {})
    dev = q_raw.device
    res = {}
    for key in ("q", "k"):
        res[key] = out.get(key) if out.get(key) is not None else torch.empty((B, H, T, d), device=dev, dtype=q_raw.dtype)
    if return_history:
        for key in ("q_hist", "k_hist"):
            res[key] = out.get(key) if out.get(key) is not None else torch.empty((B, H, W - 1, d), device=dev, dtype=q_raw.dtype)
    code_ = lib().mesa_qk_preprocess(B, H, T, d, W, code, _ptr(q_raw), _ptr(k_raw), _ptr(w_q), _ptr(w_k),
                                     _ptr(q_hist), _ptr(k_hist), float(eps), _ptr(res["q"]), _ptr(res["k"]),
                                     _ptr(res.get("q_hist")), _ptr(res.get("k_hist")), _stream(stream))
    _check(code_, "mesa_qk_preprocess")
    return res


def bwd_workspace_bytes(B, H, T, d, chunk, max_steps, tol, dtype_code=1) -> int:
    """Bytes of the backward's workspace (also a valid forward workspace)."""
    desc = make_desc(B, H, T, d, chunk, max_steps, tol, dtype_code)
    return int(lib().mesa_bwd_workspace_bytes(ctypes.byref(desc)))


def bwd_chunked(q, k, v, gamma, beta, lam, x, d_o, *, chunk: int = 64, max_steps: int = 30,
                tol: float = 0.0, h0=None, g0=None, d_hfinal=None, d_gfinal=None,
                state_grads: bool = False, return_steps: bool = False, out=None,
                workspace: Optional[torch.Tensor] = None, states_in_workspace: bool = False,
                stream=None) -> dict:
    """Backward of fwd_chunked: x is the forward's solutions (its return_x output),
    d_o [B, H, T, d] fp32 the gradient at o.  Returns dq, dk, dv [B, H, T, d],
    dgamma, dbeta [B, H, T], dlam [H, d] (fp32) and, with state_grads, dh0, dg0.
    states_in_workspace: the forward ran with ``workspace`` (bwd_workspace_bytes
    long) and left its boundary states there, so they are not recomputed."""
    return _bwd(False, q, k, v, gamma, beta, lam, x, d_o, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, d_hfinal=d_hfinal, d_gfinal=d_gfinal, state_grads=state_grads,
                return_steps=return_steps, out=out, workspace=workspace,
                states_in_workspace=states_in_workspace, stream=stream)


def bwd_chunked_ex(q, k, v, gamma, beta, lam, x, d_o, *, chunk: int = 64, max_steps: int = 30,
                   tol: float = 0.0, h0=None, g0=None, d_hfinal=None, d_gfinal=None,
                   state_grads: bool = False, return_steps: bool = False, out=None,
                   workspace: Optional[torch.Tensor] = None, states_in_workspace: bool = False,
                   stream=None) -> dict:
    """``bwd_chunked`` with ``lam`` the diagonal [H, d] or a full symmetric positive
    definite matrix per head [H, d, d]; with the full form ``dlam`` is [H, d, d],
    the partial derivative of each entry (-sum_t y_t x_t^T)."""
    return _bwd(True, q, k, v, gamma, beta, lam, x, d_o, chunk=chunk, max_steps=max_steps, tol=tol, h0=h0,
                g0=g0, d_hfinal=d_hfinal, d_gfinal=d_gfinal, state_grads=state_grads,
                return_steps=return_steps, out=out, workspace=workspace,
                states_in_workspace=states_in_workspace, stream=stream)


def _bwd(ex: bool, q, k, v, gamma, beta, lam, x, d_o, *, chunk, max_steps, tol, h0, g0, d_hfinal, d_gfinal,
         state_grads, return_steps, out, workspace, states_in_workspace, stream) -> dict:
    B, H, T, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (B, H, T, d), q.dtype)
    _need(gamma, "gamma", (B, H, T), torch.float32)
    _need(beta, "beta", (B, H, T), torch.float32)
    noalloc = ex == "noalloc"
    lam_full = ex is True and lam.dim() == 3
    _need(lam, "lam", (H, d, d) if lam_full else (H, d), torch.float32)
    for name, t in (("x", x), ("d_o", d_o)):
        _need(t, name, (B, H, T, d), torch.float32)
    for name, t in (("h0", h0), ("g0", g0), ("d_hfinal", d_hfinal), ("d_gfinal", d_gfinal)):
        if t is not None:
            _need(t, name, (B, H, d, d), torch.float32)
    desc = make_desc(B, H, T, d, chunk, max_steps, tol, code)
    L = lib()
    need = int(L.mesa_bwd_workspace_bytes(ctypes.byref(desc)))
    dev = q.device
    out = dict(out or {})
    f32 = torch.float32

    def get(key, shape, dtype=f32):
        return out.get(key) if out.get(key) is not None else torch.empty(shape, device=dev, dtype=dtype)

    res = {key: get(key, (B, H, T, d)) for key in ("dq", "dk", "dv")}
    res.update(dgamma=get("dgamma", (B, H, T)), dbeta=get("dbeta", (B, H, T)), dlam=get("dlam", (H, d, d) if lam_full else (H, d)))
    if state_grads:
        res.update(dh0=get("dh0", (B, H, d, d)), dg0=get("dg0", (B, H, d, d)))
    if return_steps:
        res["adj_steps"] = get("adj_steps", (B, H, T), torch.int32)
    if workspace is None:
        workspace = torch.empty(max(need, 1), device=dev, dtype=torch.uint8)
    wbytes = workspace.numel() * workspace.element_size()
    head = (ctypes.byref(desc), _ptr(q), _ptr(k), _ptr(v), _ptr(gamma), _ptr(beta), _ptr(lam))
    rest = (_ptr(h0), _ptr(g0), _ptr(x), _ptr(d_o), _ptr(d_hfinal), _ptr(d_gfinal),
            _ptr(res["dq"]), _ptr(res["dk"]), _ptr(res["dv"]), _ptr(res["dgamma"]),
            _ptr(res["dbeta"]), _ptr(res["dlam"]), _ptr(res.get("dh0")), _ptr(res.get("dg0")),
            _ptr(res.get("adj_steps")), 1 if states_in_workspace else 0, _ptr(workspace),
            ctypes.c_size_t(wbytes), _stream(stream))
    if ex:
        code_ = L.mesa_bwd_chunked_ex(*head, 1 if lam_full else 0, *rest)
        _check(code_, "mesa_bwd_chunked_ex")
    else:
        code_ = L.mesa_bwd_chunked(*head, *rest)
        _check(code_, "mesa_bwd_chunked")
    return res


def decode_step_ex(q, k, v, gamma, beta, lam, h_state, g_state, *, x_state=None, packed_h: bool = False,
                   max_steps: int = 32, tol: float = 1e-4, return_steps: bool = True, return_x: bool = False,
                   out=None, stream=None) -> dict:
    """The general decode step: lam [H, d] (diagonal) or [H, d, d] (full symmetric
    positive definite); h_state full or packed (packed_h); x_state [N, H, d] for a
    warm start (overwritten with the solution) or None for a cold start."""
    N, H, d = q.shape
    code = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _need(t, name, (N, H, d), q.dtype)
    _need(gamma, "gamma", (N, H), torch.float32)
    _need(beta, "beta", (N, H), torch.float32)
    full = lam.dim() == 3
    _need(lam, "lam", (H, d, d) if full else (H, d), torch.float32)
    _need(h_state, "h_state", (N, H, sym_state_floats(d)) if packed_h else (N, H, d, d), torch.float32)
    _need(g_state, "g_state", (N, H, d, d), torch.float32)
    if x_state is not None:
        _need(x_state, "x_state", (N, H, d), torch.float32)
    dev = q.device
    out = dict(out or {})
    res = {"o": out.get("o") if out.get("o") is not None else torch.empty((N, H, d), device=dev, dtype=torch.float32)}
    if return_steps:
        res["steps"] = out.get("steps") if out.get("steps") is not None else torch.empty((N, H), device=dev, dtype=torch.int32)
    if return_x and x_state is None:
        res["x"] = out.get("x") if out.get("x") is not None else torch.empty((N, H, d), device=dev, dtype=torch.float32)
    code_ = lib().mesa_decode_step_ex(N, H, d, d, _ptr(q), _ptr(k), _ptr(v), code, _ptr(gamma), _ptr(beta),
                                      _ptr(lam), 1 if full else 0, _ptr(h_state), 1 if packed_h else 0,
                                      _ptr(g_state), _ptr(x_state), _ptr(res["o"]), _ptr(res.get("steps")),
                                      _ptr(res.get("x")), int(max_steps), float(tol), _stream(stream))
    _check(code_, "mesa_decode_step_ex")
    return res
