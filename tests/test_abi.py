"""The C ABI library: load, exported symbols, host-side validation (CPU only).

No call here launches a kernel: every call either queries host-side
information or fails validation before the first launch.
"""
import ctypes
import os
import re

import pytest

from test_regression_sequence_amd import mesa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def header_functions():
    text = open(os.path.join(ROOT, "include", "mesa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mesa_[a-z_]+)\s*\(", text)))


def test_library_loads_and_exports_every_declared_symbol():
    L = mesa.lib()
    names = header_functions()
    assert {"mesa_fwd_chunked", "mesa_decode_step", "mesa_fwd_workspace_bytes",
            "mesa_status_string", "mesa_abi_version"} <= set(names)
    for name in names:
        assert hasattr(L, name), name


def test_version_and_status_strings():
    assert mesa.abi_version() == 1
    for code in range(6):
        assert mesa.status_string(code)
    assert mesa.status_string(99) == "unknown status"


def desc(**kw):
    base = dict(B=2, H=3, T=130, dk=64, dv=64, chunk=64, max_steps=5, tol=0.0, in_dtype=mesa.MESA_BF16)
    base.update(kw)
    return mesa.FwdDesc(*[base[f] for f, _ in mesa.FwdDesc._fields_])


def ws(d):
    return mesa.lib().mesa_fwd_workspace_bytes(ctypes.byref(d))


def test_workspace_sizes():
    # 2 states x B*H x ceil(T/C) chunks x d^2 x element size
    # (+ one int32 flag per chunk in 256-byte blocks for bf16 inputs)
    assert ws(desc()) == 2 * 6 * 3 * 64 * 64 * 2 + 256
    assert ws(desc(in_dtype=mesa.MESA_F32)) == 2 * 6 * 3 * 64 * 64 * 4
    assert ws(desc(T=0)) == 0
    assert ws(desc(dk=48, dv=48)) == 0
    assert ws(desc(dk=64, dv=32)) == 0
    assert ws(desc(chunk=48)) == 0
    assert ws(desc(B=8, H=16, T=4096, dk=128, dv=128)) == 512 * 1024 * 1024 + 8192 * 4
    # few (b, h) and a long sequence: the scan walks 8 segments of 64 chunks,
    # + 7 carry-in states per (b, h, state) in fp32 and one decay per (b, h, segment)
    assert ws(desc(B=1, H=16, T=32768, dk=128, dv=128)) == (
        2 * 16 * 512 * 128 * 128 * 2 + 16 * 512 * 4 + 16 * 2 * 7 * 128 * 128 * 4 + 512)


FAKE = 0x10000  # 16-byte aligned, never dereferenced: validation fails first


def call_fwd(d, q=FAKE, k=FAKE, v=FAKE, gamma=FAKE, beta=FAKE, lam=FAKE, o=FAKE,
             h0=None, workspace=FAKE, wbytes=1 << 40):
    P = ctypes.c_void_p
    return mesa.lib().mesa_fwd_chunked(ctypes.byref(d), P(q), P(k), P(v), P(gamma), P(beta), P(lam),
                                       P(h0), None, P(o), None, None, None, None, P(workspace),
                                       ctypes.c_size_t(wbytes), None)


@pytest.mark.parametrize("kw,expect", [
    (dict(B=0), 1), (dict(H=-1), 1), (dict(T=-5), 1), (dict(max_steps=-1), 1),
    (dict(tol=float("nan")), 1), (dict(in_dtype=7), 1),
    (dict(dk=48, dv=48), 2), (dict(dk=64, dv=128), 2), (dict(chunk=128), 2),
    (dict(dk=16, dv=16), 2),  # bf16 needs dk >= 32
])
def test_fwd_rejects_bad_descriptors(kw, expect):
    assert call_fwd(desc(**kw)) == expect


def call_fwd_noalloc(d, q=FAKE, lam=FAKE, o=FAKE):
    P = ctypes.c_void_p
    return mesa.lib().mesa_fwd_chunked_noalloc(ctypes.byref(d), P(q), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(lam),
                                               None, None, P(o), None, None, None, None, None)


def test_warm_forward_takes_bf16_inputs_only():
    P = ctypes.c_void_p
    d = desc(in_dtype=mesa.MESA_F32)
    code = mesa.lib().mesa_fwd_chunked_warm(ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                            None, None, P(FAKE), None, None, None, None, P(FAKE),
                                            ctypes.c_size_t(1 << 40), None)
    assert code == 2
    d = desc(B=0)
    assert mesa.lib().mesa_fwd_chunked_warm(ctypes.byref(d), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(FAKE),
                                            None, None, P(FAKE), None, None, None, None, P(FAKE),
                                            ctypes.c_size_t(1 << 40), None) == 1


def call_fwd_prep(d, window=4, eps=1e-6, q=FAKE, wq=FAKE, wk=FAKE, qh=None, kh=None, qho=None, kho=None,
                  o=FAKE, wbytes=1 << 40):
    P = ctypes.c_void_p
    return mesa.lib().mesa_fwd_chunked_prep(ctypes.byref(d), P(q), P(FAKE), P(FAKE), P(wq), P(wk), window,
                                            ctypes.c_float(eps), P(qh), P(kh), P(FAKE), P(FAKE), P(FAKE), None,
                                            None, P(o), None, None, None, None, P(qho), P(kho), P(FAKE),
                                            ctypes.c_size_t(wbytes), None)


def test_fused_preprocessing_forward_scope_and_validation():
    """mesa_fwd_chunked_prep takes bf16 inputs, chunk 64, d in {64, 128} and
    windows 1..4; every rejection happens before any launch."""
    assert call_fwd_prep(desc(in_dtype=mesa.MESA_F32)) == 2
    assert call_fwd_prep(desc(chunk=32)) == 2
    assert call_fwd_prep(desc(dk=32, dv=32)) == 2
    assert call_fwd_prep(desc(), window=5) == 2
    assert call_fwd_prep(desc(), window=0) == 1
    for eps in (0.0, -1.0, 2.0 ** -64, float("inf"), float("nan")):
        assert call_fwd_prep(desc(), eps=eps) == 1
    assert call_fwd_prep(desc(), wq=0) == 1
    assert call_fwd_prep(desc(), wk=0) == 1
    assert call_fwd_prep(desc(), wq=FAKE + 4) == 3
    assert call_fwd_prep(desc(), qh=FAKE + 8) == 3
    # the next call's histories may not overlap the raw inputs or each other
    assert call_fwd_prep(desc(), qho=FAKE + 1024) == 1
    far = FAKE + (1 << 32)
    assert call_fwd_prep(desc(), qho=far, kho=far + 256) == 1
    assert call_fwd_prep(desc(), qh=far, qho=far) == 1
    # the forward's own rules still apply
    assert call_fwd_prep(desc(B=0)) == 1
    assert call_fwd_prep(desc(dk=48, dv=48)) == 2
    assert call_fwd_prep(desc(), q=0) == 1
    assert call_fwd_prep(desc(), o=FAKE + 4) == 3
    assert call_fwd_prep(desc(), wbytes=16) == 4


def test_noalloc_forward_validates_before_any_hip_call():
    """The allocation-free forward rejects, before any HIP call (this runs without
    a GPU): a workload whose workspace exceeds the static scratch, then the
    descriptor and pointer rules of mesa_fwd_chunked."""
    assert mesa.NOALLOC_SCRATCH_BYTES == 64 << 20
    big = desc(B=8, H=16, T=4096, dk=128, dv=128)
    assert ws(big) > mesa.NOALLOC_SCRATCH_BYTES
    assert call_fwd_noalloc(big) == 2
    # the largest workload of its shape family that fits: B=4, H=8, T=2048, d=64 (16 MiB)
    assert ws(desc(B=4, H=8, T=2048, dk=64, dv=64)) <= mesa.NOALLOC_SCRATCH_BYTES
    assert call_fwd_noalloc(desc(B=0)) == 1
    assert call_fwd_noalloc(desc(dk=48, dv=48)) == 2
    assert call_fwd_noalloc(desc(), q=0) == 1
    assert call_fwd_noalloc(desc(), lam=0) == 1
    assert call_fwd_noalloc(desc(), o=FAKE + 4) == 3


def call_fwd_ex(d, lam_full, q=FAKE, lam=FAKE, o=FAKE, workspace=FAKE, wbytes=1 << 40):
    P = ctypes.c_void_p
    return mesa.lib().mesa_fwd_chunked_ex(ctypes.byref(d), P(q), P(FAKE), P(FAKE), P(FAKE), P(FAKE), P(lam),
                                          lam_full, None, None, P(o), None, None, None, None, P(workspace),
                                          ctypes.c_size_t(wbytes), None)


def test_full_lambda_forward_scope_and_validation():
    # the full-Lambda forward takes bf16 inputs, chunk 64 and d in {64, 128};
    # every other descriptor is rejected before any launch
    assert call_fwd_ex(desc(in_dtype=mesa.MESA_F32), 1) == 2
    assert call_fwd_ex(desc(chunk=32), 1) == 2
    assert call_fwd_ex(desc(dk=32, dv=32), 1) == 2
    # the descriptor rules and pointer checks of mesa_fwd_chunked still come first
    assert call_fwd_ex(desc(B=0), 1) == 1
    assert call_fwd_ex(desc(dk=48, dv=48), 1) == 2
    assert call_fwd_ex(desc(), 1, q=0) == 1
    assert call_fwd_ex(desc(), 1, lam=0) == 1
    assert call_fwd_ex(desc(), 1, o=FAKE + 4) == 3
    assert call_fwd_ex(desc(), 1, wbytes=16) == 4
    # lambda_full takes 0 or 1 only, like the backward and decode _ex calls
    assert call_fwd_ex(desc(), 2) == 1
    assert call_fwd_ex(desc(), -1) == 1
    # lambda_full = 0 keeps the diagonal forward's scope (fp32 and chunk 32 allowed)
    assert call_fwd_ex(desc(in_dtype=mesa.MESA_F32), 0, q=0) == 1
    assert call_fwd_ex(desc(chunk=32), 0, wbytes=16) == 4


def test_fwd_rejects_missing_pointers_alignment_and_workspace():
    d = desc()
    assert call_fwd(d, q=0) == 1
    assert call_fwd(d, o=0) == 1
    assert call_fwd(d, lam=0) == 1
    assert call_fwd(d, k=FAKE + 4) == 3
    assert call_fwd(d, h0=FAKE + 8) == 3
    assert call_fwd(d, workspace=0) == 4
    assert call_fwd(d, wbytes=ws(d) - 1) == 4


def call_dec(N=4, H=2, dk=128, dv=128, dtype=1, q=FAKE, h=FAKE, o=FAKE, max_steps=8, tol=1e-4):
    P = ctypes.c_void_p
    return mesa.lib().mesa_decode_step(N, H, dk, dv, P(q), P(FAKE), P(FAKE), dtype, P(FAKE), P(FAKE),
                                       P(FAKE), P(h), P(FAKE), P(o), None, None, max_steps,
                                       ctypes.c_float(tol), None)


def test_decode_validation():
    assert call_dec(N=-1) == 1
    assert call_dec(H=0) == 1
    assert call_dec(max_steps=-2) == 1
    assert call_dec(tol=float("nan")) == 1
    assert call_dec(dtype=3) == 1
    assert call_dec(dk=96, dv=96) == 2
    assert call_dec(dk=128, dv=64) == 2
    assert call_dec(q=0) == 1
    assert call_dec(h=0) == 1
    assert call_dec(o=FAKE + 2) == 3
    assert call_dec(N=0) == 0  # nothing to do, nothing launched


def test_packed_state_sizes_and_validation():
    L = mesa.lib()
    assert L.mesa_sym_state_floats(128) == 36 * 256
    assert L.mesa_sym_state_floats(64) == 10 * 256
    assert L.mesa_sym_state_floats(32) == 0
    P = ctypes.c_void_p
    assert L.mesa_sym_pack(4, 48, P(FAKE), P(FAKE), None) == 2
    assert L.mesa_sym_pack(-1, 128, P(FAKE), P(FAKE), None) == 1
    assert L.mesa_sym_pack(4, 128, None, P(FAKE), None) == 1
    assert L.mesa_sym_unpack(4, 128, P(FAKE + 4), P(FAKE), None) == 3
    assert L.mesa_sym_pack(0, 128, None, None, None) == 0
    args = [P(FAKE)] * 3 + [1] + [P(FAKE)] * 8
    assert L.mesa_decode_step_symh(2, 2, 96, 96, *args, 8, ctypes.c_float(1e-4), None) == 2
    assert L.mesa_decode_step_symh(2, 2, 128, 128, *args, -1, ctypes.c_float(1e-4), None) == 1


def test_warm_decode_validation():
    L = mesa.lib()
    P = ctypes.c_void_p

    def call(h_packed=0, x_state=FAKE, dk=128, max_steps=8):
        return L.mesa_decode_step_warm(2, 2, dk, dk, P(FAKE), P(FAKE), P(FAKE), 1, P(FAKE), P(FAKE), P(FAKE),
                                       P(FAKE), h_packed, P(FAKE), P(x_state) if x_state else None,
                                       P(FAKE), None, max_steps, ctypes.c_float(1e-4), None)

    assert call(x_state=0) == 1        # the start is required
    assert call(h_packed=2) == 1
    assert call(h_packed=-1) == 1
    assert call(dk=96) == 2
    assert call(max_steps=-1) == 1
    assert call(x_state=FAKE + 4) == 3


def test_backward_full_lambda_validation():
    L = mesa.lib()
    P = ctypes.c_void_p
    desc = mesa.make_desc(2, 2, 128, 128, 64, 8, 0.0, 1)
    need = L.mesa_bwd_workspace_bytes(ctypes.byref(desc))

    def call(desc=desc, lam_full=1, ws_bytes=need, dlam=FAKE):
        ptrs = [P(FAKE)] * 21
        ptrs[6] = ptrs[7] = ptrs[10] = ptrs[11] = None          # h0, g0, d_hfinal, d_gfinal
        ptrs[17] = P(dlam) if dlam else None
        ptrs[18] = ptrs[19] = ptrs[20] = None                    # dh0, dg0, adj_steps
        return L.mesa_bwd_chunked_ex(ctypes.byref(desc), *ptrs[:6], lam_full, *ptrs[6:], 0, P(FAKE),
                                     ctypes.c_size_t(ws_bytes), None)

    assert call(lam_full=2) == 1
    assert call(lam_full=-1) == 1
    assert call(dlam=0) == 1
    assert call(dlam=FAKE + 4) == 3
    assert call(ws_bytes=need - 1) == 4
    assert call(desc=mesa.make_desc(2, 2, 128, 128, 64, 8, 0.0, 0)) == 2   # fp32 inputs
    assert call(desc=mesa.make_desc(2, 2, 128, 128, 32, 8, 0.0, 1)) == 2   # chunk 32
    assert call(desc=mesa.make_desc(2, 2, 128, 32, 64, 8, 0.0, 1)) == 2    # d 32


def test_preprocess_validation():
    L = mesa.lib()
    P = ctypes.c_void_p
    A, Bp = 0x7F0000000000, 0x7F1000000000   # distinct 16-byte aligned fake ranges

    def call(B=2, H=2, T=8, d=128, W=4, dtype=1, eps=1e-6, q=A, k=A + 0x100000, qo=Bp, ko=Bp + 0x100000,
             wq=A + 0x200000, qh=0, qho=0):
        return L.mesa_qk_preprocess(B, H, T, d, W, dtype, P(q) if q else None, P(k) if k else None,
                                    P(wq) if wq else None, P(A + 0x300000), P(qh) if qh else None, None,
                                    ctypes.c_float(eps), P(qo) if qo else None, P(ko) if ko else None,
                                    P(qho) if qho else None, None, None)

    assert call(d=96) == 2
    assert call(W=5) == 2
    assert call(W=0) == 1
    assert call(T=-1) == 1
    assert call(eps=0.0) == 1
    assert call(eps=2.0 ** -64) == 1   # below 2^-63: the norm of a denormal squared norm
    assert call(eps=float("inf")) == 1
    assert call(dtype=3) == 1
    assert call(q=0) == 1
    assert call(wq=0) == 1
    assert call(qo=Bp + 4) == 3
    assert call(qo=A) == 1                   # output over the raw input
    assert call(qo=A + 0x100000) == 1        # output over the other raw input
    assert call(qh=Bp + 0x400000, qho=Bp + 0x400000) == 1  # history out over history in
    assert call(B=0) == 0


def test_general_decode_validation():
    L = mesa.lib()
    P = ctypes.c_void_p

    def call(lam_full=0, h_packed=0, x_state=0, x_out=0):
        return L.mesa_decode_step_ex(2, 2, 128, 128, P(FAKE), P(FAKE), P(FAKE), 1, P(FAKE), P(FAKE), P(FAKE),
                                     lam_full, P(FAKE), h_packed, P(FAKE), P(x_state) if x_state else None,
                                     P(FAKE), None, P(x_out) if x_out else None, 8, ctypes.c_float(1e-4), None)

    assert call(lam_full=2) == 1
    assert call(h_packed=3) == 1
    assert call(x_state=FAKE, x_out=FAKE) == 1
    assert call(x_state=FAKE + 4) == 3


def test_backward_validation():
    L = mesa.lib()
    P = ctypes.c_void_p
    desc = mesa.make_desc(2, 2, 128, 128, 64, 8, 0.0, 1)
    need = L.mesa_bwd_workspace_bytes(ctypes.byref(desc))
    assert need >= L.mesa_fwd_workspace_bytes(ctypes.byref(desc))
    assert L.mesa_bwd_workspace_bytes(ctypes.byref(mesa.make_desc(2, 2, 128, 128, 64, 8, 0.0, 0))) == 0  # fp32
    assert L.mesa_bwd_workspace_bytes(ctypes.byref(mesa.make_desc(2, 2, 128, 128, 32, 8, 0.0, 1))) == 0  # chunk 32

    def call(desc=desc, flag=0, ws_bytes=need, lam=FAKE, ws=FAKE):
        ptrs = [P(FAKE)] * 21
        ptrs[5] = P(lam) if lam else None
        ptrs[6] = None   # h0
        ptrs[7] = None   # g0
        ptrs[10] = None  # d_hfinal
        ptrs[11] = None  # d_gfinal
        ptrs[18] = None  # dh0
        ptrs[19] = None  # dg0
        ptrs[20] = None  # adj_steps
        return L.mesa_bwd_chunked(ctypes.byref(desc), *ptrs, flag, P(ws) if ws else None,
                                  ctypes.c_size_t(ws_bytes), None)

    assert call(flag=2) == 1
    assert call(lam=0) == 1
    assert call(ws_bytes=need - 1) == 4
    assert call(ws=0) == 4
    assert call(desc=mesa.make_desc(2, 2, 128, 96, 64, 8, 0.0, 1)) == 2
    assert call(ws=FAKE + 4) == 3
