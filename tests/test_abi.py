"""C-ABI checks that need no GPU: the library loads, exports every entry point
include/relation.h declares, and rejects every invalid call with its status
code before any HIP call (so nothing here launches a kernel)."""
import ctypes
import os
import re

import numpy as np
import pytest

from causal_self_exchange_amd import relation as R

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

OK, E_NULL, E_SHAPE, E_DTYPE, E_HEADDIM, E_TAU, E_LAMBDA, E_ALIGN, E_ALIAS, E_WS, E_LAUNCH, E_PRESTEP, E_KERNEL = range(13)

# Fake, never-dereferenced device addresses (16-byte aligned, far apart).
A, B_, C, Y = 0x10000000, 0x20000000, 0x30000000, 0x40000000


def _tau(vals):
    arr = np.asarray(vals, dtype=np.float32)
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def declared_symbols():
    text = open(os.path.join(ROOT, "include", "relation.h")).read()
    return sorted(set(re.findall(r"\b(relation_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = R.lib()
    syms = declared_symbols()
    assert set(syms) == set(R.EXPORTS)
    for s in syms:
        assert hasattr(lib, s), s


def test_library_exports_nothing_else():
    """Internal functions are built with hidden visibility: the dynamic text
    symbols of the library are exactly the declared entry points."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm is not available")
    R.lib()
    out = subprocess.run([nm, "-D", "--defined-only", R.LIB_PATH], capture_output=True, text=True, check=True).stdout
    text = {f[2] for f in (line.split() for line in out.splitlines()) if len(f) == 3 and f[1] == "T"}
    assert text == set(declared_symbols()), sorted(text ^ set(declared_symbols()))


def test_status_strings():
    lib = R.lib()
    for code in range(13):
        assert lib.relation_status_str(code) not in (b"", b"unknown status")
    assert lib.relation_status_str(99) == b"unknown status"


def fwd(P1=A, P2=B_, V=C, tau=(1.0, 1.0), lam=0.0, Yp=Y, B=1, H=2, T=16, D=64, dt=R.REL_BF16):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    return R.lib().relation_fwd_ex(P1, P2, V, tp, lam, Yp, B, H, T, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(P1=None), E_NULL), (dict(V=None), E_NULL), (dict(Yp=None), E_NULL), (dict(tau=None), E_NULL),
    (dict(T=0), E_SHAPE), (dict(B=0), E_SHAPE), (dict(H=0, tau=(1.0,)), E_SHAPE), (dict(D=-64), E_SHAPE),
    (dict(B=70000), E_SHAPE), (dict(H=257, tau=[1.0] * 257), E_SHAPE),
    (dict(T=2**31 - 1, B=65535, H=256, tau=[1.0] * 256, D=128), E_SHAPE),
    (dict(dt=7), E_DTYPE), (dict(D=96), E_HEADDIM), (dict(D=256), E_HEADDIM), (dict(D=40), E_HEADDIM),
    (dict(tau=(1.0, 0.0)), E_TAU), (dict(tau=(-1.0, 1.0)), E_TAU),
    (dict(tau=(1.0, float("nan"))), E_TAU), (dict(tau=(float("inf"), 1.0)), E_TAU),
    (dict(lam=float("nan")), E_LAMBDA), (dict(lam=float("inf")), E_LAMBDA),
    (dict(P2=B_ + 8), E_ALIGN), (dict(Yp=Y + 2), E_ALIGN),
    (dict(Yp=A), E_ALIAS), (dict(Yp=C + 16), E_ALIAS), (dict(Yp=B_ - 16), E_ALIAS),
])
def test_fwd_rejects_invalid_arguments(kw, code):
    assert fwd(**kw) == code


def test_fwd_plain_entry_rejects_like_ex():
    keep, tp = _tau([1.0, -2.0])
    assert R.lib().relation_fwd(A, B_, C, tp, Y, 1, 2, 16, 64, R.REL_BF16, None) == E_TAU
    assert R.lib().relation_fwd(None, B_, C, tp, Y, 1, 2, 16, 64, R.REL_BF16, None) == E_NULL


def test_decode_workspace_bytes():
    lib = R.lib()
    assert lib.relation_decode_workspace_bytes(64, 32, 4096, 128) == 64 * 32 * 16 * 130 * 4
    assert lib.relation_decode_workspace_bytes(2, 3, 1, 32) == 2 * 3 * 1 * 34 * 4
    assert lib.relation_decode_workspace_bytes(2, 3, 257, 64) == 2 * 3 * 2 * 66 * 4
    assert lib.relation_decode_workspace_bytes(0, 3, 10, 64) == 0
    assert lib.relation_decode_workspace_bytes(1, 1, 10, 96) == 0
    # the paper's head sizes 48 and 80 (states of d_h + 2 floats per chunk)
    assert lib.relation_decode_workspace_bytes(1, 2, 300, 48) == 1 * 2 * 2 * 50 * 4
    assert lib.relation_decode_workspace_bytes(1, 1, 256, 80) == 82 * 4


LEN, WS, YD, CP, CV = 0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000


def dec(p1=A, p2=B_, v=C, cP2=CP, cV=CV, ln=LEN, tau=(1.0, 1.0), lam=0.0, y=YD,
        B=2, H=2, L=300, D=128, dt=R.REL_BF16, ws=WS, wsb=None):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    if wsb is None:
        wsb = R.lib().relation_decode_workspace_bytes(B, H, L, D)
    return R.lib().relation_decode(p1, p2, v, cP2, cV, ln, tp, lam, y, B, H, L, D, dt, ws, wsb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(p1=None), E_NULL), (dict(cV=None), E_NULL), (dict(ln=None), E_NULL), (dict(y=None), E_NULL),
    (dict(L=0), E_SHAPE), (dict(B=-1), E_SHAPE), (dict(dt=3), E_DTYPE), (dict(D=96), E_HEADDIM),
    (dict(tau=(0.0, 1.0)), E_TAU), (dict(lam=float("-inf")), E_LAMBDA),
    (dict(ws=None), E_WS), (dict(wsb=16), E_WS),
    (dict(cP2=CP + 4), E_ALIGN), (dict(ln=LEN + 2), E_ALIGN), (dict(ws=WS + 8), E_ALIGN),
    (dict(y=A), E_ALIAS), (dict(y=CP + 1024), E_ALIAS), (dict(ws=CV + 4096), E_ALIAS),
    (dict(y=WS + 64), E_ALIAS),
])
def test_decode_rejects_invalid_arguments(kw, code):
    assert dec(**kw) == code


def dec_noalloc(p1=A, p2=B_, v=C, cP2=CP, cV=CV, ln=LEN, tau=(1.0, 1.0), lam=0.0, y=YD,
                B=2, H=2, L=300, D=128, dt=R.REL_BF16):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    return R.lib().relation_decode_noalloc(p1, p2, v, cP2, cV, ln, tp, lam, y, B, H, L, D, dt, None)


# Every rejection of relation_decode_noalloc, the size limit of its scratch
# array included, comes before its one HIP call (the array's address).
@pytest.mark.parametrize("kw,code", [
    (dict(p1=None), E_NULL), (dict(ln=None), E_NULL), (dict(y=None), E_NULL), (dict(L=0), E_SHAPE),
    (dict(dt=3), E_DTYPE), (dict(D=96), E_HEADDIM), (dict(tau=(0.0, 1.0)), E_TAU),
    (dict(lam=float("nan")), E_LAMBDA), (dict(cP2=CP + 4), E_ALIGN), (dict(ln=LEN + 2), E_ALIGN),
    (dict(y=A), E_ALIAS), (dict(y=CP + 1024), E_ALIAS), (dict(y=LEN), E_ALIAS),
    # 64 x 64 heads, 8192 cached rows, d_h 128: 64 MiB of partial states > 32 MiB
    (dict(B=64, H=64, L=8192, tau=[1.0] * 64), E_WS),
])
def test_decode_noalloc_rejects_invalid_arguments(kw, code):
    assert dec_noalloc(**kw) == code


def test_decode_noalloc_scratch_limit():
    lib = R.lib()
    assert lib.relation_decode_workspace_bytes(64, 32, 4096, 128) <= 32 << 20      # the decode workload fits
    assert lib.relation_decode_workspace_bytes(64, 64, 8192, 128) > 32 << 20


def test_cache_append_rejects_invalid_arguments():
    lib = R.lib()
    f = lib.relation_cache_append
    assert f(None, CV, LEN, A, C, 2, 2, 300, 128, R.REL_BF16, None) == E_NULL
    assert f(CP, CV, LEN, A, C, 2, 2, 0, 128, R.REL_BF16, None) == E_SHAPE
    assert f(CP, CV, LEN, A, C, 2, 2, 300, 96, R.REL_BF16, None) == E_HEADDIM
    assert f(CP, CV, LEN, A, C, 2, 2, 300, 128, 5, None) == E_DTYPE
    assert f(CP, CV, LEN + 1, A, C, 2, 2, 300, 128, R.REL_BF16, None) == E_ALIGN
    assert f(CP, CP + 256, LEN, A, C, 2, 2, 300, 128, R.REL_BF16, None) == E_ALIAS
    assert f(CP, CV, CV + 64, A, C, 2, 2, 300, 128, R.REL_BF16, None) == E_ALIAS


def test_select_kernels():
    f = R.lib().relation_select_kernels
    assert f(0, 0) == OK and f(1, 0) == OK and f(0, 1) == OK and f(1, 1) == OK
    assert f(2, 0) == E_KERNEL and f(0, -1) == E_KERNEL
    assert f(0, 0) == OK
    with pytest.raises(KeyError):
        R.select_kernels("fast")


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(1, 1, 4, 32)
    with pytest.raises(ValueError):
        R.fwd(x, x, x, 1.0)


# Fake addresses for the training forward / backward (far apart, aligned).
LSE_, DY_, G1, G2, G3, DT, DL, WS = (0x50000000, 0x60000000, 0x70000000, 0x80000000, 0x90000000,
                                     0xA0000000, 0xA0001000, 0xB0000000)


def fwd_lse(P1=A, P2=B_, V=C, tau=(1.0, 1.0), lam=0.0, Yp=Y, L=LSE_, B=1, H=2, T=16, D=64, dt=R.REL_BF16):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    return R.lib().relation_fwd_lse(P1, P2, V, tp, lam, Yp, L, B, H, T, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(L=None), E_NULL), (dict(P1=None), E_NULL), (dict(T=0), E_SHAPE), (dict(D=96), E_HEADDIM),
    (dict(tau=(1.0, 0.0)), E_TAU), (dict(L=LSE_ + 2), E_ALIGN), (dict(L=A + 64), E_ALIAS),
    (dict(L=Y + 4), E_ALIAS), (dict(L=Y - 4), E_ALIAS),
])
def test_fwd_lse_rejects_invalid_arguments(kw, code):
    assert fwd_lse(**kw) == code


def test_bwd_workspace_bytes():
    lib = R.lib()
    # statistics: B*H*ceil(T/64)*256 floats; partials: B*H*ceil(T/256)*2 floats; each 256-aligned
    def want(B, H, T):
        a = B * H * ((T + 63) // 64) * 256 * 4
        b = B * H * ((T + 255) // 256) * 2 * 4
        return ((a + 255) // 256) * 256 + ((b + 255) // 256) * 256
    assert lib.relation_bwd_workspace_bytes(1, 32, 8192, 128) == want(1, 32, 8192)
    assert lib.relation_bwd_workspace_bytes(2, 3, 1, 32) == want(2, 3, 1)
    assert lib.relation_bwd_workspace_bytes(4, 16, 2049, 64) == want(4, 16, 2049)
    assert lib.relation_bwd_workspace_bytes(0, 3, 10, 64) == 0
    assert lib.relation_bwd_workspace_bytes(1, 1, 10, 96) == 0
    assert lib.relation_bwd_workspace_bytes(4, 8, 1024, 48) == want(4, 8, 1024)


def test_bwd_stored_workspace_bytes():
    """The statistics and partials, then per head nqp (nqp + 1) blocks of
    1 KB (nqp = ceil(T / 32)), 256-aligned; 0 where the path does not exist."""
    lib = R.lib()
    def want(B, H, T, D):
        nqp = (T + 31) // 32
        du = B * H * nqp * (nqp + 1) * 1024
        return lib.relation_bwd_workspace_bytes(B, H, T, D) + ((du + 255) // 256) * 256
    for B, H, T, D in ((1, 32, 8192, 128), (2, 3, 1, 64), (4, 16, 2049, 64), (1, 2, 300, 48), (1, 1, 77, 80),
                       (2, 2, 100, 32)):
        assert lib.relation_bwd_stored_workspace_bytes(B, H, T, D) == want(B, H, T, D)
    assert lib.relation_bwd_stored_workspace_bytes(1, 32, 8192, 128) == 2_155_872_256 + \
        lib.relation_bwd_workspace_bytes(1, 32, 8192, 128)
    assert lib.relation_bwd_stored_workspace_bytes(1, 1, 10, 96) == 0
    assert lib.relation_bwd_stored_workspace_bytes(0, 1, 10, 64) == 0
    assert lib.relation_bwd_stored_workspace_bytes(1, 1, 46304, 64) > 0     # largest length with 31-bit offsets
    assert lib.relation_bwd_stored_workspace_bytes(1, 1, 46305, 64) == 0


def bwd(P1=A, P2=B_, V=C, tau=(1.0, 1.0), lam=0.0, Yp=Y, L=LSE_, dY=DY_, dP1=G1, dP2=G2, dV=G3,
        dtau=DT, dlam=DL, B=1, H=2, T=16, D=64, dt=R.REL_BF16, ws=WS, ws_bytes=None):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    if ws_bytes is None:
        ws_bytes = R.lib().relation_bwd_workspace_bytes(B, H, T, D) if T > 0 and B > 0 else 0
    return R.lib().relation_bwd(P1, P2, V, tp, lam, Yp, L, dY, dP1, dP2, dV, dtau, dlam, B, H, T, D, dt,
                                ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(dY=None), E_NULL), (dict(L=None), E_NULL), (dict(dtau=None), E_NULL), (dict(dlam=None), E_NULL),
    (dict(dP2=None), E_NULL), (dict(tau=None), E_NULL),
    (dict(T=0), E_SHAPE), (dict(B=70000), E_SHAPE), (dict(H=257, tau=[1.0] * 257), E_SHAPE),
    (dict(dt=3), E_DTYPE), (dict(D=96), E_HEADDIM), (dict(tau=(1.0, float("nan"))), E_TAU),
    (dict(lam=float("inf")), E_LAMBDA),
    (dict(ws=None), E_WS), (dict(ws_bytes=1000), E_WS),
    (dict(dP1=G1 + 8), E_ALIGN), (dict(ws=WS + 8), E_ALIGN), (dict(dtau=DT + 2), E_ALIGN),
    (dict(L=LSE_ + 1), E_ALIGN),
    (dict(dP1=A), E_ALIAS), (dict(dV=DY_ + 16), E_ALIAS), (dict(dtau=LSE_ + 4), E_ALIAS),
    (dict(dP2=G1 + 16), E_ALIAS), (dict(dlam=DT + 4), E_ALIAS), (dict(ws=G3), E_ALIAS),
    (dict(dV=Y - 16), E_ALIAS),
])
def test_bwd_rejects_invalid_arguments(kw, code):
    assert bwd(**kw) == code


def prestep(P1=A, P2=B_, I=C, pos0=None, rope=1, base=1e4, theta=(0.3,), pairing=0, P1o=G1, P2o=G2, Io=G3,
            B=1, H=2, T=16, D=64, dt=R.REL_BF16):
    keep, tp = _tau(theta) if theta is not None else (None, None)
    return R.lib().relation_prestep(P1, P2, I, pos0, rope, base, tp, pairing, P1o, P2o, Io, B, H, T, D, dt, None)


@pytest.mark.parametrize("kw,code", [
    (dict(P1=None), E_NULL), (dict(Io=None), E_NULL), (dict(T=0), E_SHAPE), (dict(D=96), E_HEADDIM),
    (dict(dt=5), E_DTYPE), (dict(H=3, theta=(0.1,)), E_SHAPE), (dict(rope=3), E_PRESTEP),
    (dict(pairing=2), E_PRESTEP), (dict(base=1.0), E_PRESTEP), (dict(base=float("nan")), E_PRESTEP),
    (dict(theta=(float("inf"),)), E_PRESTEP), (dict(P1o=G1 + 8), E_ALIGN), (dict(pos0=DT + 2), E_ALIGN),
    (dict(P1o=B_), E_ALIAS), (dict(Io=G1 + 16), E_ALIAS), (dict(P2o=A + 64), E_ALIAS),
    (dict(pos0=G3 + 32), E_ALIAS),
])
def test_prestep_rejects_invalid_arguments(kw, code):
    assert prestep(**kw) == code


def test_fwd_model_workspace_bytes():
    lib = R.lib()
    n = 1 * 32 * 8192 * 128
    assert lib.relation_fwd_model_workspace_bytes(1, 32, 8192, 128, R.REL_BF16) == 3 * n * 2
    assert lib.relation_fwd_model_workspace_bytes(1, 1, 3, 32, R.REL_F32) == 3 * 512
    assert lib.relation_fwd_model_workspace_bytes(1, 1, 3, 96, R.REL_F32) == 0
    # the paper's head sizes 48 and 80 are accepted by the forward family
    assert lib.relation_fwd_model_workspace_bytes(1, 1, 3, 48, R.REL_F32) == 3 * 768
    assert lib.relation_fwd_model_workspace_bytes(2, 8, 1024, 80, R.REL_BF16) == 3 * 2 * 8 * 1024 * 80 * 2


def fwd_model(P1=A, P2=B_, I=C, pos0=None, rope=1, base=1e4, theta=(0.3,), pairing=0, tau=(1.0, 1.0), lam=0.0,
              Yp=Y, L=None, B=1, H=2, T=16, D=64, dt=R.REL_BF16, ws=WS, ws_bytes=None):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    keep2, thp = _tau(theta) if theta is not None else (None, None)
    if ws_bytes is None:
        ws_bytes = R.lib().relation_fwd_model_workspace_bytes(B, H, T, D, dt) if T > 0 else 0
    return R.lib().relation_fwd_model(P1, P2, I, pos0, rope, base, thp, pairing, tp, lam, Yp, L, B, H, T, D, dt,
                                      ws, ws_bytes, None)


# Every check of relation_fwd_model, including those of the forward it runs
# after the pre-steps (Y and LSE against the inputs, the workspace, each
# other and pos0), happens before the pre-step kernel is enqueued.
@pytest.mark.parametrize("kw,code", [
    (dict(P1=None), E_NULL), (dict(Yp=None), E_NULL), (dict(tau=None), E_NULL), (dict(T=0), E_SHAPE),
    (dict(D=96), E_HEADDIM), (dict(dt=5), E_DTYPE), (dict(ws=None), E_WS), (dict(ws_bytes=1024), E_WS),
    (dict(rope=3), E_PRESTEP), (dict(theta=(float("inf"),)), E_PRESTEP), (dict(tau=(1.0, 0.0)), E_TAU),
    (dict(lam=float("nan")), E_LAMBDA), (dict(Yp=Y + 2), E_ALIGN), (dict(L=LSE_ + 2), E_ALIGN),
    (dict(Yp=A), E_ALIAS), (dict(Yp=WS + 64), E_ALIAS), (dict(L=A + 64), E_ALIAS), (dict(L=WS + 16), E_ALIAS),
    (dict(L=Y + 4), E_ALIAS), (dict(L=Y - 4), E_ALIAS), (dict(L=LSE_, pos0=LSE_ + 8), E_ALIAS),
])
def test_fwd_model_rejects_invalid_arguments(kw, code):
    assert fwd_model(**kw) == code


def linear(P1=A, P2=B_, I=C, alpha=DY_, tau=(1.0, 1.0), Yp=Y, state=None, B=1, H=2, T=100, D=64,
           dt=R.REL_BF16, ws=WS, ws_bytes=None):
    keep, tp = _tau(tau) if tau is not None else (None, None)
    if ws_bytes is None:
        ws_bytes = R.lib().relation_linear_workspace_bytes(B, H, T, D) if T > 0 and B > 0 else 0
    return R.lib().relation_linear_fwd(P1, P2, I, alpha, tp, Yp, state, B, H, T, D, dt, ws, ws_bytes, None)


@pytest.mark.parametrize("kw,code", [
    (dict(alpha=None), E_NULL), (dict(Yp=None), E_NULL), (dict(tau=None), E_NULL), (dict(T=0), E_SHAPE),
    (dict(D=48), E_HEADDIM), (dict(dt=9), E_DTYPE), (dict(tau=(1.0, -1.0)), E_TAU), (dict(ws=None), E_WS),
    (dict(ws_bytes=100), E_WS), (dict(alpha=DY_ + 4), E_ALIGN), (dict(state=G1 + 8), E_ALIGN),
    (dict(Yp=A), E_ALIAS), (dict(state=DY_ + 64), E_ALIAS), (dict(ws=C + 16), E_ALIAS), (dict(state=WS), E_ALIAS),
])
def test_linear_rejects_invalid_arguments(kw, code):
    assert linear(**kw) == code


def test_linear_workspace_bytes():
    lib = R.lib()
    # chunk states, chunk decays and two row factors per token, each 256-byte aligned
    assert lib.relation_linear_workspace_bytes(1, 32, 8192, 128) == (32 * 128 * 128 * 128 * 4 + 32 * 128 * 128 * 4
                                                                     + 32 * 8192 * 2 * 4)
    assert lib.relation_linear_workspace_bytes(1, 1, 1, 32) == 32 * 32 * 4 + 256 + 256
    assert lib.relation_linear_workspace_bytes(1, 1, 10, 48) == 0
