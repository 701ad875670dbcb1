"""Thin Python binding over librelation.so (ctypes).

Argument marshalling only: every step of the forward, backward and decode runs in the
HIP kernels behind the C ABI (include/relation.h). PyTorch supplies device
memory and the current stream. There is no CPU fallback: if the library is
missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np
import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "librelation.so")

REL_F32, REL_BF16 = 0, 1
_DT = {torch.float32: REL_F32, torch.bfloat16: REL_BF16}

_lib = None


class RelationError(RuntimeError):
    def __init__(self, fn: str, status: int):
        msg = lib().relation_status_str(status).decode()
        super().__init__(f"{fn} failed: status {status} ({msg})")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load librelation.so once; raise if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run causal_self_exchange_amd.build first")
        L = ctypes.CDLL(LIB_PATH)
        vp, i, f, fp, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_float, ctypes.POINTER(ctypes.c_float), ctypes.c_size_t
        L.relation_fwd.argtypes = [vp, vp, vp, fp, vp, i, i, i, i, i, vp]
        L.relation_fwd.restype = i
        L.relation_fwd_ex.argtypes = [vp, vp, vp, fp, f, vp, i, i, i, i, i, vp]
        L.relation_fwd_ex.restype = i
        L.relation_fwd_lse.argtypes = [vp, vp, vp, fp, f, vp, vp, i, i, i, i, i, vp]
        L.relation_fwd_lse.restype = i
        L.relation_bwd_workspace_bytes.argtypes = [i, i, i, i]
        L.relation_bwd_workspace_bytes.restype = sz
        L.relation_bwd_stored_workspace_bytes.argtypes = [i, i, i, i]
        L.relation_bwd_stored_workspace_bytes.restype = sz
        L.relation_bwd.argtypes = [vp, vp, vp, fp, f, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.relation_bwd.restype = i
        L.relation_prestep.argtypes = [vp, vp, vp, vp, i, f, fp, i, vp, vp, vp, i, i, i, i, i, vp]
        L.relation_prestep.restype = i
        L.relation_fwd_model_workspace_bytes.argtypes = [i, i, i, i, i]
        L.relation_fwd_model_workspace_bytes.restype = sz
        L.relation_fwd_model.argtypes = [vp, vp, vp, vp, i, f, fp, i, fp, f, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.relation_fwd_model.restype = i
        L.relation_linear_workspace_bytes.argtypes = [i, i, i, i]
        L.relation_linear_workspace_bytes.restype = sz
        L.relation_linear_fwd.argtypes = [vp, vp, vp, vp, fp, vp, vp, i, i, i, i, i, vp, sz, vp]
        L.relation_linear_fwd.restype = i
        L.relation_decode_workspace_bytes.argtypes = [i, i, i, i]
        L.relation_decode_workspace_bytes.restype = sz
        L.relation_decode.argtypes = [vp, vp, vp, vp, vp, vp, fp, f, vp, i, i, i, i, i, vp, sz, vp]
        L.relation_decode.restype = i
        L.relation_decode_noalloc.argtypes = [vp, vp, vp, vp, vp, vp, fp, f, vp, i, i, i, i, i, vp]
        L.relation_decode_noalloc.restype = i
        L.relation_cache_append.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, vp]
        L.relation_cache_append.restype = i
        L.relation_status_str.argtypes = [i]
        L.relation_status_str.restype = ctypes.c_char_p
        L.relation_select_kernels.argtypes = [i, i]
        L.relation_select_kernels.restype = i
        _lib = L
    return _lib


EXPORTS = ("relation_fwd", "relation_fwd_ex", "relation_fwd_lse", "relation_bwd_workspace_bytes",
           "relation_bwd_stored_workspace_bytes", "relation_bwd", "relation_prestep", "relation_fwd_model_workspace_bytes",
           "relation_fwd_model", "relation_linear_workspace_bytes", "relation_linear_fwd",
           "relation_decode_workspace_bytes", "relation_decode", "relation_decode_noalloc",
           "relation_cache_append", "relation_status_str", "relation_select_kernels")

KERNELS = {"auto": 0, "scan": 1}


def select_kernels(fwd: str = "auto", bwd: str = "auto"):
    """Process-wide choice of the bf16 forward / backward kernels: "auto"
    (the MFMA kernels wherever they apply) or "scan" (the row-scan kernels)."""
    _check("relation_select_kernels", lib().relation_select_kernels(KERNELS[fwd], KERNELS[bwd]))


class kernels:
    """Context manager: select kernels for the block, then back to "auto"."""

    def __init__(self, fwd: str = "auto", bwd: str = "auto"):
        self.sel = (fwd or "auto", bwd or "auto")

    def __enter__(self):
        select_kernels(*self.sel)
        return self

    def __exit__(self, *exc):
        select_kernels("auto", "auto")

ROPE = {"none": 0, "interleaved": 1, "half": 2}
PAIRS = {"A": 0, "B": 1}


def _ptr(t) -> int | None:
    return None if t is None else t.data_ptr()


def _stream(stream) -> int | None:
    if stream is None:
        stream = torch.cuda.current_stream()
    return stream.cuda_stream


def _tau_arg(tau, H: int):
    arr = np.ascontiguousarray(np.broadcast_to(np.asarray(tau, dtype=np.float32), (H,)))
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _check(fn: str, st: int):
    if st != 0:
        raise RelationError(fn, st)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype not in _DT:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return _DT[t.dtype]


class _Args:
    """Checks of caller-supplied tensors before anything reaches the library
    (which sees bare pointers and sizes and cannot check them). Every tensor
    is first checked for its shape and dtype (all of them, so a mismatch is
    reported whatever device the tensors are on), then for being a contiguous
    tensor on the device of the first one."""

    def __init__(self, fn: str):
        self.fn = fn
        self.ts = []

    def __call__(self, name, t, shape=None, dtype=None, optional=False):
        if t is None:
            if optional:
                return self
            raise ValueError(f"{self.fn}: {name} is required")
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{self.fn}: {name} must be a torch.Tensor")
        if shape is not None and tuple(t.shape) != tuple(shape):
            raise ValueError(f"{self.fn}: {name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
        if dtype is not None and t.dtype != dtype:
            raise TypeError(f"{self.fn}: {name} has dtype {t.dtype}, expected {dtype}")
        self.ts.append((name, t))
        return self

    def bytes(self, name, t, need: int):
        """A workspace: uint8, at least `need` bytes."""
        self(name, t, dtype=torch.uint8)
        if t.dim() != 1 or t.numel() < need:
            raise ValueError(f"{self.fn}: {name} holds {t.numel()} bytes, {need} needed")
        return self

    def done(self):
        dev = None
        for name, t in self.ts:
            if not t.is_cuda:
                raise ValueError(f"{self.fn}: {name} must be a device tensor")
            if not t.is_contiguous():
                raise ValueError(f"{self.fn}: {name} must be contiguous")
            if dev is None:
                dev = t.device
            elif t.device != dev:
                raise ValueError(f"{self.fn}: {name} is on {t.device}, the inputs on {dev}")


def _shape4(fn, P1):
    if not isinstance(P1, torch.Tensor) or P1.dim() != 4:
        raise ValueError(f"{fn}: P1 must be a [B, H, T, d_h] tensor")
    return tuple(P1.shape)


def fwd(P1, P2, V, tau, lam: float = 0.0, out=None, stream=None):
    """Y = relation forward of [B, H, T, d_h] device tensors; tau: float or [H]."""
    shp = _shape4("fwd", P1)
    B, H, T, D = shp
    a = _Args("fwd")("P1", P1)("P2", P2, shp, P1.dtype)("V", V, shp, P1.dtype)
    a("out", out, shp, P1.dtype, optional=True).done()
    if out is None:
        out = torch.empty_like(V)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_fwd_ex(_ptr(P1), _ptr(P2), _ptr(V), tau_p, float(lam), _ptr(out),
                               B, H, T, D, _dtype_code(P1), _stream(stream))
    del tau_keep
    _check("relation_fwd_ex", st)
    return out


def fwd_lse(P1, P2, V, tau, lam: float = 0.0, out=None, lse=None, stream=None):
    """Training forward: (Y, LSE) with LSE the fp32 [B, H, T] row log normaliser."""
    shp = _shape4("fwd_lse", P1)
    B, H, T, D = shp
    a = _Args("fwd_lse")("P1", P1)("P2", P2, shp, P1.dtype)("V", V, shp, P1.dtype)
    a("out", out, shp, P1.dtype, optional=True)("lse", lse, (B, H, T), torch.float32, optional=True).done()
    if out is None:
        out = torch.empty_like(V)
    if lse is None:
        lse = torch.empty((B, H, T), dtype=torch.float32, device=P1.device)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_fwd_lse(_ptr(P1), _ptr(P2), _ptr(V), tau_p, float(lam), _ptr(out), _ptr(lse),
                                B, H, T, D, _dtype_code(P1), _stream(stream))
    del tau_keep
    _check("relation_fwd_lse", st)
    return out, lse


def bwd_workspace_bytes(B: int, H: int, T: int, d_h: int) -> int:
    return int(lib().relation_bwd_workspace_bytes(B, H, T, d_h))


def bwd_stored_workspace_bytes(B: int, H: int, T: int, d_h: int) -> int:
    return int(lib().relation_bwd_stored_workspace_bytes(B, H, T, d_h))


def bwd(P1, P2, V, tau, lam, Y, lse, dY, grads=None, workspace=None, stream=None, store_du=None):
    """Gradients (dP1, dP2, dV, dtau [H] fp32, dlambda [1] fp32) of sum(Y * dY),
    from the forward's inputs and its outputs Y, LSE (fwd_lse).

    store_du (when no workspace is given): True or None allocates the workspace
    with which the bf16 MFMA path stores dU (where that path exists), False
    the smaller one with which it recomputes the evidence for dP1."""
    shp = _shape4("bwd", P1)
    B, H, T, D = shp
    dt = P1.dtype
    a = _Args("bwd")("P1", P1)("P2", P2, shp, dt)("V", V, shp, dt)("Y", Y, shp, dt)("dY", dY, shp, dt)
    a("lse", lse, (B, H, T), torch.float32)
    if grads is not None:
        if len(grads) != 5:
            raise ValueError("bwd: grads must be (dP1, dP2, dV, dtau, dlam)")
        a("dP1", grads[0], shp, dt)("dP2", grads[1], shp, dt)("dV", grads[2], shp, dt)
        a("dtau", grads[3], (H,), torch.float32)("dlam", grads[4], (1,), torch.float32)
    need = bwd_workspace_bytes(B, H, T, D)
    if workspace is not None:
        a.bytes("workspace", workspace, need)
    elif store_du is not False and dt == torch.bfloat16:
        need = max(need, bwd_stored_workspace_bytes(B, H, T, D))
    a.done()
    if grads is None:
        grads = (torch.empty_like(P1), torch.empty_like(P2), torch.empty_like(V),
                 torch.empty(H, dtype=torch.float32, device=P1.device),
                 torch.empty(1, dtype=torch.float32, device=P1.device))
    dP1, dP2, dV, dtau, dlam = grads
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=P1.device)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_bwd(_ptr(P1), _ptr(P2), _ptr(V), tau_p, float(lam), _ptr(Y), _ptr(lse), _ptr(dY),
                            _ptr(dP1), _ptr(dP2), _ptr(dV), _ptr(dtau), _ptr(dlam), B, H, T, D,
                            _dtype_code(P1), _ptr(workspace), workspace.numel(), _stream(stream))
    del tau_keep
    _check("relation_bwd", st)
    return dP1, dP2, dV, dtau, dlam


def _theta_arg(theta, H: int):
    if theta is None:
        return None, None
    arr = np.ascontiguousarray(np.asarray(theta, dtype=np.float32).reshape(-1))
    if arr.size != H // 2:
        raise ValueError(f"theta needs H/2 = {H // 2} angles")
    return arr, arr.ctypes.data_as(ctypes.POINTER(ctypes.c_float))


def _check_prestep(fn, P1, P2, I, pos0, out):
    shp = _shape4(fn, P1)
    a = _Args(fn)("P1", P1)("P2", P2, shp, P1.dtype)("I", I, shp, P1.dtype)
    a("pos0", pos0, (shp[0],), torch.int32, optional=True)
    if out is not None:
        if len(out) != 3:
            raise ValueError(f"{fn}: out must be (P1o, P2o, Io)")
        a("out[0]", out[0], shp, P1.dtype)("out[1]", out[1], shp, P1.dtype)("out[2]", out[2], shp, P1.dtype)
    a.done()
    return shp


def prestep(P1, P2, I, pos0=None, rope="interleaved", rope_base: float = 1e4, theta=None, pairing="A",
            out=None, stream=None):
    """RoPE on P1/P2 and Givens mixing of I ([B,H,T,d_h] device tensors); pos0:
    device int32[B] or None; theta: H/2 angles or None. out=(P1o, P2o, Io) may
    be the inputs themselves (in place)."""
    B, H, T, D = _check_prestep("prestep", P1, P2, I, pos0, out)
    if out is None:
        out = (torch.empty_like(P1), torch.empty_like(P2), torch.empty_like(I))
    th_keep, th_p = _theta_arg(theta, H)
    st = lib().relation_prestep(_ptr(P1), _ptr(P2), _ptr(I), _ptr(pos0), ROPE[rope], float(rope_base), th_p,
                                PAIRS[pairing], _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), B, H, T, D,
                                _dtype_code(P1), _stream(stream))
    del th_keep
    _check("relation_prestep", st)
    return out


def prestep_launcher(P1, P2, I, pos0, rope, rope_base, theta, pairing, out, stream=None):
    """relation_prestep with its arguments marshalled once: returns a callable
    that launches it again on the same tensors (for timing loops, where a
    short kernel would otherwise wait on the per-call marshalling)."""
    if out is None:
        raise ValueError("prestep_launcher: out is required")
    B, H, T, D = _check_prestep("prestep_launcher", P1, P2, I, pos0, out)
    th_keep, th_p = _theta_arg(theta, H)
    args = (_ptr(P1), _ptr(P2), _ptr(I), _ptr(pos0), ROPE[rope], float(rope_base), th_p, PAIRS[pairing],
            _ptr(out[0]), _ptr(out[1]), _ptr(out[2]), B, H, T, D, _dtype_code(P1), _stream(stream))
    f = lib().relation_prestep

    def launch():
        _check("relation_prestep", f(*args))
        return th_keep

    return launch


def fwd_model(P1, P2, I, tau, lam: float = 0.0, pos0=None, rope="interleaved", rope_base: float = 1e4,
              theta=None, pairing="A", out=None, lse=None, workspace=None, stream=None):
    """The operator on raw projections: pre-steps, then the forward. Returns
    (Y, LSE or None, workspace): the workspace holds the pre-stepped P2 and I
    (second and third slots) and, unless the bf16 MFMA forward rotated P1
    itself, the rotated P1 (first slot)."""
    shp = _shape4("fwd_model", P1)
    B, H, T, D = shp
    a = _Args("fwd_model")("P1", P1)("P2", P2, shp, P1.dtype)("I", I, shp, P1.dtype)
    a("pos0", pos0, (B,), torch.int32, optional=True)("out", out, shp, P1.dtype, optional=True)
    a("lse", lse, (B, H, T), torch.float32, optional=True)
    need = int(lib().relation_fwd_model_workspace_bytes(B, H, T, D, _dtype_code(P1)))
    if workspace is not None:
        a.bytes("workspace", workspace, need)
    a.done()
    if out is None:
        out = torch.empty_like(I)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=P1.device)
    tau_keep, tau_p = _tau_arg(tau, H)
    th_keep, th_p = _theta_arg(theta, H)
    st = lib().relation_fwd_model(_ptr(P1), _ptr(P2), _ptr(I), _ptr(pos0), ROPE[rope], float(rope_base), th_p,
                                  PAIRS[pairing], tau_p, float(lam), _ptr(out), _ptr(lse), B, H, T, D,
                                  _dtype_code(P1), _ptr(workspace), workspace.numel(), _stream(stream))
    del tau_keep, th_keep
    _check("relation_fwd_model", st)
    return out, lse, workspace


def linear_fwd(P1, P2, I, alpha, tau, out=None, state=None, workspace=None, stream=None):
    """Linear Relation forward; alpha fp32 [B,H,T,d_h]; state: optional fp32
    [B,H,d_h,d_h] output for C_T. Returns (Y, state)."""
    shp = _shape4("linear_fwd", P1)
    B, H, T, D = shp
    a = _Args("linear_fwd")("P1", P1)("P2", P2, shp, P1.dtype)("I", I, shp, P1.dtype)
    a("alpha", alpha, shp, torch.float32)("out", out, shp, P1.dtype, optional=True)
    a("state", state, (B, H, D, D), torch.float32, optional=True)
    need = int(lib().relation_linear_workspace_bytes(B, H, T, D))
    if workspace is not None:
        a.bytes("workspace", workspace, need)
    a.done()
    if out is None:
        out = torch.empty_like(I)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=P1.device)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_linear_fwd(_ptr(P1), _ptr(P2), _ptr(I), _ptr(alpha), tau_p, _ptr(out), _ptr(state),
                                   B, H, T, D, _dtype_code(P1), _ptr(workspace), workspace.numel(),
                                   _stream(stream))
    del tau_keep
    _check("relation_linear_fwd", st)
    return out, state


def decode_workspace_bytes(B: int, H: int, L_cap: int, d_h: int) -> int:
    return int(lib().relation_decode_workspace_bytes(B, H, L_cap, d_h))


def decode(p1, p2, v, cache_P2, cache_V, lens, tau, lam: float = 0.0, out=None,
           workspace=None, stream=None):
    """One Relation Cache decode step; p1/p2/v [B,H,d_h], caches [B,H,L_cap,d_h],
    lens int32[B] on the device."""
    if not isinstance(cache_P2, torch.Tensor) or cache_P2.dim() != 4:
        raise ValueError("decode: cache_P2 must be a [B, H, L_cap, d_h] tensor")
    B, H, L_cap, D = cache_P2.shape
    dt = cache_P2.dtype
    a = _Args("decode")("cache_P2", cache_P2)("cache_V", cache_V, cache_P2.shape, dt)
    a("p1", p1, (B, H, D), dt)("p2", p2, (B, H, D), dt)("v", v, (B, H, D), dt)("lens", lens, (B,), torch.int32)
    a("out", out, (B, H, D), dt, optional=True)
    need = decode_workspace_bytes(B, H, L_cap, D)
    if workspace is not None:
        a.bytes("workspace", workspace, need)
    a.done()
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=p1.device)
    if out is None:
        out = torch.empty_like(v)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_decode(_ptr(p1), _ptr(p2), _ptr(v), _ptr(cache_P2), _ptr(cache_V),
                               _ptr(lens), tau_p, float(lam), _ptr(out), B, H, L_cap, D,
                               _dtype_code(p1), _ptr(workspace), workspace.numel(), _stream(stream))
    del tau_keep
    _check("relation_decode", st)
    return out


def decode_noalloc(p1, p2, v, cache_P2, cache_V, lens, tau, lam: float = 0.0, out=None, stream=None):
    """relation_decode_noalloc: decode with the library's scratch array for the
    partial states (no workspace; `out` must be given for a call that may not
    allocate)."""
    if not isinstance(cache_P2, torch.Tensor) or cache_P2.dim() != 4:
        raise ValueError("decode_noalloc: cache_P2 must be a [B, H, L_cap, d_h] tensor")
    B, H, L_cap, D = cache_P2.shape
    dt = cache_P2.dtype
    a = _Args("decode_noalloc")("cache_P2", cache_P2)("cache_V", cache_V, cache_P2.shape, dt)
    a("p1", p1, (B, H, D), dt)("p2", p2, (B, H, D), dt)("v", v, (B, H, D), dt)("lens", lens, (B,), torch.int32)
    a("out", out, (B, H, D), dt, optional=True).done()
    if out is None:
        out = torch.empty_like(v)
    tau_keep, tau_p = _tau_arg(tau, H)
    st = lib().relation_decode_noalloc(_ptr(p1), _ptr(p2), _ptr(v), _ptr(cache_P2), _ptr(cache_V), _ptr(lens),
                                       tau_p, float(lam), _ptr(out), B, H, L_cap, D, _dtype_code(p1),
                                       _stream(stream))
    del tau_keep
    _check("relation_decode_noalloc", st)
    return out


def cache_append(cache_P2, cache_V, lens, p2, v, stream=None):
    """Append the token's p2, v [B,H,d_h] at row lens[b] and increment lens."""
    if not isinstance(cache_P2, torch.Tensor) or cache_P2.dim() != 4:
        raise ValueError("cache_append: cache_P2 must be a [B, H, L_cap, d_h] tensor")
    B, H, L_cap, D = cache_P2.shape
    dt = cache_P2.dtype
    a = _Args("cache_append")("cache_P2", cache_P2)("cache_V", cache_V, cache_P2.shape, dt)
    a("lens", lens, (B,), torch.int32)("p2", p2, (B, H, D), dt)("v", v, (B, H, D), dt).done()
    st = lib().relation_cache_append(_ptr(cache_P2), _ptr(cache_V), _ptr(lens), _ptr(p2), _ptr(v),
                                     B, H, L_cap, D, _dtype_code(p2), _stream(stream))
    _check("relation_cache_append", st)
