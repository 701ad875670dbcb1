"""relation_decode_noalloc (partial states in the library's scratch array, no
workspace) against relation_decode with its own workspace: the same kernels,
so the outputs must be identical, on two calls in a row, the second smaller
than the first (the array keeps the first call's states; the second must not
read them), and again after a call of the other entry point."""
import ctypes

import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _case(B, H, L_cap, D, lens, seed, dt="bf16"):
    """Seeded new-token states and caches: rows below lens[b] random, rows at
    or past it NaN (they must never be read)."""
    cfg = W.DecodeConfig("n", B, H, D, 0, L_cap, L_cap, dtype=dt, tau=0.8)
    inp = W.make_decode_inputs(cfg, seed)
    tdt = W.torch_dtype(dt)
    rng = np.random.default_rng(seed)
    for key in ("cache_P2", "cache_V"):
        c = torch.full((B, H, L_cap, D), float("nan"), dtype=tdt)
        for b, L in enumerate(lens):
            c[b, :, :L] = torch.from_numpy(rng.standard_normal((H, L, D)).astype(np.float32)).to(tdt)
        inp[key] = c
    d = {k: inp[k].to(DEV).contiguous() for k in ("p1", "p2", "v", "cache_P2", "cache_V")}
    d["lens"] = torch.from_numpy(np.asarray(lens, dtype=np.int32)).to(DEV)
    return d, inp["tau"]


def _noalloc(d, tau, lam):
    """Through the C ABI directly (the call takes no workspace)."""
    B, H, L_cap, D = d["cache_P2"].shape
    y = torch.empty_like(d["v"])
    t = np.ascontiguousarray(np.broadcast_to(np.asarray(tau, np.float32), (H,)))
    st = R.lib().relation_decode_noalloc(d["p1"].data_ptr(), d["p2"].data_ptr(), d["v"].data_ptr(),
                                         d["cache_P2"].data_ptr(), d["cache_V"].data_ptr(), d["lens"].data_ptr(),
                                         t.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), float(lam),
                                         y.data_ptr(), B, H, L_cap, D, R.REL_BF16 if y.dtype == torch.bfloat16
                                         else R.REL_F32, torch.cuda.current_stream().cuda_stream)
    assert st == 0, R.lib().relation_status_str(st)
    return y


def _with_workspace(d, tau, lam):
    return R.decode(d["p1"], d["p2"], d["v"], d["cache_P2"], d["cache_V"], d["lens"], tau, lam)


def test_decode_noalloc_matches_decode_twice_then_smaller():
    big = _case(16, 8, 1500, 128, [0, 1, 255, 256, 257, 700, 1499, 1500, 3, 1024, 77, 900, 1200, 64, 511, 1000], 11)
    small = _case(3, 2, 300, 64, [299, 5, 0], 12)
    for lam in (0.0, 0.5):
        y1 = _noalloc(*big, lam)
        r1 = _with_workspace(*big, lam)
        y2 = _noalloc(*small, lam)
        r2 = _with_workspace(*small, lam)
        y3 = _noalloc(*big, lam)
        torch.cuda.synchronize()
        assert torch.equal(y1, r1) and torch.equal(y2, r2) and torch.equal(y3, r1)
        assert torch.isfinite(y1.float()).all() and torch.isfinite(y2.float()).all()


def test_decode_noalloc_binding_and_fp32():
    d, tau = _case(4, 3, 600, 80, [599, 600, 0, 256], 13, dt="f32")
    y = R.decode_noalloc(d["p1"], d["p2"], d["v"], d["cache_P2"], d["cache_V"], d["lens"], tau, 0.25)
    r = _with_workspace(d, tau, 0.25)
    torch.cuda.synchronize()
    assert torch.equal(y, r)


def test_decode_noalloc_rejects_oversize_without_launch():
    # 64 x 64 heads, 8192 cached rows, d_h 128 need 64 MiB of partial states:
    # rejected on the host (fake, never-dereferenced addresses).
    t = np.ones(64, np.float32)
    st = R.lib().relation_decode_noalloc(0x1000000, 0x2000000, 0x3000000, 0x4000000, 0x5000000, 0x6000000,
                                         t.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), 0.0, 0x7000000,
                                         64, 64, 8192, 128, R.REL_BF16, None)
    assert st == 9       # REL_E_WORKSPACE
