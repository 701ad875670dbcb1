"""The Python binding checks every caller-supplied tensor before any call
reaches the library (which takes bare pointers and sizes and cannot check
them): shape and dtype against the inputs, workspace dtype and size, then
device and contiguity. These tests run on the host: each builds CPU tensors of
the right shapes with one argument wrong and expects the binding to raise;
with every shape right, the CPU tensors themselves are rejected."""
import pytest
import torch

from causal_self_exchange_amd import relation as R

B, H, T, D, L = 2, 4, 8, 64, 16
bf, f32 = torch.bfloat16, torch.float32


def z(*shape, dtype=bf):
    return torch.zeros(shape, dtype=dtype)


def x4(dtype=bf):
    return z(B, H, T, D, dtype=dtype)


def ws(n):
    return torch.zeros(n, dtype=torch.uint8)


def grads(**kw):
    g = dict(dP1=x4(), dP2=x4(), dV=x4(), dtau=z(H, dtype=f32), dlam=z(1, dtype=f32))
    g.update(kw)
    return (g["dP1"], g["dP2"], g["dV"], g["dtau"], g["dlam"])


def bwd(**kw):
    a = dict(P1=x4(), P2=x4(), V=x4(), tau=1.0, lam=0.0, Y=x4(), lse=z(B, H, T, dtype=f32), dY=x4())
    a.update(kw)
    return lambda: R.bwd(**a)


def decode(**kw):
    a = dict(p1=z(B, H, D), p2=z(B, H, D), v=z(B, H, D), cache_P2=z(B, H, L, D), cache_V=z(B, H, L, D),
             lens=z(B, dtype=torch.int32), tau=1.0)
    a.update(kw)
    return lambda: R.decode(**a)


def append(**kw):
    a = dict(cache_P2=z(B, H, L, D), cache_V=z(B, H, L, D), lens=z(B, dtype=torch.int32), p2=z(B, H, D),
             v=z(B, H, D))
    a.update(kw)
    return lambda: R.cache_append(**a)


CASES = {
    # forward
    "fwd P1 not 4-d": (lambda: R.fwd(z(B, H, T), x4(), x4(), 1.0), ValueError, "P1 must be"),
    "fwd P2 shape": (lambda: R.fwd(x4(), z(B, H, T + 1, D), x4(), 1.0), ValueError, "P2 has shape"),
    "fwd V dtype": (lambda: R.fwd(x4(), x4(), x4(f32), 1.0), TypeError, "V has dtype"),
    "fwd out shape": (lambda: R.fwd(x4(), x4(), x4(), 1.0, out=z(B, H, T, D + 16)), ValueError, "out has shape"),
    "fwd out dtype": (lambda: R.fwd(x4(), x4(), x4(), 1.0, out=x4(f32)), TypeError, "out has dtype"),
    "fwd host tensors": (lambda: R.fwd(x4(), x4(), x4(), 1.0), ValueError, "device tensor"),
    "fwd_lse lse shape": (lambda: R.fwd_lse(x4(), x4(), x4(), 1.0, lse=z(B, H, T + 1, dtype=f32)), ValueError,
                          "lse has shape"),
    "fwd_lse lse dtype": (lambda: R.fwd_lse(x4(), x4(), x4(), 1.0, lse=z(B, H, T)), TypeError, "lse has dtype"),
    "fwd_lse out shape": (lambda: R.fwd_lse(x4(), x4(), x4(), 1.0, out=z(B, H, T - 1, D)), ValueError,
                          "out has shape"),
    # backward
    "bwd Y shape": (bwd(Y=z(B, H, T, D + 8)), ValueError, "Y has shape"),
    "bwd dY dtype": (bwd(dY=x4(f32)), TypeError, "dY has dtype"),
    "bwd lse shape": (bwd(lse=z(B, H, dtype=f32)), ValueError, "lse has shape"),
    "bwd dP1 shape": (bwd(grads=grads(dP1=z(B, H, T, 32))), ValueError, "dP1 has shape"),
    "bwd dV dtype": (bwd(grads=grads(dV=x4(f32))), TypeError, "dV has dtype"),
    "bwd dtau size": (bwd(grads=grads(dtau=z(H - 1, dtype=f32))), ValueError, "dtau has shape"),
    "bwd dlam dtype": (bwd(grads=grads(dlam=z(1))), TypeError, "dlam has dtype"),
    "bwd grads count": (bwd(grads=grads()[:4]), ValueError, "grads must be"),
    "bwd workspace small": (bwd(workspace=ws(16)), ValueError, "bytes"),
    "bwd workspace dtype": (bwd(workspace=torch.zeros(1 << 24, dtype=f32)), TypeError, "workspace has dtype"),
    "bwd host tensors": (bwd(), ValueError, "device tensor"),
    # pre-steps and the model forward
    "prestep I shape": (lambda: R.prestep(x4(), x4(), z(B, H, T, 32)), ValueError, "I has shape"),
    "prestep pos0 dtype": (lambda: R.prestep(x4(), x4(), x4(), pos0=z(B, dtype=torch.int64)), TypeError,
                           "pos0 has dtype"),
    "prestep pos0 size": (lambda: R.prestep(x4(), x4(), x4(), pos0=z(B + 1, dtype=torch.int32)), ValueError,
                          "pos0 has shape"),
    "prestep out shape": (lambda: R.prestep(x4(), x4(), x4(), out=(x4(), z(B, H, T, 32), x4())), ValueError,
                          r"out\[1\] has shape"),
    "prestep out count": (lambda: R.prestep(x4(), x4(), x4(), out=(x4(), x4())), ValueError, "out must be"),
    "prestep_launcher out": (lambda: R.prestep_launcher(x4(), x4(), x4(), None, "interleaved", 1e4, None, "A",
                                                        None), ValueError, "out is required"),
    "fwd_model out shape": (lambda: R.fwd_model(x4(), x4(), x4(), 1.0, out=z(B, H, T, 32)), ValueError,
                            "out has shape"),
    "fwd_model lse dtype": (lambda: R.fwd_model(x4(), x4(), x4(), 1.0, lse=z(B, H, T)), TypeError,
                            "lse has dtype"),
    "fwd_model workspace": (lambda: R.fwd_model(x4(), x4(), x4(), 1.0, workspace=ws(64)), ValueError, "bytes"),
    "fwd_model host": (lambda: R.fwd_model(x4(), x4(), x4(), 1.0), ValueError, "device tensor"),
    # linear relation
    "linear alpha dtype": (lambda: R.linear_fwd(x4(), x4(), x4(), x4(), 1.0), TypeError, "alpha has dtype"),
    "linear state shape": (lambda: R.linear_fwd(x4(), x4(), x4(), x4(f32), 1.0, state=z(B, H, D, dtype=f32)),
                           ValueError, "state has shape"),
    "linear workspace": (lambda: R.linear_fwd(x4(), x4(), x4(), x4(f32), 1.0, workspace=ws(8)), ValueError,
                         "bytes"),
    # decode and the cache
    "decode p1 shape": (decode(p1=z(B, H, D + 16)), ValueError, "p1 has shape"),
    "decode p2 dtype": (decode(p2=z(B, H, D, dtype=f32)), TypeError, "p2 has dtype"),
    "decode v shape": (decode(v=z(B, H + 1, D)), ValueError, "v has shape"),
    "decode lens dtype": (decode(lens=z(B, dtype=torch.int64)), TypeError, "lens has dtype"),
    "decode lens size": (decode(lens=z(B - 1, dtype=torch.int32)), ValueError, "lens has shape"),
    "decode cache_V shape": (decode(cache_V=z(B, H, L + 1, D)), ValueError, "cache_V has shape"),
    "decode out shape": (decode(out=z(B, H, D - 8)), ValueError, "out has shape"),
    "decode workspace": (decode(workspace=ws(4)), ValueError, "bytes"),
    "decode host": (decode(), ValueError, "device tensor"),
    "decode_noalloc v dtype": (lambda: R.decode_noalloc(z(B, H, D), z(B, H, D), z(B, H, D, dtype=f32),
                                                        z(B, H, L, D), z(B, H, L, D), z(B, dtype=torch.int32), 1.0),
                               TypeError, "v has dtype"),
    "decode_noalloc host": (lambda: R.decode_noalloc(z(B, H, D), z(B, H, D), z(B, H, D), z(B, H, L, D),
                                                     z(B, H, L, D), z(B, dtype=torch.int32), 1.0),
                            ValueError, "device tensor"),
    "append p2 dtype": (append(p2=z(B, H, D, dtype=f32)), TypeError, "p2 has dtype"),
    "append lens size": (append(lens=z(B + 1, dtype=torch.int32)), ValueError, "lens has shape"),
    "append v shape": (append(v=z(B, H, D, 2)), ValueError, "v has shape"),
    "append host": (append(), ValueError, "device tensor"),
}


@pytest.mark.parametrize("case", sorted(CASES))
def test_binding_rejects(case):
    call, exc, match = CASES[case]
    with pytest.raises(exc, match=match):
        call()


@pytest.mark.gpu
def test_binding_rejects_non_contiguous_device_tensors():
    x = torch.zeros(B, H, T, D, dtype=bf, device="cuda")
    out = torch.zeros(B, H, D, T, dtype=bf, device="cuda").transpose(2, 3)   # right shape, not contiguous
    with pytest.raises(ValueError, match="out must be contiguous"):
        R.fwd(x, x, x, 1.0, out=out)
    with pytest.raises(ValueError, match="P2 must be contiguous"):
        R.fwd(x, out, x, 1.0)
