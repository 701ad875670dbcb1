"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle on
the same seeded inputs, plus properties that hold at any size.

Sizes: Tiny and Small are compared in full; Mid and Long (full size, the
launch configuration the benchmark times) are compared on sampled rows of
every head, each row computed by the oracle straight from the definition.
"""

import os

import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W
from oracle import relation_oracle as O
from tests import fp32_bars as FB
from tests._helpers import assert_parity, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _dev(inp):
    return [inp[k].to(DEV).contiguous() for k in ("P1", "P2", "V")]


def _gpu_fwd(inp, lam=0.0):
    P1, P2, V = _dev(inp)
    Y = R.fwd(P1, P2, V, inp["tau"], lam)
    torch.cuda.synchronize()
    return Y


def _oracle_full(inp, lam=0.0):
    return O.relation_fwd(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]),
                          inp["tau"].astype(np.float64), lam)


def _sample_rows(T, rng, n=40):
    fixed = [0, 1, 2, 15, 16, 31, 32, 63, 64, 65, 127, 128, 129, 255, 256, T - 2, T - 1]
    rows = set(r for r in fixed if 0 <= r < T)
    rows.update(int(x) for x in rng.integers(0, T, n))
    return sorted(rows)


def _oracle_sampled_compare(inp, Y, lam, seed, dtype, n=40):
    P1, P2, V = f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"])
    Yg = f64(Y)
    B, H, T, _ = P1.shape
    rng = np.random.default_rng(seed + 1000)
    worst = 0.0
    for b in range(B):
        for h in range(H):
            rows = _sample_rows(T, rng, n)
            ref = O.relation_rows(P1[b, h], P2[b, h], V[b, h], float(inp["tau"][h]), lam, rows)
            worst = max(worst, assert_parity(Yg[b, h, rows], ref, dtype, f"b={b} h={h}"))
    return worst


def _kernel_env(name):
    return R.kernels(fwd=name or "auto")


# ------------------------------------------------------------ configs -----

@pytest.mark.parametrize("seed", W.SEEDS)
@pytest.mark.parametrize("name", ["tiny", "small"])
def test_config_full_parity(name, seed):
    cfg = W.CONFIGS[name]
    inp = W.make_fwd_inputs(cfg, seed)
    Y = _gpu_fwd(inp)
    assert_parity(f64(Y), _oracle_full(inp), W.torch_dtype(cfg.dtype), f"{name} seed {seed}")


@pytest.mark.parametrize("seed", W.SEEDS)
def test_mid_config_sampled_parity(seed):
    cfg = W.CONFIGS["mid"]
    inp = W.make_fwd_inputs(cfg, seed)
    Y = _gpu_fwd(inp)
    _oracle_sampled_compare(inp, Y, 0.0, seed, torch.bfloat16, n=24)


@pytest.mark.parametrize("seed", W.SEEDS)
def test_long_config_sampled_parity(seed):
    cfg = W.CONFIGS["long"]
    inp = W.make_fwd_inputs(cfg, seed)
    Y = _gpu_fwd(inp)
    _oracle_sampled_compare(inp, Y, 0.0, seed, torch.bfloat16, n=24)


def _oracle_heads(inp, heads, lam=0.0):
    """The fp64 oracle on the listed (b, h) heads, one head per thread (numpy
    releases the interpreter lock in its BLAS and elementwise loops; BLAS is
    held to one thread per head)."""
    from concurrent.futures import ThreadPoolExecutor

    from threadpoolctl import threadpool_limits
    P1, P2, V = f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"])
    tau = inp["tau"].astype(np.float64)

    def one(bh):
        b, h = bh
        return O.relation_head(P1[b, h], P2[b, h], V[b, h], float(tau[h]), lam)

    n = max(1, min(len(os.sched_getaffinity(0)), len(heads), 16))
    with threadpool_limits(limits=1), ThreadPoolExecutor(n) as ex:
        return list(ex.map(one, heads))


def test_mid_config_full_parity():
    """Every element of every head of the mid workload (one seed)."""
    cfg = W.CONFIGS["mid"]
    inp = W.make_fwd_inputs(cfg, W.SEEDS[0])
    Y = f64(_gpu_fwd(inp))
    heads = [(b, h) for b in range(cfg.B) for h in range(cfg.H)]
    for (b, h), ref in zip(heads, _oracle_heads(inp, heads)):
        assert_parity(Y[b, h], ref, torch.bfloat16, f"mid b={b} h={h}")


@pytest.mark.parametrize("group", range(4))
def test_long_config_full_parity(group):
    """Every element of every head of the long workload (one seed), in four
    groups of eight heads (the launch is the whole workload each time)."""
    cfg = W.CONFIGS["long"]
    inp = W.make_fwd_inputs(cfg, W.SEEDS[0])
    Y = f64(_gpu_fwd(inp))
    heads = [(0, h) for h in range(8 * group, 8 * group + 8)]
    for (b, h), ref in zip(heads, _oracle_heads(inp, heads)):
        assert_parity(Y[b, h], ref, torch.bfloat16, f"long h={h}")


def test_relation_fwd_entry_point_small():
    """relation_fwd itself (not only relation_fwd_ex) on the small workload."""
    import ctypes
    cfg = W.CONFIGS["small"]
    inp = W.make_fwd_inputs(cfg, W.SEEDS[0])
    P1, P2, V = _dev(inp)
    Y = torch.empty_like(V)
    tau = np.ascontiguousarray(np.broadcast_to(np.asarray(inp["tau"], np.float32), (cfg.H,)))
    st = R.lib().relation_fwd(P1.data_ptr(), P2.data_ptr(), V.data_ptr(),
                              tau.ctypes.data_as(ctypes.POINTER(ctypes.c_float)), Y.data_ptr(),
                              cfg.B, cfg.H, cfg.T, cfg.d_h, R.REL_BF16, torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == 0
    assert_parity(f64(Y), _oracle_full(inp, 0.0), torch.bfloat16, "relation_fwd small")
    assert torch.equal(Y, _gpu_fwd(inp, 0.0))          # relation_fwd_ex with lambda = 0


def test_scan_kernel_bf16_mid_sampled():
    """The row-scan kernel, forced for bf16, meets the same bar."""
    cfg = W.CONFIGS["mid"]
    inp = W.make_fwd_inputs(cfg, 42)
    with _kernel_env("scan"):
        Y = _gpu_fwd(inp)
    _oracle_sampled_compare(inp, Y, 0.0, 42, torch.bfloat16, n=12)


# ------------------------------------------------------- ragged shapes ----

SHAPES = [
    (1, 1, 1, 32, "f32"), (1, 1, 2, 64, "bf16"), (1, 1, 1, 128, "bf16"),
    (2, 3, 100, 64, "bf16"), (1, 2, 129, 128, "bf16"), (1, 1, 1000, 128, "bf16"),
    (2, 2, 257, 32, "bf16"), (1, 2, 333, 128, "f32"), (1, 1, 64, 64, "f32"),
    (3, 1, 191, 64, "bf16"), (1, 1, 513, 128, "bf16"), (1, 2, 77, 32, "f32"),
    (1, 3, 700, 32, "bf16"), (1, 1, 1, 32, "bf16"),
]


@pytest.mark.parametrize("lam", [0.0, 0.5])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_ragged_shapes(shape, lam):
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0), lam=lam)
    inp = W.make_fwd_inputs(cfg, 7 + T)
    Y = _gpu_fwd(inp, lam)
    assert_parity(f64(Y), _oracle_full(inp, lam), W.torch_dtype(dt), str(shape))


@pytest.mark.parametrize("kernel", [None, "scan"])
@pytest.mark.parametrize("D", [32, 64, 128])
def test_large_evidence_regime(D, kernel):
    """U_ij ~ 30: the running maximum moves and every Exchange weight is huge
    relative to Self; stresses the rescaling path."""
    rng = np.random.default_rng(D)
    T = 300
    base = np.float32(np.sqrt(30.0 / np.sqrt(D)))
    P1 = (base + 0.4 * rng.standard_normal((1, 2, T, D))).astype(np.float32)
    P2 = (base + 0.4 * rng.standard_normal((1, 2, T, D))).astype(np.float32)
    V = rng.standard_normal((1, 2, T, D)).astype(np.float32)
    for dt in (torch.float32, torch.bfloat16):
        inp = dict(P1=torch.from_numpy(P1).to(dt), P2=torch.from_numpy(P2).to(dt),
                   V=torch.from_numpy(V).to(dt), tau=np.array([1.0, 0.5], np.float32))
        with _kernel_env(kernel):
            Y = _gpu_fwd(inp, 0.5)
        ref = _oracle_full(inp, 0.5)
        if dt == torch.float32:
            # fp32 rounding of U_ij grows linearly with |U| and enters Y through
            # the weights, so the fixed 1e-5 bar does not apply at |U| ~ 45:
            # the first-order rounding-error bound of tests/fp32_bars.py does.
            bar = FB.fwd_bar(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]),
                             inp["tau"].astype(np.float64), 0.5)
            ratio = FB.excess(f64(Y), ref, bar)
            print(f"\nD={D} fp32 large evidence: error/bar {ratio:.2e}", flush=True)
            assert ratio <= 1.0, f"D={D}: fp32 error exceeds its derived bar ({ratio:.2f}x)"
        else:
            assert_parity(f64(Y), ref, dt, f"D={D} {dt}")



@pytest.mark.parametrize("with_lse", [False, True])
@pytest.mark.parametrize("D", [64, 128])
def test_overflowing_evidence_takes_the_redo_pass(D, with_lse):
    """U ~ 100 on the rows of one 256-row query tile: with the fixed offset
    m = 0 their weights would reach 2^144, past the 2^100 row-sum bound, so
    the work-group redoes that tile with each row's evidence maximum as the
    offset; the other tiles (|U| ~ 1.5) stay on the fixed-offset path. bf16
    MFMA kernel; Y (and LSE) against the oracle everywhere."""
    T, H = 700, 2
    rng = np.random.default_rng(100 + D)
    base = np.float32(np.sqrt(100.0 / np.sqrt(D)))
    P2 = (base + 0.4 * rng.standard_normal((1, H, T, D))).astype(np.float32)
    P1 = (0.5 * rng.standard_normal((1, H, T, D))).astype(np.float32)
    P1[:, :, 256:512] = base + 0.4 * rng.standard_normal((1, H, 256, D))
    V = (0.5 * rng.standard_normal((1, H, T, D))).astype(np.float32)
    inp = dict(P1=torch.from_numpy(P1).to(torch.bfloat16), P2=torch.from_numpy(P2).to(torch.bfloat16),
               V=torch.from_numpy(V).to(torch.bfloat16), tau=np.array([1.0, 0.7], np.float32))
    ref = _oracle_full(inp, 0.5)
    U = O.evidence(f64(inp["P1"])[0, 0], f64(inp["P2"])[0, 0])
    assert float(np.max(U[300])) > 90.0 and float(np.max(np.abs(U[100, :100]))) < 10.0
    P1d, P2d, Vd = _dev(inp)
    if with_lse:
        Y, L = R.fwd_lse(P1d, P2d, Vd, inp["tau"], 0.5)
        torch.cuda.synchronize()
        want = np.stack([O.row_lse(f64(inp["P1"])[0, h], f64(inp["P2"])[0, h], float(inp["tau"][h]), 0.5)
                         for h in range(H)])
        assert float(np.max(np.abs(f64(L)[0] - want))) <= 1e-4
    else:
        Y = R.fwd(P1d, P2d, Vd, inp["tau"], 0.5)
        torch.cuda.synchronize()
    assert_parity(f64(Y), ref, torch.bfloat16, f"redo D={D} lse={with_lse}")

def test_zero_evidence_rows():
    """P2 = 0: S = 1/2, E = 0; the oracle's closed form holds on the GPU too."""
    for dt in (torch.float32, torch.bfloat16):
        rng = np.random.default_rng(3)
        P1 = torch.from_numpy(rng.standard_normal((2, 2, 200, 64)).astype(np.float32)).to(dt)
        V = torch.from_numpy(rng.standard_normal((2, 2, 200, 64)).astype(np.float32)).to(dt)
        inp = dict(P1=P1, P2=torch.zeros_like(P1), V=V, tau=np.array([1.0, 2.0], np.float32))
        Y = _gpu_fwd(inp, 0.5)
        assert_parity(f64(Y), _oracle_full(inp, 0.5), dt, str(dt))


# --------------------------------------------------------- properties ----

@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_first_row_is_v1_bitwise(dt):
    cfg = W.FwdConfig("t", 2, 4, 300, 128, "f32" if dt == torch.float32 else "bf16",
                      tau=("uniform", 0.5, 2.0))
    inp = W.make_fwd_inputs(cfg, 11)
    Y = _gpu_fwd(inp, 0.7)
    assert torch.equal(Y[:, :, 0].cpu(), inp["V"][:, :, 0])


@pytest.mark.parametrize("dt,D", [(torch.bfloat16, 128), (torch.bfloat16, 64), (torch.float32, 64)])
def test_identity_information_gives_the_flow(dt, D):
    """V = I_T (T = d_h) makes Y = F: rows sum to 1, strict upper triangle is 0."""
    T = D
    rng = np.random.default_rng(5)
    P1 = torch.from_numpy(rng.standard_normal((1, 1, T, D)).astype(np.float32)).to(dt)
    P2 = torch.from_numpy(rng.standard_normal((1, 1, T, D)).astype(np.float32)).to(dt)
    V = torch.eye(T, dtype=dt).reshape(1, 1, T, D)
    inp = dict(P1=P1, P2=P2, V=V, tau=np.array([1.0], np.float32))
    Y = f64(_gpu_fwd(inp))[0, 0]
    _, F = O.relation_head(f64(P1)[0, 0], f64(P2)[0, 0], np.eye(T), 1.0, 0.0, return_flow=True)
    tol = 1e-5 if dt == torch.float32 else 2e-2
    np.testing.assert_allclose(Y, F, rtol=0, atol=tol)
    np.testing.assert_allclose(Y.sum(axis=1), 1.0, rtol=0, atol=tol * 4)
    assert np.all(Y[np.triu_indices(T, k=1)] == 0.0)


@pytest.mark.parametrize("dt", [torch.float32, torch.bfloat16])
def test_causality_bitwise(dt):
    cfg = W.FwdConfig("t", 1, 3, 700, 128, "f32" if dt == torch.float32 else "bf16")
    inp = W.make_fwd_inputs(cfg, 21)
    Y0 = _gpu_fwd(inp).cpu()
    cut = 301
    pert = dict(inp)
    for k in ("P1", "P2", "V"):
        t = inp[k].clone()
        t[:, :, cut + 1:] = -t[:, :, cut + 1:] * 3
        pert[k] = t
    Y1 = _gpu_fwd(pert).cpu()
    assert torch.equal(Y0[:, :, :cut + 1], Y1[:, :, :cut + 1])
    assert not torch.equal(Y0[:, :, cut + 1:], Y1[:, :, cut + 1:])


def test_deterministic_and_guard_bands():
    cfg = W.CONFIGS["small"]
    inp = W.make_fwd_inputs(cfg, 42)
    P1, P2, V = _dev(inp)
    n = V.numel()
    buf = torch.full((n + 4096,), float("nan"), dtype=V.dtype, device=DEV)
    out = buf[2048:2048 + n].view(V.shape)
    R.fwd(P1, P2, V, inp["tau"], out=out)
    Y2 = R.fwd(P1, P2, V, inp["tau"])
    torch.cuda.synchronize()
    assert torch.equal(out, Y2)
    assert torch.isnan(buf[:2048]).all() and torch.isnan(buf[2048 + n:]).all()


# ------------------------------------------------------------- decode -----

def _gpu_decode(inp, lam=0.0):
    d = {k: inp[k].to(DEV).contiguous() for k in ("p1", "p2", "v", "cache_P2", "cache_V")}
    lens = torch.from_numpy(np.asarray(inp["lens"], dtype=np.int32)).to(DEV)
    y = R.decode(d["p1"], d["p2"], d["v"], d["cache_P2"], d["cache_V"], lens, inp["tau"], lam)
    torch.cuda.synchronize()
    return y


def _oracle_decode(inp, lam=0.0, lens=None):
    return O.relation_decode(f64(inp["p1"]), f64(inp["p2"]), f64(inp["v"]), f64(inp["cache_P2"]),
                             f64(inp["cache_V"]), inp["lens"] if lens is None else lens,
                             inp["tau"].astype(np.float64), lam)


def test_decode_full_config_parity():
    cfg = W.DECODE_CONFIG
    inp = W.make_decode_inputs(cfg, 42)
    y = _gpu_decode(inp)
    assert_parity(f64(y), _oracle_decode(inp), torch.bfloat16, "decode")


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [32, 48, 64, 80, 128])
def test_decode_ragged_lengths(D, dt):
    cfg = W.DecodeConfig("d", 7, 3, D, 0, 600, 600, dtype=dt, tau=0.8)
    inp = W.make_decode_inputs(cfg, 3 + D)
    inp["lens"] = np.array([0, 1, 255, 256, 257, 599, 600], dtype=np.int32)
    inp["cache_P2"][:] = float("nan")
    inp["cache_V"][:] = float("nan")
    rng = np.random.default_rng(D)
    tdt = W.torch_dtype(dt)
    for b, L in enumerate(inp["lens"]):
        inp["cache_P2"][b, :, :L] = torch.from_numpy(rng.standard_normal((3, L, D)).astype(np.float32)).to(tdt)
        inp["cache_V"][b, :, :L] = torch.from_numpy(rng.standard_normal((3, L, D)).astype(np.float32)).to(tdt)
    for lam in (0.0, 0.5):
        y = _gpu_decode(inp, lam)
        assert_parity(f64(y), _oracle_decode(inp, lam), tdt, f"lam={lam}")
        assert torch.equal(y[0].cpu(), inp["v"][0])


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 80, 128])
def test_decode_large_evidence(D, dt):
    """U ~ 30 between the new query and every cached key (correlated rows):
    the split-length partials carry large, different maxima and the merge
    must rescale them exactly; lengths span one to several partial blocks.
    fp32 is held to the derived rounding-error bound, as for the forward."""
    B, H, Lc = 4, 2, 2100
    cfg = W.DecodeConfig("d", B, H, D, 0, Lc, Lc, dtype=dt, tau=0.7)
    inp = W.make_decode_inputs(cfg, 70 + D)
    inp["lens"] = np.array([1, 300, 1029, Lc], dtype=np.int32)
    rng = np.random.default_rng(D)
    tdt = W.torch_dtype(dt)
    base = np.float32(np.sqrt(30.0 / np.sqrt(D)))
    g = lambda *shape: torch.from_numpy((base + 0.4 * rng.standard_normal(shape)).astype(np.float32)).to(tdt)
    inp["p1"], inp["p2"], inp["cache_P2"] = g(B, H, D), g(B, H, D), g(B, H, Lc, D)
    inp["cache_V"] = torch.from_numpy(rng.standard_normal((B, H, Lc, D)).astype(np.float32)).to(tdt)
    y = _gpu_decode(inp, 0.5)
    ref = _oracle_decode(inp, 0.5)
    if dt == "f32":
        tau = np.broadcast_to(np.asarray(inp["tau"], np.float64), (H,))
        bar = FB.decode_bar(f64(inp["p1"]), f64(inp["p2"]), f64(inp["v"]), f64(inp["cache_P2"]),
                            f64(inp["cache_V"]), inp["lens"], tau, 0.5)
        ratio = FB.excess(f64(y), ref, bar)
        print(f"\nD={D} fp32 decode large evidence: error/bar {ratio:.2e}", flush=True)
        assert ratio <= 1.0, f"D={D}: fp32 error exceeds its derived bar ({ratio:.2f}x)"
    else:
        assert_parity(f64(y), ref, tdt, f"D={D} {dt}")


def test_decode_clamps_out_of_range_lengths():
    """len[b] outside [0, L_cap] is clamped: -5 reads nothing, L_cap + 10 reads
    the whole cache."""
    cfg = W.DecodeConfig("d", 3, 2, 64, 40, 40, 40, tau=1.0)
    inp = W.make_decode_inputs(cfg, 9)
    inp["lens"] = np.array([-5, 50, 17], dtype=np.int32)
    y = _gpu_decode(inp)
    ref = _oracle_decode(inp, lens=np.array([0, 40, 17]))
    assert torch.equal(y[0].cpu(), inp["v"][0])
    assert_parity(f64(y), ref, torch.bfloat16, "clamped")


@pytest.mark.parametrize("D", [48, 64, 80])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_autoregressive_decode_matches_forward(dt, D):
    """Empty cache; for t = 0..T-1 decode token t then append it. Every decode
    output must equal row t of the forward on the whole sequence (exact cache,
    App. A.5), both checked against the oracle."""
    B, H, T = 2, 2, 70
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0))
    inp = W.make_fwd_inputs(cfg, 5)
    P1, P2, V = _dev(inp)
    tdt = W.torch_dtype(dt)
    cP2 = torch.full((B, H, T, D), float("nan"), dtype=tdt, device=DEV)
    cV = torch.full((B, H, T, D), float("nan"), dtype=tdt, device=DEV)
    lens = torch.zeros(B, dtype=torch.int32, device=DEV)
    outs = []
    for t in range(T):
        p1, p2, v = (x[:, :, t].contiguous() for x in (P1, P2, V))
        outs.append(R.decode(p1, p2, v, cP2, cV, lens, inp["tau"], 0.5))
        R.cache_append(cP2, cV, lens, p2, v)
    torch.cuda.synchronize()
    Yd = torch.stack(outs, dim=2)
    assert lens.cpu().tolist() == [T] * B
    assert torch.equal(cP2.cpu(), inp["P2"]) and torch.equal(cV.cpu(), inp["V"])
    ref = _oracle_full(inp, 0.5)
    assert_parity(f64(Yd), ref, tdt, "decode loop")
    R.cache_append(cP2, cV, lens, p2, v)          # full cache: unchanged
    torch.cuda.synchronize()
    assert lens.cpu().tolist() == [T] * B


# ---------------------------- padded head sizes: the paper's 48, 80, and 32 ----

PAPER_SHAPES = [
    (2, 8, 300, 48, "bf16"), (1, 8, 513, 80, "bf16"), (1, 2, 129, 48, "f32"), (1, 2, 100, 80, "f32"),
    (1, 1, 1, 48, "bf16"), (1, 3, 257, 80, "bf16"), (2, 2, 520, 32, "bf16"),
]


@pytest.mark.parametrize("kernel", [None, "scan"])
@pytest.mark.parametrize("lam", [0.0, 0.5])
@pytest.mark.parametrize("shape", PAPER_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_paper_head_sizes(shape, lam, kernel):
    """d_h = 48 and 80 ([paper] Table 6 geometries) and 32: bf16 runs the
    MFMA kernel on the 64 / 128 tile layouts with zero-filled padding chunks;
    the row-scan kernel is checked too. LSE from the training forward as well."""
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0), lam=lam)
    inp = W.make_fwd_inputs(cfg, 31 + T)
    P1, P2, V = _dev(inp)
    with _kernel_env(kernel):
        Y, L = R.fwd_lse(P1, P2, V, inp["tau"], lam)
    torch.cuda.synchronize()
    assert_parity(f64(Y), _oracle_full(inp, lam), W.torch_dtype(dt), f"{shape} {kernel}")
    want = np.stack([np.stack([O.row_lse(f64(inp["P1"])[b, h], f64(inp["P2"])[b, h], float(inp["tau"][h]), lam)
                               for h in range(H)]) for b in range(B)])
    assert float(np.max(np.abs(f64(L) - want))) <= 1e-4



def test_head_size_32_long_sequence_sampled():
    """d_h = 32 on the padded 64-wide MFMA layout at a long sequence (T =
    16,384, two heads, lambda = 0.5): sampled rows of every head, the last
    ones included, against the oracle row by row."""
    cfg = W.FwdConfig("t", 1, 2, 16384, 32, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_fwd_inputs(cfg, 32)
    Y = _gpu_fwd(inp, 0.5)
    _oracle_sampled_compare(inp, Y, 0.5, 32, torch.bfloat16, n=24)

def test_paper_head_size_guard_columns_untouched():
    """Padded columns are never stored: a Y buffer with guard rows after the
    last head keeps its sentinel values."""
    cfg = W.FwdConfig("t", 1, 2, 200, 80, "bf16")
    inp = W.make_fwd_inputs(cfg, 2)
    P1, P2, V = _dev(inp)
    n = P1.numel()
    buf = torch.full((n + 4096,), 7.0, dtype=torch.bfloat16, device=DEV)
    Y = buf[:n].view(P1.shape)
    R.fwd(P1, P2, V, inp["tau"], 0.0, out=Y)
    torch.cuda.synchronize()
    assert torch.all(buf[n:] == 7.0)
    assert_parity(f64(Y), _oracle_full(inp), torch.bfloat16, "guard")
