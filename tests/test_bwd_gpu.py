"""GPU parity of the training forward (Y, LSE) and the backward (dP1, dP2, dV,
dtau, dlambda) through the C ABI against the fp64 CPU oracle on the same
seeded inputs (the oracle's gradients are pinned separately, on the CPU).

Tolerances (the pages fix none for gradients; these follow the forward's bar):
  tensors, per row i of each gradient g:
      ||g_i - g*_i||_inf <= tol * max(1, ||g*_i||_inf)
    tol = 2e-2 for bf16 (the forward's absolute bar, relative once a row's
    gradient exceeds 1 -- the bf16 output rounding alone is up to 2^-8 relative),
    tol = 1e-5 for fp32.
  scalars: each row's share of dtau / dlambda is formed from F_ii, dY_i . V_i
    and D_i = dY_i . Y_i, so the bar is tol times the sum over rows of
      |d R_ii / d theta| * F_ii * sum_d |dY_id| (|V_id| + |Y_id|)
    (theta = tau: S_i (1 - S_i) |U_ii| / tau^2; theta = lambda: log i), the
    size of the quantities each share is computed from.
  LSE: absolute 1e-4 (fp32 exponent sums over up to T terms; |LSE| ~ log T).
"""
import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W
from oracle import relation_oracle as O
from tests import fp32_bars as FB
from tests._helpers import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"
TOL = {"bf16": 2e-2, "f32": 1e-5}
LSE_ATOL = 1e-4


def _dev(inp, keys=("P1", "P2", "V", "dY")):
    return [inp[k].to(DEV).contiguous() for k in keys]


def _gpu_train(inp, lam, bwd_kernel=None, store_du=None):
    P1, P2, V, dY = _dev(inp)
    with R.kernels(bwd=bwd_kernel or "auto"):
        Y, L = R.fwd_lse(P1, P2, V, inp["tau"], lam)
        g = R.bwd(P1, P2, V, inp["tau"], lam, Y, L, dY, store_du=store_du)
    torch.cuda.synchronize()
    return Y, L, g


def row_err(g, ref):
    """max_i ||g_i - ref_i||_inf / max(1, ||ref_i||_inf) over the last axis."""
    num = np.max(np.abs(g - ref), axis=-1)
    den = np.maximum(1.0, np.max(np.abs(ref), axis=-1))
    return float(np.max(num / den))


def _oracle(inp, lam):
    P1, P2, V, dY = (f64(inp[k]) for k in ("P1", "P2", "V", "dY"))
    tau = inp["tau"].astype(np.float64)
    B, H, T, D = P1.shape
    out = dict(dP1=np.empty(P1.shape), dP2=np.empty(P1.shape), dV=np.empty(P1.shape),
               dtau=np.zeros(H), dlam=0.0, lse=np.empty((B, H, T)),
               tau_scale=np.zeros(H), lam_scale=0.0, dlam_diag=0.0)
    log_i = np.log(np.arange(1, T + 1, dtype=np.float64))
    for b in range(B):
        for h in range(H):
            *g, t = O.relation_head_bwd(P1[b, h], P2[b, h], V[b, h], tau[h], lam, dY[b, h], return_terms=True)
            out["dP1"][b, h], out["dP2"][b, h], out["dV"][b, h] = g[0], g[1], g[2]
            out["dtau"][h] += g[3]
            out["dlam"] += g[4]
            out["lse"][b, h] = O.row_lse(P1[b, h], P2[b, h], tau[h], lam)
            Y = O.relation_head(P1[b, h], P2[b, h], V[b, h], tau[h], lam)
            size = t["F_self"] * np.sum(np.abs(dY[b, h]) * (np.abs(V[b, h]) + np.abs(Y)), axis=1)
            out["tau_scale"][h] += np.sum(size * t["S"] * (1 - t["S"]) * np.abs(t["U_self"]) / tau[h] ** 2)
            out["lam_scale"] += np.sum(size * log_i)
            out["dlam_diag"] += float(np.sum(log_i * t["dR_self"]))
    return out


def _check(inp, lam, dt, Y, L, g, what, tol=None, bars=None):
    """bars (elementwise absolute bounds, tests/fp32_bars.py) replace the
    row-relative tol where given."""
    ref = _oracle(inp, lam)
    tol = TOL[dt] if tol is None else tol
    if bars is not None:
        return _check_bars(ref, L, g, what, bars)
    errs = {}
    lse_err = float(np.max(np.abs(f64(L) - ref["lse"])))
    errs["lse"] = lse_err
    for name, got in zip(("dP1", "dP2", "dV"), g[:3]):
        x = f64(got)
        assert np.all(np.isfinite(x)), f"{what}: non-finite {name}"
        errs[name] = row_err(x, ref[name])
    dtau = f64(g[3])
    dlam = float(f64(g[4])[0])
    errs["dtau"] = float(np.max(np.abs(dtau - ref["dtau"]) / (ref["tau_scale"] + 1e-30)))
    errs["dlam"] = abs(dlam - ref["dlam"]) / (ref["lam_scale"] + 1e-30)
    print(f"\n{what}: " + " ".join(f"{k}={v:.2e}" for k, v in errs.items()), flush=True)
    assert lse_err <= LSE_ATOL, f"{what}: LSE error {lse_err:.3e}"
    for name in ("dP1", "dP2", "dV"):
        assert errs[name] <= tol, f"{what}: {name} row error {errs[name]:.3e} > {tol}"
    assert np.all(np.abs(dtau - ref["dtau"]) <= tol * ref["tau_scale"] + 1e-6), (what, dtau, ref["dtau"])
    assert abs(dlam - ref["dlam"]) <= tol * ref["lam_scale"] + 1e-6, (what, dlam, ref["dlam"])
    return errs


def _check_bars(ref, L, g, what, bars):
    lse_err = float(np.max(np.abs(f64(L) - ref["lse"])))
    assert lse_err <= LSE_ATOL, f"{what}: LSE error {lse_err:.3e}"
    ratios = {}
    for name, got in zip(("dP1", "dP2", "dV"), g[:3]):
        x = f64(got)
        assert np.all(np.isfinite(x)), f"{what}: non-finite {name}"
        ratios[name] = FB.excess(x, ref[name], bars[name])
    ratios["dtau"] = FB.excess(f64(g[3]), ref["dtau"], bars["dtau"])
    # dlambda against the diagonal form sum_i log i dR_ii of the oracle's dR:
    # equal to its off-diagonal sum in exact arithmetic (rows of dR sum to
    # zero), but free of that sum's fp64 cancellation error (~1e-16 per unit
    # of sum_j |dR_ij|), which reaches the fp32 bound when F_ii ~ 1e-15
    ratios["dlam"] = FB.excess(float(f64(g[4])[0]), ref["dlam_diag"], bars["dlam"])
    print(f"\n{what}: lse={lse_err:.2e} error/bar " + " ".join(f"{k}={v:.2e}" for k, v in ratios.items()),
          flush=True)
    for name, r in ratios.items():
        assert r <= 1.0, f"{what}: {name} error exceeds its derived fp32 bar ({r:.2f}x)"
    return ratios


SHAPES = [
    # B, H, T, d_h, dtype  (bf16: MFMA kernels; fp32: row-scan kernels)
    (1, 1, 1, 64, "bf16"), (1, 2, 2, 128, "bf16"), (1, 1, 65, 128, "bf16"), (2, 3, 100, 64, "bf16"),
    (1, 2, 129, 128, "bf16"), (3, 1, 191, 64, "bf16"), (1, 2, 300, 128, "bf16"), (1, 1, 513, 128, "bf16"),
    (2, 2, 100, 32, "bf16"), (1, 2, 77, 32, "f32"), (1, 1, 64, 64, "f32"), (1, 1, 150, 128, "f32"),
    (1, 1, 1, 32, "f32"), (1, 3, 333, 32, "bf16"), (1, 1, 1, 32, "bf16"),
    # the paper's head sizes: MFMA kernels on the 64 / 128 layouts (bf16), row-scan kernels (fp32)
    (2, 4, 300, 48, "bf16"), (1, 2, 257, 80, "bf16"), (1, 1, 1, 48, "bf16"), (1, 2, 130, 48, "f32"),
    (1, 1, 99, 80, "f32"),
]


@pytest.mark.parametrize("lam", [0.0, 0.5])
@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_ragged_shapes(shape, lam):
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0), lam=lam)
    inp = W.make_bwd_inputs(cfg, 11 + T)
    Y, L, g = _gpu_train(inp, lam)
    _check(inp, lam, dt, Y, L, g, f"{shape} lam={lam}")


MFMA_SHAPES = [s for s in SHAPES if s[4] == "bf16" and s[3] in (32, 48, 64, 80, 128)]


@pytest.mark.parametrize("shape", MFMA_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_bwd_recompute_path(shape):
    """The bf16 MFMA backward with the small workspace: the query pass
    recomputes the evidence and weights instead of reading the stored dU."""
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 11 + T)
    Y, L, g = _gpu_train(inp, 0.5, store_du=False)
    _check(inp, 0.5, dt, Y, L, g, f"recompute {shape}")


def test_bwd_stored_path_uses_the_stored_workspace():
    """With the larger workspace the stored-dU path runs and writes dU
    blocks there (the recompute path leaves the workspace past the
    statistics untouched)."""
    cfg = W.FwdConfig("t", 1, 2, 200, 64, "bf16", tau=("uniform", 0.5, 2.0))
    inp = W.make_bwd_inputs(cfg, 3)
    P1, P2, V, dY = _dev(inp)
    Y, L = R.fwd_lse(P1, P2, V, inp["tau"], 0.0)
    small = R.bwd_workspace_bytes(1, 2, 200, 64)
    big = R.bwd_stored_workspace_bytes(1, 2, 200, 64)
    assert big > small
    for ws_bytes, touched in ((big, True), (small, False)):
        ws = torch.full((big,), 0x7F, dtype=torch.uint8, device=DEV)
        R.bwd(P1, P2, V, inp["tau"], 0.0, Y, L, dY, workspace=ws[:ws_bytes])
        torch.cuda.synchronize()
        tail = ws[-(big - small) // 2:]
        assert bool((tail != 0x7F).any()) == touched


def test_bwd_stored_path_at_its_longest_length():
    """T = 46,304, the longest sequence the stored-dU path takes: one head's
    dU blocks end just below 2^31 bytes, so the last query blocks use the
    largest offsets a 32-bit buffer offset holds. Two heads, d_h = 64, bf16,
    lambda = 0.5: dP1 on sampled rows (the last ones included) against the
    oracle row by row, and all three gradient tensors against the recompute
    path, which shares the key/value pass but forms dP1 without stored dU."""
    B, H, T, D = 1, 2, 46304, 64
    assert R.bwd_stored_workspace_bytes(B, H, T, D) > 0
    cfg = W.FwdConfig("t", B, H, T, D, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 46)
    _, _, g = _gpu_train(inp, 0.5, store_du=True)
    _, _, g2 = _gpu_train(inp, 0.5, store_du=False)
    rng = np.random.default_rng(46)
    rows = sorted(set([0, 1, 31, 32, 4095, T - 65, T - 64, T - 33, T - 32, T - 2, T - 1] +
                      [int(x) for x in rng.integers(0, T, 8)]))
    for h in range(H):
        p1, p2, v, dy = (f64(inp[k])[0, h] for k in ("P1", "P2", "V", "dY"))
        ref = O.relation_head_dp1_rows(p1, p2, v, float(inp["tau"][h]), 0.5, dy, rows)
        err = row_err(f64(g[0])[0, h, rows], ref)
        print(f"\nT={T} h={h}: dP1 sampled rows {err:.2e}", flush=True)
        assert err <= TOL["bf16"], (h, err)
    for name, a, b in zip(("dP1", "dP2", "dV"), g[:3], g2[:3]):
        e = row_err(f64(a), f64(b))
        print(f"stored vs recompute {name}: {e:.2e}", flush=True)
        assert e <= TOL["bf16"], (name, e)


def test_bwd_head_size_32_long_sequence():
    """d_h = 32 on the padded 64-wide MFMA layout at T = 16,384 (two heads,
    stored-dU path): dP1 on sampled rows against the oracle row by row, and
    all gradients against the recompute path."""
    B, H, T, D = 1, 2, 16384, 32
    cfg = W.FwdConfig("t", B, H, T, D, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 33)
    _, _, g = _gpu_train(inp, 0.5, store_du=True)
    _, _, g2 = _gpu_train(inp, 0.5, store_du=False)
    rng = np.random.default_rng(33)
    rows = sorted(set([0, 1, 31, 32, 4095, T - 33, T - 32, T - 2, T - 1] + [int(x) for x in rng.integers(0, T, 8)]))
    for h in range(H):
        p1, p2, v, dy = (f64(inp[k])[0, h] for k in ("P1", "P2", "V", "dY"))
        ref = O.relation_head_dp1_rows(p1, p2, v, float(inp["tau"][h]), 0.5, dy, rows)
        err = row_err(f64(g[0])[0, h, rows], ref)
        print(f"\nd_h=32 T={T} h={h}: dP1 sampled rows {err:.2e}", flush=True)
        assert err <= TOL["bf16"], (h, err)
    for name, a, b in zip(("dP1", "dP2", "dV"), g[:3], g2[:3]):
        e = row_err(f64(a), f64(b))
        assert e <= TOL["bf16"], (name, e)


@pytest.mark.parametrize("lam", [-2.0, 4.0])
@pytest.mark.parametrize("shape", [(1, 2, 1500, 128, "bf16"), (1, 2, 700, 64, "f32")], ids=lambda s: "x".join(map(str, s)))
def test_bwd_count_calibration_range(shape, lam):
    """lambda far from its initial 0.5, both signs: -lambda log i then
    outweighs the evidence (4.0) or lifts Exchange above Self (-2.0) over
    most of the sequence. Y, LSE and every gradient against the oracle."""
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("t", B, H, T, D, dt, tau=("uniform", 0.5, 2.0), lam=lam)
    inp = W.make_bwd_inputs(cfg, 17 + T)
    Y, L, g = _gpu_train(inp, lam)
    ref = O.relation_fwd(*(f64(inp[k]) for k in ("P1", "P2", "V")), inp["tau"].astype(np.float64), lam)
    if dt == "bf16":
        assert float(np.max(np.abs(f64(Y) - ref))) <= 2e-2
    else:
        num = np.max(np.abs(f64(Y) - ref), axis=-1)
        assert float(np.max(num / np.max(np.abs(ref), axis=-1))) <= 1e-5
    _check(inp, lam, dt, Y, L, g, f"{shape} lam={lam}")


@pytest.mark.parametrize("name", ["tiny", "small"])
def test_bwd_config_full(name):
    """Tiny (fp32, row-scan kernels) and Small (bf16, MFMA kernels) in full."""
    cfg = W.CONFIGS[name]
    inp = W.make_bwd_inputs(cfg, 42)
    Y, L, g = _gpu_train(inp, 0.0)
    _check(inp, 0.0, cfg.dtype, Y, L, g, name)


@pytest.mark.parametrize("dt", ["bf16", "f32"])
@pytest.mark.parametrize("D", [64, 128])
def test_bwd_large_evidence_regime(D, dt):
    """U_ij ~ 30 (correlated P1 and P2): F concentrates on few keys per row
    and the recomputed F_ij = 2^(SiLU(u) log2 e - L2_i) sits next to the
    exponent's range limits. bf16 runs the MFMA kernels, fp32 the row-scan
    kernels. fp32 rounding of U grows with |U|, so fp32 is held to the
    first-order rounding-error bounds of tests/fp32_bars.py instead of the
    fixed bar."""
    rng = np.random.default_rng(100 + D)
    B, H, T = 1, 2, 300
    base = np.float32(np.sqrt(30.0 / np.sqrt(D)))
    P1 = (base + 0.4 * rng.standard_normal((B, H, T, D))).astype(np.float32)
    P2 = (base + 0.4 * rng.standard_normal((B, H, T, D))).astype(np.float32)
    V = rng.standard_normal((B, H, T, D)).astype(np.float32)
    dY = rng.standard_normal((B, H, T, D)).astype(np.float32)
    tdt = W.torch_dtype(dt)
    inp = dict(P1=torch.from_numpy(P1).to(tdt), P2=torch.from_numpy(P2).to(tdt), V=torch.from_numpy(V).to(tdt),
               dY=torch.from_numpy(dY).to(tdt), tau=np.array([1.0, 0.5], np.float32))
    Y, L, g = _gpu_train(inp, 0.5)
    bars = None
    if dt == "f32":
        bars = FB.bwd_bars(*(f64(inp[k]) for k in ("P1", "P2", "V")), inp["tau"].astype(np.float64),
                           0.5, f64(inp["dY"]))
    _check(inp, 0.5, dt, Y, L, g, f"large evidence D={D} {dt}", bars=bars)


@pytest.mark.parametrize("D", [64, 128])
def test_bwd_scan_kernels_bf16(D):
    """The row-scan backward forced for bf16 meets the same bar."""
    cfg = W.FwdConfig("t", 1, 2, 200, D, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 5)
    Y, L, g = _gpu_train(inp, 0.5, bwd_kernel="scan")
    _check(inp, 0.5, "bf16", Y, L, g, f"scan D={D}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_fwd_lse_output_matches_plain_forward(dt):
    """relation_fwd_lse and relation_fwd_ex compute the same Y. In fp32 both
    run the same arithmetic, bit for bit. In bf16 the training variant forms
    the evidence in fp32 and sums the row from the fp32 weights (its log
    normaliser feeds the backward), while the plain forward scales P1 by
    log2 e / sqrt(d_h) in bf16 and sums the row from the bf16 weights; each
    must meet the bf16 bar against the fp64 oracle, and so the two differ by
    at most twice that bar."""
    cfg = W.FwdConfig("t", 2, 3, 333, 128, dt, tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_fwd_inputs(cfg, 3)
    P1, P2, V = _dev(inp, ("P1", "P2", "V"))
    Y1 = R.fwd(P1, P2, V, inp["tau"], 0.5)
    Y2, _ = R.fwd_lse(P1, P2, V, inp["tau"], 0.5)
    torch.cuda.synchronize()
    if dt == "f32":
        assert torch.equal(Y1, Y2)
        return
    ref = O.relation_fwd(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), inp["tau"], 0.5)
    for Y in (Y1, Y2):
        assert float(np.max(np.abs(f64(Y) - ref))) <= TOL["bf16"]
    assert float((Y1.float() - Y2.float()).abs().max()) <= 2 * TOL["bf16"]


def test_bwd_single_token_passes_dY_to_dV():
    """T = 1: Y_1 = V_1, so dV = dY exactly and every other gradient is 0."""
    cfg = W.FwdConfig("t", 2, 2, 1, 128, "bf16", tau=("uniform", 0.5, 2.0))
    inp = W.make_bwd_inputs(cfg, 9)
    Y, L, (dP1, dP2, dV, dtau, dlam) = _gpu_train(inp, 0.5)
    dY = inp["dY"].to(DEV)
    assert torch.equal(dV, dY)
    assert float(dP1.abs().max()) == 0.0 and float(dP2.abs().max()) == 0.0
    assert float(dtau.abs().max()) == 0.0 and float(dlam.abs().max()) == 0.0


def test_bwd_zero_upstream_gives_zero_gradients():
    cfg = W.FwdConfig("t", 1, 2, 300, 128, "bf16")
    inp = W.make_bwd_inputs(cfg, 2)
    inp["dY"] = torch.zeros_like(inp["dY"])
    _, _, g = _gpu_train(inp, 0.5)
    for x in g:
        assert float(x.abs().max()) == 0.0


def test_bwd_deterministic():
    """Two calls on the same inputs give identical bits (no atomics)."""
    cfg = W.FwdConfig("t", 2, 4, 700, 128, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 4)
    P1, P2, V, dY = _dev(inp)
    Y, L = R.fwd_lse(P1, P2, V, inp["tau"], 0.5)
    g1 = R.bwd(P1, P2, V, inp["tau"], 0.5, Y, L, dY)
    g2 = R.bwd(P1, P2, V, inp["tau"], 0.5, Y, L, dY)
    torch.cuda.synchronize()
    for a, b in zip(g1, g2):
        assert torch.equal(a, b)


def test_bwd_gradients_of_the_future_do_not_reach_the_past():
    """dY zero on rows < k: dP1 is exactly 0 there (row i's query feeds only Y_i)."""
    cfg = W.FwdConfig("t", 1, 2, 400, 64, "bf16")
    inp = W.make_bwd_inputs(cfg, 6)
    inp["dY"][:, :, :150] = 0
    _, _, (dP1, *_rest) = _gpu_train(inp, 0.0)
    assert float(dP1[:, :, :150].abs().max()) == 0.0


def _sample(T, rng, n=24):
    fixed = [0, 1, 2, 31, 32, 63, 64, 255, 256, 257, 4095, 4096, T - 65, T - 64, T - 2, T - 1]
    s = set(r for r in fixed if 0 <= r < T)
    s.update(int(x) for x in rng.integers(0, T, n))
    return sorted(s)


@pytest.mark.parametrize("name,b,h", [("long", 0, 0), ("long", 0, 13), ("long", 0, 31), ("mid", 0, 0),
                                      ("mid", 3, 15)])
def test_bwd_config_sampled(name, b, h):
    """The T = 8192 workload (B=1 H=32 d_h=128, the bench's backward call) and
    the Mid workload (B=4 H=16 T=2048 d_h=64), bf16, on sampled rows of dP1
    and sampled key rows of dV / dP2 of one (b, h), every row's LSE, and (for
    B = 1) the head's dtau, each computed by the oracle from the definition
    row by row / column by column."""
    cfg = W.CONFIGS[name]
    inp = W.make_bwd_inputs(cfg, 42)
    Y, L, g = _gpu_train(inp, 0.0)
    rng = np.random.default_rng(100 + 17 * b + h)
    rows, cols = _sample(cfg.T, rng), _sample(cfg.T, rng)
    p1, p2, v, dy = (f64(inp[k])[b, h] for k in ("P1", "P2", "V", "dY"))
    tau = float(inp["tau"][h])
    ref = O.relation_head_bwd_sampled(p1, p2, v, tau, 0.0, dy, rows, cols)
    assert float(np.max(np.abs(f64(L)[b, h] - ref["lse"]))) <= LSE_ATOL
    errs = {"dP1": row_err(f64(g[0])[b, h, rows], ref["dP1"]),
            "dP2": row_err(f64(g[1])[b, h, cols], ref["dP2"]),
            "dV": row_err(f64(g[2])[b, h, cols], ref["dV"])}
    print(f"\n{name} b={b} h={h}: " + " ".join(f"{k}={e:.2e}" for k, e in errs.items()), flush=True)
    for k, e in errs.items():
        assert e <= TOL["bf16"], (k, e)
    if cfg.B == 1:
        size = ref["F_self"] * np.sum(np.abs(dy) * (np.abs(v) + np.abs(ref["Y"])), axis=1)
        scale = float(np.sum(size * ref["S"] * (1 - ref["S"]) * np.abs(ref["U_self"]) / tau ** 2))
        assert abs(float(f64(g[3])[h]) - ref["dtau"]) <= TOL["bf16"] * scale + 1e-6
