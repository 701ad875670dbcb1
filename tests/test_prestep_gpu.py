"""GPU parity of the model-side pre-steps (RoPE on P1/P2, Givens mixing of the
information heads) and of the forward on raw projections, through the C ABI,
against the fp64 CPU oracle on the same seeded inputs.

Tolerances: a pre-step output is a rotation of two inputs computed in fp32
(cos / sin of an fp64-reduced angle, one fma): its error is a few fp32 ulps
of the row's largest input. fp32: per row ||out - ref||_inf <= 2e-6 * ||in||_inf.
bf16: the fp32 value is rounded to nearest even (8 significant bits, unit
roundoff 2^-8), so per element |out - ref| <= 2^-8 |ref| + 2e-6 ||in||_inf.
The model forward meets the forward's own bars (bf16 max abs 2e-2, fp32
per-row normwise 1e-5).
"""
import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W
from oracle import prestep_oracle as PO
from tests._helpers import assert_parity, f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _inputs(B, H, T, D, dt, seed):
    cfg = W.FwdConfig("p", B, H, T, D, dt, tau=("uniform", 0.5, 2.0))
    inp = W.make_fwd_inputs(cfg, seed)
    rng = np.random.default_rng(seed + 77)
    theta = rng.uniform(-np.pi, np.pi, H // 2).astype(np.float32)
    pos0 = rng.integers(0, 4000, B).astype(np.int32)
    return inp, theta, pos0


def _check_rows(got, ref, inp_rows_max, dt, what):
    assert np.all(np.isfinite(got)), what
    if dt == "f32":
        err = np.max(np.abs(got - ref), axis=-1) / np.maximum(inp_rows_max, 1e-30)
        assert float(np.max(err)) <= 2e-6, (what, float(np.max(err)))
    else:
        bound = 2.0 ** -8 * np.abs(ref) + 2e-6 * inp_rows_max[..., None]
        bad = np.abs(got - ref) > bound
        assert not bad.any(), (what, float(np.max(np.abs(got - ref) - bound)))


CASES = [
    (1, 2, 7, 32, "f32"), (2, 4, 65, 64, "bf16"), (1, 8, 300, 128, "bf16"), (2, 2, 129, 128, "f32"),
    (3, 6, 33, 64, "f32"), (1, 8, 1, 128, "bf16"),
]


@pytest.mark.parametrize("pairing", ["A", "B"])
@pytest.mark.parametrize("mode", ["interleaved", "half", "none"])
@pytest.mark.parametrize("case", CASES, ids=lambda c: "x".join(map(str, c)))
def test_prestep_matches_oracle(case, mode, pairing):
    B, H, T, D, dt = case
    inp, theta, pos0 = _inputs(B, H, T, D, dt, 3 + T)
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    p0 = torch.from_numpy(pos0).to(DEV)
    o1, o2, o3 = R.prestep(P1, P2, I, p0, mode, 1e4, theta, pairing)
    torch.cuda.synchronize()
    r1, r2, r3 = PO.prestep(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), pos0, 1e4, mode,
                            theta.astype(np.float64), pairing)
    for got, ref, src, name in ((o1, r1, inp["P1"], "P1"), (o2, r2, inp["P2"], "P2")):
        _check_rows(f64(got), ref, np.max(np.abs(f64(src)), axis=-1), dt, f"{case} {mode} {name}")
    # I rows mix two heads: bound by the larger of the pair's rows (the max over heads).
    imax = np.max(np.abs(f64(inp["V"])), axis=(1, 3))[:, None, :]
    _check_rows(f64(o3), r3, np.broadcast_to(imax, r3.shape[:3]), dt, f"{case} {pairing} I")


@pytest.mark.parametrize("D", [48, 80, 128])
def test_prestep_far_positions(D):
    """Positions up to 2^31 - 2 (the angle is formed and reduced in fp64):
    fp32 rows, both rotary layouts, head sizes off and on powers of two."""
    B, H, T = 4, 2, 40
    inp, theta, _ = _inputs(B, H, T, D, "f32", 11 + D)
    pos0 = np.array([0, 123456, 16777000, 2 ** 31 - T - 1], dtype=np.int32)
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    p0 = torch.from_numpy(pos0).to(DEV)
    for mode in ("interleaved", "half"):
        o1, o2, _ = R.prestep(P1, P2, I, p0, mode, 1e4, theta, "A")
        torch.cuda.synchronize()
        r1, r2, _ = PO.prestep(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), pos0, 1e4, mode,
                               theta.astype(np.float64), "A")
        for got, ref, src, name in ((o1, r1, inp["P1"], "P1"), (o2, r2, inp["P2"], "P2")):
            _check_rows(f64(got), ref, np.max(np.abs(f64(src)), axis=-1), "f32", f"far D={D} {mode} {name}")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_prestep_in_place_equals_out_of_place(dt):
    inp, theta, pos0 = _inputs(2, 4, 100, 64, dt, 5)
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    p0 = torch.from_numpy(pos0).to(DEV)
    want = R.prestep(P1, P2, I, p0, "half", 1e4, theta, "B")
    a, b, c = P1.clone(), P2.clone(), I.clone()
    R.prestep(a, b, c, p0, "half", 1e4, theta, "B", out=(a, b, c))
    torch.cuda.synchronize()
    for x, y in zip((a, b, c), want):
        assert torch.equal(x, y)


def test_prestep_without_angles_copies_information_and_allows_odd_heads():
    inp, _, _ = _inputs(1, 3, 50, 32, "bf16", 6)
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    _, _, o3 = R.prestep(P1, P2, I, None, "interleaved", 1e4, None, "A")
    torch.cuda.synchronize()
    assert torch.equal(o3, I)


def _fused(D, dt, mode):
    """Whether the bf16 MFMA forward rotates P1 itself (relation_fwd_model):
    interleaved pairs at every head size, half-split pairs when d_h % 32 == 0."""
    return dt == "bf16" and D in (32, 48, 64, 80, 128) and (mode == "interleaved" or D % 32 == 0)


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("mode,pairing", [("interleaved", "A"), ("half", "B")])
@pytest.mark.parametrize("case", [(2, 4, 300, 64, "bf16"), (1, 8, 513, 128, "bf16"), (1, 2, 128, 32, "f32"),
                                  (1, 4, 200, 80, "bf16"), (2, 2, 150, 48, "bf16"), (1, 4, 270, 32, "bf16")],
                         ids=lambda c: "x".join(map(str, c)))
def test_model_forward_matches_oracle(case, mode, pairing, with_lse):
    B, H, T, D, dt = case
    inp, theta, pos0 = _inputs(B, H, T, D, dt, 8 + T)
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    p0 = torch.from_numpy(pos0).to(DEV)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV) if with_lse else None
    Y, L, ws = R.fwd_model(P1, P2, I, inp["tau"], 0.5, p0, mode, 1e4, theta, pairing, lse=lse)
    torch.cuda.synchronize()
    ref = PO.relation_fwd_model(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), inp["tau"].astype(np.float64),
                                0.5, pos0, 1e4, mode, theta.astype(np.float64), pairing)
    assert_parity(f64(Y), ref, W.torch_dtype(dt), f"{case} {mode}")
    # The workspace holds the pre-stepped P2 and I the forward consumed, and
    # P1 too unless the forward rotated it itself as it loaded each query
    # tile. Either way the result is the forward on the pre-stepped tensors,
    # bit for bit (same angles, same fp32 rotation, same bf16 rounding).
    n = B * H * T * D
    es = 2 if dt == "bf16" else 4
    part = ((n * es + 255) // 256) * 256
    tdt = W.torch_dtype(dt)
    pre = [ws[k * part: k * part + n * es].view(tdt).view(B, H, T, D) for k in range(3)]
    want = R.prestep(P1, P2, I, p0, mode, 1e4, theta, pairing)
    if with_lse:
        Y2, L2 = R.fwd_lse(want[0], want[1], want[2], inp["tau"], 0.5)
    else:
        Y2, L2 = R.fwd(want[0], want[1], want[2], inp["tau"], 0.5), None
    torch.cuda.synchronize()
    for k in ((1, 2) if _fused(D, dt, mode) else (0, 1, 2)):
        assert torch.equal(pre[k], want[k])
    assert torch.equal(Y, Y2)
    if with_lse:
        assert torch.equal(L, L2)


@pytest.mark.parametrize("with_lse", [True, False])
@pytest.mark.parametrize("mode", ["interleaved", "half"])
def test_model_forward_redo_with_rotation_fused(mode, with_lse):
    """The fused-rotation forward on rows whose rotated evidence reaches
    U ~ 100 (one 256-row query tile): raw P1 and P2 are the target rows
    rotated back by their positions, so the pre-step restores them. The
    work-group redoes that tile, reloading and rotating its P1 rows again;
    the result must match the oracle and, bit for bit, the forward on the
    pre-stepped tensors."""
    B, H, T, D = 1, 2, 600, 128
    rng = np.random.default_rng(7)
    base = np.sqrt(100.0 / np.sqrt(D))
    pos = np.arange(T)
    w2 = base + 0.4 * rng.standard_normal((B, H, T, D))
    w1 = 0.5 * rng.standard_normal((B, H, T, D))
    w1[:, :, 256:512] = base + 0.4 * rng.standard_normal((B, H, 256, D))
    raw1 = PO.rope(w1, -pos, 1e4, mode)
    raw2 = PO.rope(w2, -pos, 1e4, mode)
    Vr = 0.5 * rng.standard_normal((B, H, T, D))
    inp = {"P1": torch.from_numpy(raw1).to(torch.bfloat16), "P2": torch.from_numpy(raw2).to(torch.bfloat16),
           "V": torch.from_numpy(Vr).to(torch.bfloat16), "tau": np.array([1.0, 0.8], np.float32)}
    theta = np.array([0.3], np.float32)
    pos0 = np.zeros(B, np.int32)
    a, b, _ = PO.prestep(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), pos0, 1e4, mode, theta.astype(np.float64), "A")
    assert float(np.max(a[0, 0, 300] @ b[0, 0, :301].T)) / np.sqrt(D) > 90.0
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    p0 = torch.from_numpy(pos0).to(DEV)
    lse = torch.empty((B, H, T), dtype=torch.float32, device=DEV) if with_lse else None
    Y, L, ws = R.fwd_model(P1, P2, I, inp["tau"], 0.5, p0, mode, 1e4, theta, "A", lse=lse)
    torch.cuda.synchronize()
    ref = PO.relation_fwd_model(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), inp["tau"].astype(np.float64),
                                0.5, pos0, 1e4, mode, theta.astype(np.float64), "A")
    assert_parity(f64(Y), ref, torch.bfloat16, f"redo fused {mode}")
    want = R.prestep(P1, P2, I, p0, mode, 1e4, theta, "A")
    if with_lse:
        Y2, _ = R.fwd_lse(want[0], want[1], want[2], inp["tau"], 0.5)
    else:
        Y2 = R.fwd(want[0], want[1], want[2], inp["tau"], 0.5)
    torch.cuda.synchronize()
    assert torch.equal(Y, Y2)
