"""GPU parity of the Linear Relation forward (chunk-parallel kernels, through
the C ABI) against the fp64 recurrence of the oracle on the same seeded
inputs.

Tolerances: the final state C_T (fp32 output) meets max |C - C*| <= 1e-5 *
max(1, max |C*|) for either input dtype. fp32 inputs run on fp32 MFMA; bf16
inputs take the chunk products on bf16 MFMA with the fp32 factor split into
a bf16 pair (at most 2^-18 relative per product, I being exact), which puts
the state error at 2-3e-6 on these shapes against 2-4e-7 for fp32. Y: fp32 per row ||Y_t - Y*_t||_inf <= 1e-5 * ||Y*_t||_inf
(the forward's bar); bf16 per row ||Y_t - Y*_t||_inf <= 2e-2 * max(1,
||Y*_t||_inf) (the forward's absolute bar, relative once the history makes a
row exceed 1: Y_t = I_t + E_t is not bounded by the inputs here, and bf16
storage alone rounds at 2^-8 relative).
"""
import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W
from oracle import linear_oracle as LO
from tests._helpers import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _run(inp, want_state=True):
    P1, P2, I = (inp[k].to(DEV) for k in ("P1", "P2", "V"))
    A = inp["alpha"].to(DEV)
    B, H, T, D = P1.shape
    st = torch.empty((B, H, D, D), dtype=torch.float32, device=DEV) if want_state else None
    Y, st = R.linear_fwd(P1, P2, I, A, inp["tau"], state=st)
    torch.cuda.synchronize()
    return Y, st


def _check(inp, Y, st, dt, what):
    ref, C = LO.linear_relation_fwd(f64(inp["P1"]), f64(inp["P2"]), f64(inp["V"]), f64(inp["alpha"]),
                                    inp["tau"].astype(np.float64), return_state=True)
    y = f64(Y)
    assert np.all(np.isfinite(y)), what
    num = np.max(np.abs(y - ref), axis=-1)
    mx = np.max(np.abs(ref), axis=-1)
    if dt == "f32":
        err = float(np.max(num / np.maximum(mx, 1e-30)))
        assert err <= 1e-5, (what, err)
    else:
        err = float(np.max(num / np.maximum(1.0, mx)))
        assert err <= 2e-2, (what, err)
    serr = float("nan")
    if st is not None:
        c = f64(st)
        serr = float(np.max(np.abs(c - C)) / max(1.0, float(np.max(np.abs(C)))))
        assert serr <= 1e-5, (what, "state", serr)
    print(f"\n{what}: Y err {err:.2e}, state err {serr:.2e}", flush=True)


SHAPES = [
    (1, 2, 1, 32, "f32"), (1, 2, 63, 64, "bf16"), (2, 3, 130, 64, "f32"), (1, 2, 200, 128, "bf16"),
    (1, 1, 64, 128, "f32"), (1, 2, 300, 32, "bf16"), (1, 1, 129, 128, "f32"),
]


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_linear_matches_oracle(shape):
    B, H, T, D, dt = shape
    cfg = W.FwdConfig("l", B, H, T, D, dt, tau=("uniform", 0.5, 2.0))
    inp = W.make_linear_inputs(cfg, 21 + T)
    Y, st = _run(inp)
    _check(inp, Y, st, dt, str(shape))


def test_linear_without_state_output_and_single_token():
    cfg = W.FwdConfig("l", 2, 2, 1, 64, "bf16")
    inp = W.make_linear_inputs(cfg, 3)
    Y, _ = _run(inp, want_state=False)
    assert torch.equal(Y, inp["V"].to(DEV))          # Y_1 = I_1: no history


def test_linear_edge_retention_values():
    """alpha = 1 everywhere (no forgetting) and alpha = 0 on one token (the
    state is wiped; values outside (0, 1] are clamped to [1e-30, 1])."""
    cfg = W.FwdConfig("l", 1, 2, 150, 64, "f32")
    inp = W.make_linear_inputs(cfg, 4)
    inp["alpha"] = torch.ones_like(inp["alpha"])
    Y, st = _run(inp)
    _check(inp, Y, st, "f32", "alpha=1")
    inp["alpha"][:, :, 77] = 0.0
    Y0, st0 = _run(inp)
    inp["alpha"][:, :, 77] = 1e-30
    _check(inp, Y0, st0, "f32", "alpha=0 at one token")


@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_linear_fast_decay_takes_exact_diagonal_blocks(dt):
    """Retention 1e-3 on a third of the channels (log alpha = -6.9 per token,
    more than e^-40 within 8 tokens): every diagonal 16-row block of those
    chunks leaves the factored path for the exact exponentials, while the
    chunks of the second half keep alpha in [0.5, 1] and stay factored."""
    cfg = W.FwdConfig("l", 1, 2, 256, 64, dt)
    inp = W.make_linear_inputs(cfg, 9)
    a = inp["alpha"].clone()
    a[:, :, :128, ::3] = 1e-3
    a[:, :, 128:] = a[:, :, 128:].clamp(0.5, 1.0)
    inp["alpha"] = a
    Y, st = _run(inp)
    _check(inp, Y, st, dt, f"fast decay {dt}")


def test_linear_deterministic():
    cfg = W.FwdConfig("l", 1, 4, 500, 128, "bf16")
    inp = W.make_linear_inputs(cfg, 5)
    a = _run(inp)
    b = _run(inp)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


@pytest.mark.parametrize("h", [0, 31])
def test_linear_long_shape_full_heads(h):
    """The bench's Linear Relation call (B=1 H=32 T=8192 d_h=128 bf16, seeded
    retention), every output row and the final state of one head against the
    oracle's recurrence."""
    cfg = W.CONFIGS["long"]
    inp = W.make_linear_inputs(cfg, 42)
    Y, st = _run(inp)
    sub = {k: inp[k][:, h:h + 1] for k in ("P1", "P2", "V", "alpha")}
    sub["tau"] = inp["tau"][h:h + 1]
    _check(sub, Y[:, h:h + 1], st[:, h:h + 1], "bf16", f"long h={h}")


# Shapes whose chunk count selects grouped walks (on a 256-CU device: 2, 4, 8
# and 16 chunks per group), with ragged last chunks and last groups shorter
# than the rest. Heads are flattened as b * H + h; the first, a middle and
# the last are checked against the oracle.
GROUP_SHAPES = [
    (1, 100, 350, 32), (1, 64, 1000, 64), (2, 32, 2000, 128), (4, 64, 600, 64),
    (1, 96, 600, 128),      # groups of 4, 4 and 2 chunks per head; 288 groups on 256 work-groups
]


@pytest.mark.parametrize("shape", GROUP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_linear_grouped_chunk_walks(shape):
    B, H, T, D = shape
    cfg = W.FwdConfig("l", B, H, T, D, "bf16")
    inp = W.make_linear_inputs(cfg, 77)
    Y, st = _run(inp)
    for bh in sorted({0, (B * H) // 2 + 1, B * H - 1}):
        b, h = divmod(bh, H)
        sub = {k: inp[k][b:b + 1, h:h + 1] for k in ("P1", "P2", "V", "alpha")}
        sub["tau"] = inp["tau"][h:h + 1]
        _check(sub, Y[b:b + 1, h:h + 1], st[b:b + 1, h:h + 1], "bf16", f"{shape} head {bh}")
