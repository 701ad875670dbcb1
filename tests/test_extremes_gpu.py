"""The largest batch and head counts the boundary accepts (B = 65535;
H = REL_MAX_HEADS = 256), on short sequences: the training forward, the
backward, the Linear Relation and the decode step, each compared with the
oracle on a sample of (b, h) slices that includes the first and the last.
Every kernel indexes heads through b * H + h over the whole grid, so a
mistake in that arithmetic at the largest counts shows in the last slices."""
import numpy as np
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W
from oracle import linear_oracle as LO
from oracle import relation_oracle as O
from tests._helpers import f64

pytestmark = pytest.mark.gpu

DEV = "cuda"


def _slices(B, H, rng, n=6):
    s = {(0, 0), (B - 1, H - 1), (B - 1, 0), (0, H - 1)}
    s.update((int(b), int(h)) for b, h in zip(rng.integers(0, B, n), rng.integers(0, H, n)))
    return sorted(s)


def _row_err(g, ref):
    num = np.max(np.abs(g - ref), axis=-1)
    return float(np.max(num / np.maximum(1.0, np.max(np.abs(ref), axis=-1))))


@pytest.mark.parametrize("B,H,T,D", [(65535, 1, 3, 64), (2, 256, 70, 64), (4, 256, 5, 128)])
def test_largest_batch_and_head_counts(B, H, T, D):
    cfg = W.FwdConfig("t", B, H, T, D, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 5 + H)
    P1, P2, V, dY = (inp[k].to(DEV).contiguous() for k in ("P1", "P2", "V", "dY"))
    Y, L = R.fwd_lse(P1, P2, V, inp["tau"], 0.5)
    g = R.bwd(P1, P2, V, inp["tau"], 0.5, Y, L, dY)
    torch.cuda.synchronize()
    Yh, Lh, gh = f64(Y), f64(L), [f64(x) for x in g[:3]]
    rng = np.random.default_rng(B + H)
    for b, h in _slices(B, H, rng):
        x = [f64(inp[k])[b, h] for k in ("P1", "P2", "V", "dY")]
        tau = float(inp["tau"][h])
        ref_y = O.relation_head(x[0], x[1], x[2], tau, 0.5)
        assert float(np.max(np.abs(Yh[b, h] - ref_y))) <= 2e-2, ("Y", b, h)
        assert float(np.max(np.abs(Lh[b, h] - O.row_lse(x[0], x[1], tau, 0.5)))) <= 1e-4, ("LSE", b, h)
        ref_g = O.relation_head_bwd(x[0], x[1], x[2], tau, 0.5, x[3])
        for n, name in enumerate(("dP1", "dP2", "dV")):
            assert _row_err(gh[n][b, h], ref_g[n]) <= 2e-2, (name, b, h)


def test_linear_and_decode_at_the_largest_batch():
    B, H, T, D = 65535, 1, 3, 64
    cfg = W.FwdConfig("t", B, H, T, D, "bf16")
    inp = W.make_linear_inputs(cfg, 8)
    P1, P2, I = (inp[k].to(DEV).contiguous() for k in ("P1", "P2", "V"))
    A = inp["alpha"].to(DEV)
    Y, _ = R.linear_fwd(P1, P2, I, A, inp["tau"])
    # decode: the cache holds the first T - 1 tokens, the new token is the last
    cP2 = P2[:, :, : T - 1].contiguous()
    cV = I[:, :, : T - 1].contiguous()
    lens = torch.full((B,), T - 1, dtype=torch.int32, device=DEV)
    y = R.decode(P1[:, :, T - 1].contiguous(), P2[:, :, T - 1].contiguous(), I[:, :, T - 1].contiguous(),
                 cP2, cV, lens, inp["tau"], 0.0)
    torch.cuda.synchronize()
    Yh, yh = f64(Y), f64(y)
    rng = np.random.default_rng(9)
    for b, h in _slices(B, H, rng):
        sub = lambda k: f64(inp[k])[b:b + 1, h:h + 1]
        ref = LO.linear_relation_fwd(sub("P1"), sub("P2"), sub("V"), sub("alpha"), inp["tau"][h:h + 1].astype(np.float64))
        assert _row_err(Yh[b, h], ref[0, 0]) <= 2e-2, ("linear", b, h)
        x = [f64(inp[k])[b, h] for k in ("P1", "P2", "V")]
        full = O.relation_head(x[0], x[1], x[2], float(inp["tau"][h]), 0.0)
        assert float(np.max(np.abs(yh[b, h] - full[T - 1]))) <= 2e-2, ("decode", b, h)
