"""The entry points under stream capture: the training forward, the
backward (stored-dU workspace), the inference forward, the Linear Relation
(on a shape that walks groups of chunks) and the allocation-free decode step
are captured once into a graph (torch.cuda.CUDAGraph, a hipGraph
on this platform) and replayed several times, with eager work and
synchronisations between the replays. Every replay must reproduce the eager
results bit for bit (the kernels use no atomics, so every path is
deterministic). The library itself issues no memset, copy, allocation or
synchronisation, only kernel launches on the caller's stream."""
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_forward_backward_linear_and_decode_replay_in_a_graph():
    cfg = W.FwdConfig("t", 2, 4, 600, 128, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
    inp = W.make_bwd_inputs(cfg, 71)
    P1, P2, V, dY = (inp[k].to(DEV).contiguous() for k in ("P1", "P2", "V", "dY"))
    tau = inp["tau"]
    dc = W.DecodeConfig("d", 3, 4, 128, 0, 500, 500, dtype="bf16", tau=0.8)
    di = W.make_decode_inputs(dc, 72)
    p1, p2, v, cP2, cV = (di[k].to(DEV).contiguous() for k in ("p1", "p2", "v", "cache_P2", "cache_V"))
    lens = torch.from_numpy(di["lens"]).to(DEV)
    li = W.make_linear_inputs(W.FwdConfig("l", 1, 96, 600, 128, "bf16"), 73)
    lP1, lP2, lI, lA = (li[k].to(DEV).contiguous() for k in ("P1", "P2", "V", "alpha"))
    lws = torch.empty(R.lib().relation_linear_workspace_bytes(1, 96, 600, 128), dtype=torch.uint8, device=DEV)

    def work():
        Yf = R.fwd(P1, P2, V, tau, 0.5)
        Y, L = R.fwd_lse(P1, P2, V, tau, 0.5)
        g = R.bwd(P1, P2, V, tau, 0.5, Y, L, dY)
        y = R.decode_noalloc(p1, p2, v, cP2, cV, lens, di["tau"], 0.5, out=torch.empty_like(v))
        Yl, C = R.linear_fwd(lP1, lP2, lI, lA, li["tau"], state=torch.empty((1, 96, 128, 128), device=DEV),
                             workspace=lws)
        return (Yf, Y, L) + tuple(g) + (y, Yl, C)

    eager = [t.clone() for t in work()]
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        work()                                   # warm-up on a side stream before capture
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        outs = work()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs:                           # eager work between replays
            t.fill_(float("nan") if t.is_floating_point() else 0)
        junk = torch.randn(1 << 20, device=DEV).square().sum()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert bool(torch.isfinite(junk))
        for n, (a, b) in enumerate(zip(outs, eager)):
            assert torch.equal(a, b), f"replay {rep}: output {n} differs from the eager call"
