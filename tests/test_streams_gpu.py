"""Calls on several streams at once: the forward and the backward hold no
state between calls, so independent calls issued on different streams
without synchronisation between them give the results of the same calls
issued one at a time."""
import pytest
import torch

from causal_self_exchange_amd import relation as R
from causal_self_exchange_amd import workloads as W

pytestmark = pytest.mark.gpu

DEV = "cuda"


def test_concurrent_calls_on_separate_streams():
    cases = []
    for n, (T, D) in enumerate(((700, 128), (1100, 64), (300, 80))):
        cfg = W.FwdConfig("t", 1, 4, T, D, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
        inp = W.make_bwd_inputs(cfg, 90 + n)
        cases.append(([inp[k].to(DEV).contiguous() for k in ("P1", "P2", "V", "dY")], inp["tau"]))

    def run(case, stream=None):
        (P1, P2, V, dY), tau = case
        Y, L = R.fwd_lse(P1, P2, V, tau, 0.5, stream=stream)
        g = R.bwd(P1, P2, V, tau, 0.5, Y, L, dY, stream=stream)
        return (Y, L) + tuple(g)

    serial = []
    for c in cases:
        serial.append([t.clone() for t in run(c)])
        torch.cuda.synchronize()
    streams = [torch.cuda.Stream() for _ in cases]
    for s in streams:
        s.wait_stream(torch.cuda.current_stream())
    outs = []
    for c, s in zip(cases, streams):
        with torch.cuda.stream(s):
            outs.append(run(c, stream=s))
    torch.cuda.synchronize()
    for n, (a, b) in enumerate(zip(outs, serial)):
        for k, (x, y) in enumerate(zip(a, b)):
            assert torch.equal(x, y), f"case {n} output {k}"
