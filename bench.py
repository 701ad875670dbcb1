"""Benchmark: causal Self-Exchange Relation forward (FlashRelation) on one GPU.

One step = one relation_fwd call over the T = 8192 workload
(B=1, H=32, T=8192, d_h=128, bf16, P1/P2/V ~ 0.5 N(0,1), tau = 1, seed 42),
inputs resident in HBM before timing starts. Throughput counts the causal
FLOPs 2 B H T^2 d_h (evidence over j <= i plus transport over j < i).
The default warm-up (200 launches, ~0.15 s) lets the engine clock reach its
sustained level under MFMA load before the timed region; the paper likewise
reports steady-state throughput with warm-up excluded.

Prints ONE JSON line. Also reported (not the headline): the backward
(relation_bwd) on the same workload, the model-side pre-steps (RoPE + Givens,
relation_prestep) and the forward on raw projections (relation_fwd_model) on
its shape, the Linear Relation forward on its shape, the paper-geometry
comparison with PyTorch FlashAttention on this GPU, one Relation Cache
decode step (B=64,
H=32, d_h=128, cache lengths U{1024..4096}) in GB/s of algorithmic cache
traffic, and the CPU oracle timed on a bounded sample.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "relation_fwd TFLOP/s (causal) and % of MI355X bf16 MFMA peak at T=8192"
PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA (256 CU x 4096 FLOP/clk x 2.4 GHz)
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
FWD_KERNEL_SRC = os.path.join(ROOT, "causal_self_exchange_amd", "csrc", "fwd_mfma.hip")
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "fwd_long_traffic.json")


def _src_sha(path):
    with open(path, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def _traffic(launch_bytes_key="bytes_per_launch"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, only
    while the kernel source is unchanged since the counters were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("source_sha") != _src_sha(FWD_KERNEL_SRC):
        return None
    return t.get(launch_bytes_key)


def time_launches(fn, steps, warmup, torch, batch=False):
    """Per-launch durations (ms) from HIP events on the launching stream. With
    batch=True only the first and last events are recorded (for kernels short
    enough that an event between launches shows in the time); every launch
    is then given the batch mean."""
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 if batch else steps + 1)]
    t0 = time.perf_counter()
    evs[0].record(stream)
    for i in range(steps):
        fn()
        if not batch:
            evs[i + 1].record(stream)
    if batch:
        evs[1].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    total = evs[0].elapsed_time(evs[-1])
    per = [total / steps] * steps if batch else [evs[i].elapsed_time(evs[i + 1]) for i in range(steps)]
    return per, total, wall


def _oracle_head_seconds(args):
    """One head of the oracle in this (single-threaded) worker process."""
    from oracle import relation_oracle as O
    p1, p2, v, tau = args
    t0 = time.perf_counter()
    O.relation_head(p1, p2, v, tau, 0.0)
    return time.perf_counter() - t0


def cpu_baseline(inp, max_procs=16):
    """The CPU oracle (materialised fp64 definition), timed on the host before
    any GPU work: one head per worker process, each process single-threaded
    (BLAS limited to one thread; numpy's elementwise work is single-threaded
    anyway), as many processes as the CPUs this process may run on (at most
    `max_procs`, about 2 GB of memory each at T = 8192). `cores` is the number
    of threads that did the work. Reported in the headline unit."""
    import multiprocessing as mp

    from threadpoolctl import threadpool_limits
    import torch
    _, H, T, d = inp["P1"].shape
    avail = len(os.sched_getaffinity(0))
    n = max(1, min(avail, H, max_procs))
    work = [(inp["P1"][0, h].to(torch.float64).numpy(), inp["P2"][0, h].to(torch.float64).numpy(),
             inp["V"][0, h].to(torch.float64).numpy(), float(inp["tau"][h])) for h in range(n)]
    with threadpool_limits(limits=1):
        ctx = mp.get_context("fork")          # no GPU has been touched in this process yet
        with ctx.Pool(n) as pool:
            t0 = time.perf_counter()
            per_head = pool.map(_oracle_head_seconds, work, chunksize=1)
            dt = time.perf_counter() - t0
    return {"value": n * 2.0 * T * T * d / dt / 1e12, "unit": "TFLOP/s", "cores": n, "kind": "oracle",
            "seconds": round(dt, 3), "host_cpus_available": avail,
            "sample": f"{n} of {H} heads (b=0, h=0..{n - 1}) of the B=1 H={H} T={T} d_h={d} workload, fp64 "
                      f"materialised R and F, one head per process, {n} single-threaded processes "
                      f"(slowest head {max(per_head):.2f} s)"}


def bench_decode(torch, R, W, steps, warmup):
    cfg = W.DECODE_CONFIG
    inp = W.make_decode_inputs(cfg, 42)
    d = {k: inp[k].cuda() for k in ("p1", "p2", "v", "cache_P2", "cache_V")}
    lens = torch.from_numpy(inp["lens"]).cuda()
    ws = torch.empty(R.decode_workspace_bytes(cfg.B, cfg.H, cfg.L_cap, cfg.d_h), dtype=torch.uint8,
                     device="cuda")
    y = torch.empty_like(d["v"])

    def fn():
        R.decode(d["p1"], d["p2"], d["v"], d["cache_P2"], d["cache_V"], lens, inp["tau"], 0.0,
                 out=y, workspace=ws)

    per, total, _ = time_launches(fn, steps, warmup, torch)
    L = inp["lens"].astype(np.int64)
    bytes_alg = float(np.sum(L) * cfg.H * cfg.d_h * 2 * 2 + 4 * cfg.B * cfg.H * cfg.d_h * 2)
    ms = total / steps
    return {"workload": "decode: B=64 H=32 d_h=128 bf16, cache lengths U{1024..4096}, seed 42",
            "us_per_step": round(ms * 1e3, 2), "GB/s": round(bytes_alg / (ms * 1e-3) / 1e9, 1),
            "frac_of_hbm_peak": round(bytes_alg / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": bytes_alg}


def bench_backward(torch, R, W, steps, warmup):
    """relation_bwd on the T = 8192 workload with a seeded N(0, 1) upstream
    gradient; LSE and Y from relation_fwd_lse (outside the timed region).
    Throughput counts the 5 causal products of the gradient (recomputed U,
    dY V^T, F^T dY, dU P2, dU^T P1): 5 B H T^2 d_h FLOPs, 2.5x the forward's.
    The call gets the workspace with which dU is stored once; the path that
    recomputes the evidence for dP1 instead (small workspace) is timed
    beside it."""
    cfg = W.CONFIGS["long"]
    inp = W.make_bwd_inputs(cfg, 42)
    P1, P2, V, dY = (inp[k].cuda() for k in ("P1", "P2", "V", "dY"))
    tau = inp["tau"]
    Y, L = R.fwd_lse(P1, P2, V, tau, 0.0)
    grads = (torch.empty_like(P1), torch.empty_like(P2), torch.empty_like(V),
             torch.empty(cfg.H, dtype=torch.float32, device="cuda"),
             torch.empty(1, dtype=torch.float32, device="cuda"))
    small = R.bwd_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d_h)
    stored = R.bwd_stored_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d_h)
    ws = torch.empty(max(small, stored), dtype=torch.uint8, device="cuda")

    def timed(nbytes):
        def fn():
            R.bwd(P1, P2, V, tau, 0.0, Y, L, dY, grads=grads, workspace=ws[:nbytes])
        _, total, _ = time_launches(fn, steps, warmup, torch)
        return total / steps

    ms = timed(max(small, stored))
    ms_recompute = timed(small)
    flops = 5.0 * cfg.B * cfg.H * cfg.T * cfg.T * cfg.d_h
    return {"workload": "backward: B=1 H=32 T=8192 d_h=128 bf16, dY ~ N(0,1), seed 42 "
                        "(row statistics, dkv storing dU, dP1 from the stored dU, reduce)",
            "ms_per_step": round(ms, 4), "TFLOP/s": round(flops / (ms * 1e-3) / 1e12, 2),
            "pct_of_peak": round(100.0 * flops / (ms * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2),
            "flops_counted": flops, "workspace_bytes": max(small, stored),
            "recompute_path_ms_per_step": round(ms_recompute, 4), "recompute_path_workspace_bytes": small}


def bench_prestep(torch, R, W, steps, warmup):
    """relation_prestep (RoPE on P1/P2 + Givens mixing of I, one HBM pass) and
    relation_fwd_model (pre-step + forward) on the T = 8192 workload's shape,
    interleaved rotary pairs, base 1e4, pairing A, seeded angles."""
    cfg = W.CONFIGS["long"]
    inp = W.make_fwd_inputs(cfg, 42)
    P1, P2, I = (inp[k].cuda() for k in ("P1", "P2", "V"))
    theta = np.random.default_rng(43).uniform(-np.pi, np.pi, cfg.H // 2).astype(np.float32)
    out = (torch.empty_like(P1), torch.empty_like(P2), torch.empty_like(I))

    # Arguments marshalled once: the kernel is shorter than a call's Python
    # marshalling, which would otherwise be what the events time.
    pre = R.prestep_launcher(P1, P2, I, None, "interleaved", 1e4, theta, "A", out)
    per, total, _ = time_launches(pre, steps, warmup, torch, batch=True)
    ms = total / steps
    nbytes = 6.0 * cfg.B * cfg.H * cfg.T * cfg.d_h * 2      # read P1, P2, I; write three outputs
    Y = torch.empty_like(I)
    ws = torch.empty(R.lib().relation_fwd_model_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d_h, R.REL_BF16),
                     dtype=torch.uint8, device="cuda")

    def model():
        R.fwd_model(P1, P2, I, inp["tau"], 0.0, None, "interleaved", 1e4, theta, "A", out=Y, workspace=ws)

    _, mtotal, _ = time_launches(model, steps, warmup, torch)
    mms = mtotal / steps
    return {"workload": "pre-steps: B=1 H=32 T=8192 d_h=128 bf16, interleaved RoPE base 1e4, Givens pairing A",
            "prestep_us": round(ms * 1e3, 2), "prestep_GB/s": round(nbytes / (ms * 1e-3) / 1e9, 1),
            "prestep_frac_of_hbm_peak": round(nbytes / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, 4),
            "algorithmic_bytes": nbytes, "fwd_model_ms": round(mms, 4),
            "fwd_model_TFLOP/s": round(cfg.flops / (mms * 1e-3) / 1e12, 2)}


def bench_linear(torch, R, W, steps, warmup):
    """relation_linear_fwd (chunk-parallel Linear Relation) on the T = 8192
    workload's shape (B=1, H=32, d_h=128, bf16) with the seeded retention of
    workloads.make_linear_inputs. Work per chunk of L = 64 tokens and head:
    the chunk state 2 L d^2, the read from the entering state 2 L d^2, the
    intra-chunk coefficients and their application 2 L^2 d (half of it
    masked), the scan 2 d^2: counted as (4 d^2 + 2 L d) FLOP per token (the
    on-chip state update within a group repeats the chunk state's product
    and is not counted)."""
    cfg = W.CONFIGS["long"]
    inp = W.make_linear_inputs(cfg, 42)
    P1, P2, I = (inp[k].cuda() for k in ("P1", "P2", "V"))
    A = inp["alpha"].cuda()
    Y = torch.empty_like(I)
    ws = torch.empty(R.lib().relation_linear_workspace_bytes(cfg.B, cfg.H, cfg.T, cfg.d_h), dtype=torch.uint8,
                     device="cuda")

    def fn():
        R.linear_fwd(P1, P2, I, A, inp["tau"], out=Y, workspace=ws)

    _, total, _ = time_launches(fn, steps, warmup, torch)
    ms = total / steps
    d, L = cfg.d_h, 64
    ntok = cfg.B * cfg.H * cfg.T
    flops = float(ntok) * (4 * d * d + 2 * L * d)
    io_bytes = float(ntok) * d * (3 * 2 + 4 + 2)          # P1, P2, I bf16 + alpha fp32 in, Y bf16 out
    # Chunks per group as the library picks them for bf16 inputs: the largest
    # power of two up to 16 that leaves one group per compute unit.
    nc, bh = (cfg.T + L - 1) // L, cfg.B * cfg.H
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    group = next((g for g in (16, 8, 4, 2) if bh * ((nc + g - 1) // g) >= n_cu), 1)
    groups = bh * ((nc + group - 1) // group)
    # group states (write, scan read and write, read) and row factors (write, read)
    state_bytes = float(groups) * d * d * 4 * 4 + float(ntok) * 2 * 4 * 2
    return {"workload": f"linear relation: B=1 H=32 T=8192 d_h=128 bf16, seeded retention, 64-token chunks in groups of {group}",
            "us_per_call": round(ms * 1e3, 2), "tokens/s": round(cfg.B * cfg.T / (ms * 1e-3), 1),
            "TFLOP/s_counted": round(flops / (ms * 1e-3) / 1e12, 2),
            "arithmetic": "fp32 accumulation; products on bf16 MFMA over split bf16 operand pairs",
            "GB/s_io_plus_states": round((io_bytes + state_bytes) / (ms * 1e-3) / 1e9, 1),
            "flops_counted": flops, "io_bytes": io_bytes, "state_bytes": state_bytes}


PAPER_GEOMETRY = (   # ([paper] Table 6 / Table 4(b)): d_h, T; H = 8, 131,072 tokens per step
    ("10M", 48, 1024), ("30M", 64, 2048), ("100M", 80, 4096))


def _flash_sdpa(torch):
    """A context forcing PyTorch's flash (else memory-efficient) SDPA kernel;
    never the math path (it issues batched bf16 products). None if neither
    backend is available."""
    try:
        from torch.nn.attention import SDPBackend, sdpa_kernel
    except ImportError:
        return None, None
    for name, be in (("flash", SDPBackend.FLASH_ATTENTION), ("efficient", SDPBackend.EFFICIENT_ATTENTION)):
        try:
            q = torch.randn(1, 1, 64, 64, dtype=torch.bfloat16, device="cuda")
            with sdpa_kernel([be]):
                torch.nn.functional.scaled_dot_product_attention(q, q, q, is_causal=True)
            torch.cuda.synchronize()
            return name, be
        except RuntimeError:
            continue
    return None, None


def bench_paper_geometry(torch, R, W, steps, warmup):
    """The operator-level counterpart of the paper's Table 4(b): FlashRelation
    (relation_fwd_ex, lambda = 0.5 as in the paper's models) against PyTorch
    FlashAttention (scaled_dot_product_attention, causal, flash backend
    forced) on the same MI355X, H = 8 and 131,072 tokens per step at the three
    model geometries (d_h, T) = (48, 1024), (64, 2048), (80, 4096), forward
    and forward + backward (relation_fwd_lse + relation_bwd against SDPA with
    autograd). Tokens/s and the FR / FA ratio."""
    from torch.nn.attention import sdpa_kernel
    be_name, be = _flash_sdpa(torch)
    out = {"attention_backend": be_name, "rows": []}
    for scale, d, T in PAPER_GEOMETRY:
        B, H = 131072 // T, 8
        cfg = W.FwdConfig("paper", B, H, T, d, "bf16", tau=("uniform", 0.5, 2.0), lam=0.5)
        inp = W.make_bwd_inputs(cfg, 42)
        P1, P2, V, dY = (inp[k].cuda() for k in ("P1", "P2", "V", "dY"))
        Y = torch.empty_like(V)
        _, fr_ms, _ = time_launches(lambda: R.fwd(P1, P2, V, inp["tau"], 0.5, out=Y), steps, warmup, torch)
        fr_ms /= steps
        row = {"scale": scale, "B": B, "H": H, "T": T, "d_h": d, "tokens": B * T,
               "FR_fwd_ms": round(fr_ms, 4), "FR_fwd_tok/s": round(B * T / (fr_ms * 1e-3), 0)}
        if be is not None:
            with sdpa_kernel([be]):
                _, fa_ms, _ = time_launches(
                    lambda: torch.nn.functional.scaled_dot_product_attention(P1, P2, V, is_causal=True),
                    steps, warmup, torch)
            fa_ms /= steps
            row.update({"FA_fwd_ms": round(fa_ms, 4), "FA_fwd_tok/s": round(B * T / (fa_ms * 1e-3), 0),
                        "FR_over_FA_fwd": round(fa_ms / fr_ms, 3)})
        Yl, L = R.fwd_lse(P1, P2, V, inp["tau"], 0.5)
        grads = (torch.empty_like(P1), torch.empty_like(P2), torch.empty_like(V),
                 torch.empty(H, device="cuda"), torch.empty(1, device="cuda"))
        ws = torch.empty(max(R.bwd_workspace_bytes(B, H, T, d), R.bwd_stored_workspace_bytes(B, H, T, d)),
                         dtype=torch.uint8, device="cuda")

        def fr_train():
            R.fwd_lse(P1, P2, V, inp["tau"], 0.5, out=Yl, lse=L)
            R.bwd(P1, P2, V, inp["tau"], 0.5, Yl, L, dY, grads=grads, workspace=ws)

        _, frt, _ = time_launches(fr_train, steps, warmup, torch)
        frt /= steps
        row.update({"FR_fwd_bwd_ms": round(frt, 4), "FR_fwd_bwd_tok/s": round(B * T / (frt * 1e-3), 0)})
        if be is not None:
            q, k, v = (x.detach().clone().requires_grad_(True) for x in (P1, P2, V))

            def fa_train():
                with sdpa_kernel([be]):
                    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True)
                o.backward(dY)

            _, fat, _ = time_launches(fa_train, steps, warmup, torch)
            fat /= steps
            row.update({"FA_fwd_bwd_ms": round(fat, 4), "FA_fwd_bwd_tok/s": round(B * T / (fat * 1e-3), 0),
                        "FR_over_FA_fwd_bwd": round(fat / frt, 3)})
        out["rows"].append(row)
        del P1, P2, V, dY, Y
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-backward", action="store_true")
    ap.add_argument("--no-prestep", action="store_true")
    ap.add_argument("--no-linear", action="store_true")
    ap.add_argument("--no-paper", action="store_true")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB (read MIB, write MIB) "
                         "5 times: the reference kernel for scaling HBM byte counters")
    args = ap.parse_args()
    if args.copy_calibration:
        import torch
        n = args.copy_calibration * (1 << 20)
        src = torch.empty(n, dtype=torch.uint8, device="cuda").random_(0, 255)
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": n, "launches": 5}), flush=True)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only (the operator shards over heads with no "
              f"communication); --gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    from causal_self_exchange_amd import relation as R
    from causal_self_exchange_amd import workloads as W

    cfg = W.CONFIGS["long"]
    inp = W.make_fwd_inputs(cfg, 42)
    # The CPU baseline runs first, while no GPU context exists in this process
    # (its worker processes are forked).
    cpu = None if args.no_cpu_baseline else cpu_baseline(inp)
    P1, P2, V = (inp[k].cuda() for k in ("P1", "P2", "V"))
    Y = torch.empty_like(V)
    tau = inp["tau"]

    def step():
        R.fwd(P1, P2, V, tau, 0.0, out=Y)

    per, total, wall = time_launches(step, args.steps, args.warmup, torch)
    ms_step = total / args.steps
    avg_launch_ms = float(np.mean(per))
    flops = cfg.flops
    value = flops / (ms_step * 1e-3) / 1e12
    achieved = flops / (avg_launch_ms * 1e-3) / 1e12
    traffic = _traffic()

    out = {
        "metric": METRIC, "value": round(value, 2), "unit": "TFLOP/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_step, 4),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "long-context SER/MHR forward: B=1 H=32 T=8192 d_h=128 bf16, "
                               "P1/P2/V ~ 0.5 N(0,1), tau=1, causal, seed 42",
                   "B": cfg.B, "H": cfg.H, "T": cfg.T, "d_h": cfg.d_h},
        "pct_of_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic,
                     "kernel": "relation_fwd (bf16 MFMA FlashRelation)",
                     "avg_launch_us": round(avg_launch_ms * 1e3, 2),
                     "median_launch_us": round(float(np.median(per)) * 1e3, 2),
                     "min_launch_us": round(float(np.min(per)) * 1e3, 2)},
        "wall_s_timed_region": round(wall, 4),
    }
    if not args.no_backward:
        out["backward"] = bench_backward(torch, R, W, max(10, args.steps // 4), max(10, args.warmup // 4))
    if not args.no_prestep:
        out["prestep"] = bench_prestep(torch, R, W, max(10, args.steps // 4), max(10, args.warmup // 4))
    if not args.no_linear:
        out["linear"] = bench_linear(torch, R, W, max(10, args.steps // 4), max(10, args.warmup // 4))
    if not args.no_paper:
        out["paper_geometry"] = bench_paper_geometry(torch, R, W, max(10, args.steps // 10), max(5, args.warmup // 10))
    if not args.no_decode:
        out["decode"] = bench_decode(torch, R, W, max(10, args.steps // 2), args.warmup)
    if cpu is not None:
        out["cpu_baseline"] = cpu
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
