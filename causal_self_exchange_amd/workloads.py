"""Seeded synthetic workloads for the causal Self-Exchange Relation forward, backward and decode.

This module only draws and stores numbers. It holds none of the operator's
arithmetic, so both the HIP path and the CPU oracle can consume what it makes
without sharing any of the method's code.

Shapes follow the paper's per-head layout (P1, P2 and the mixed information
state I~, written V here, each T x d_h per head; "Ask Self, Ask Others: Relation
Is All You Need", App. A.1.1), stored as contiguous [B, H, T, d_h] tensors.
The paper's own systems runs are whole training steps on text corpora that are
not available here; the operator's cost depends only on (B, H, T, d_h), so
seeded Gaussian inputs of the same shapes stand in for them.

Recipe (all draws float32 from numpy's PCG64 ``default_rng(seed)``):
  forward: P1, P2, V ~ scale * N(0, 1) drawn in that order, then tau
           (a per-head uniform draw when ``tau`` is "uniform"), then rounded
           to the storage dtype with round-to-nearest-even.
  backward: the forward's draws, then dY ~ N(0, 1) [B, H, T, d_h] from
           ``default_rng(seed + 1000003)``, rounded to the storage dtype.
  linear : the forward's draws, then the retention alpha (see
           make_linear_inputs) from ``default_rng(seed + 2000003)``.
  decode : cache lengths L_b ~ U{lo..hi}, then for each sequence b in order
           its cached P2 rows [H, L_b, d_h] and cached V rows; then the new
           token's p1, p2, v [B, H, d_h]. Cache rows past L_b hold NaN.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np
import torch

SEEDS = (42, 43, 44)


@dataclass(frozen=True)
class FwdConfig:
    name: str
    B: int
    H: int
    T: int
    d_h: int
    dtype: str            # "f32" or "bf16"
    scale: float = 1.0
    tau: object = 1.0     # a float, or ("uniform", lo, hi)
    lam: float = 0.0

    @property
    def flops(self) -> float:
        """Causal FLOPs: evidence over j <= i plus transport over j < i."""
        return 2.0 * self.B * self.H * self.T * self.T * self.d_h


@dataclass(frozen=True)
class DecodeConfig:
    name: str
    B: int
    H: int
    d_h: int
    L_lo: int
    L_hi: int
    L_cap: int
    dtype: str = "bf16"
    tau: float = 1.0
    lam: float = 0.0


CONFIGS = {
    "tiny": FwdConfig("tiny", 1, 2, 128, 32, "f32"),
    "small": FwdConfig("small", 8, 8, 512, 64, "bf16"),
    "mid": FwdConfig("mid", 4, 16, 2048, 64, "bf16", tau=("uniform", 0.5, 2.0)),
    "long": FwdConfig("long", 1, 32, 8192, 128, "bf16", scale=0.5),
}

DECODE_CONFIG = DecodeConfig("decode", 64, 32, 128, 1024, 4096, 4096)

_TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def torch_dtype(name: str) -> torch.dtype:
    return _TORCH_DTYPE[name]


def _store(x: np.ndarray, dtype: str) -> torch.Tensor:
    """float32 numpy -> CPU tensor in the storage dtype (RNE for bf16)."""
    return torch.from_numpy(np.ascontiguousarray(x)).to(_TORCH_DTYPE[dtype])


def make_fwd_inputs(cfg: FwdConfig, seed: int):
    """Returns dict(P1, P2, V: CPU tensors [B,H,T,d_h]; tau: float32[H]; lam)."""
    rng = np.random.default_rng(seed)
    shape = (cfg.B, cfg.H, cfg.T, cfg.d_h)
    s = np.float32(cfg.scale)
    P1 = rng.standard_normal(shape, dtype=np.float32) * s
    P2 = rng.standard_normal(shape, dtype=np.float32) * s
    V = rng.standard_normal(shape, dtype=np.float32) * s
    if isinstance(cfg.tau, tuple):
        _, lo, hi = cfg.tau
        tau = rng.uniform(lo, hi, cfg.H).astype(np.float32)
    else:
        tau = np.full(cfg.H, cfg.tau, dtype=np.float32)
    return dict(P1=_store(P1, cfg.dtype), P2=_store(P2, cfg.dtype),
                V=_store(V, cfg.dtype), tau=tau, lam=float(cfg.lam))


def make_bwd_inputs(cfg: FwdConfig, seed: int):
    """make_fwd_inputs plus an upstream gradient dY ~ N(0, 1) [B,H,T,d_h] in
    the storage dtype, drawn from its own stream (seed + 1000003) so that the
    forward inputs are the same as make_fwd_inputs(cfg, seed)."""
    inp = make_fwd_inputs(cfg, seed)
    rng = np.random.default_rng(seed + 1000003)
    dY = rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.d_h), dtype=np.float32)
    inp["dY"] = _store(dY, cfg.dtype)
    return inp


def make_linear_inputs(cfg: FwdConfig, seed: int):
    """make_fwd_inputs plus a retention alpha [B,H,T,d_h] (fp32) drawn like the
    paper's parameterisation with random weights: per (h, channel) a rate
    a ~ U(1, 16) and a bias beta = log(e^dt - 1) with dt log-uniform in
    [1e-3, 1e-1]; per token z ~ 0.5 N(0, 1); alpha = exp(-a softplus(z + beta)).
    Drawn from default_rng(seed + 2000003), so the other inputs equal
    make_fwd_inputs(cfg, seed)."""
    inp = make_fwd_inputs(cfg, seed)
    rng = np.random.default_rng(seed + 2000003)
    a = rng.uniform(1.0, 16.0, (cfg.H, cfg.d_h))
    dt = np.exp(rng.uniform(np.log(1e-3), np.log(1e-1), (cfg.H, cfg.d_h)))
    beta = np.log(np.expm1(dt))
    z = 0.5 * rng.standard_normal((cfg.B, cfg.H, cfg.T, cfg.d_h))
    alpha = np.exp(-a[None, :, None, :] * np.logaddexp(0.0, z + beta[None, :, None, :]))
    inp["alpha"] = torch.from_numpy(alpha.astype(np.float32))
    return inp


def make_decode_inputs(cfg: DecodeConfig, seed: int):
    """Returns dict(p1, p2, v [B,H,d_h]; cache_P2, cache_V [B,H,L_cap,d_h] with
    NaN past each length; lens int32[B]; tau float32[H]; lam)."""
    rng = np.random.default_rng(seed)
    lens = rng.integers(cfg.L_lo, cfg.L_hi, cfg.B, endpoint=True).astype(np.int32)
    tdt = _TORCH_DTYPE[cfg.dtype]
    cache_P2 = torch.full((cfg.B, cfg.H, cfg.L_cap, cfg.d_h), float("nan"), dtype=tdt)
    cache_V = torch.full((cfg.B, cfg.H, cfg.L_cap, cfg.d_h), float("nan"), dtype=tdt)
    for b in range(cfg.B):
        L = int(lens[b])
        cache_P2[b, :, :L] = _store(rng.standard_normal((cfg.H, L, cfg.d_h), dtype=np.float32), cfg.dtype)
        cache_V[b, :, :L] = _store(rng.standard_normal((cfg.H, L, cfg.d_h), dtype=np.float32), cfg.dtype)
    shape = (cfg.B, cfg.H, cfg.d_h)
    p1 = _store(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    p2 = _store(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    v = _store(rng.standard_normal(shape, dtype=np.float32), cfg.dtype)
    tau = np.full(cfg.H, cfg.tau, dtype=np.float32)
    return dict(p1=p1, p2=p2, v=v, cache_P2=cache_P2, cache_V=cache_V, lens=lens,
                tau=tau, lam=float(cfg.lam))


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Exact widening of a stored tensor (f32 or bf16) to float64 numpy."""
    return t.detach().cpu().to(torch.float64).numpy()
