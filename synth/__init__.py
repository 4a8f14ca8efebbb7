"""Seeded synthetic inputs for the selective-scan workloads.

This module holds only the input recipe: random draws, bf16 rounding of the
draws and the workload table.  It contains none of the scan's arithmetic, and
both the oracle-side code (tests, CPU baseline) and the GPU-side code (tests,
benchmark, smoke check) take their inputs from here.

Every tensor comes from its own numpy PCG64 stream keyed by (seed, tensor
name), so the draws do not depend on generation order.  bf16 tensors are
drawn in float32 and rounded to nearest-even bf16; the returned float32
arrays hold exactly the rounded values, which is what both sides consume.
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional, Tuple

import numpy as np

# ---------------------------------------------------------------------------
# Workloads.  Mamba-1 shapes use the [batch, dim, seqlen] layout with B and C
# as [batch, dstate, seqlen]; the SSD shape uses [batch, seqlen, heads, P].
# ---------------------------------------------------------------------------


@dataclasses.dataclass(frozen=True)
class Mamba1Config:
    name: str
    batch: int
    dim: int
    dstate: int
    seqlen: int
    dtype: str                 # "f32" or "bf16": u, delta, B, C, z, y
    delta_mean: float = 0.0    # delta_raw ~ N(delta_mean, delta_std)
    delta_std: float = 1.0
    delta_bias: bool = False   # inverse-softplus of dt ~ logU[1e-3, 1e-1] per channel
    gate: bool = False         # z given (silu gate on)
    use_D: bool = True
    softplus: bool = True
    sample_rows: Optional[int] = None  # compare y on this many seeded rows only


@dataclasses.dataclass(frozen=True)
class SSDConfig:
    name: str
    batch: int
    seqlen: int
    nheads: int
    headdim: int
    dstate: int
    ngroups: int
    chunk: int
    dtype: str = "bf16"


MAMBA1_CONFIGS: Dict[str, Mamba1Config] = {
    # Tiny fp32 case: every output compared.
    "tiny": Mamba1Config("tiny", 1, 16, 4, 64, "f32"),
    # Mamba-130M-shaped layer, fp32.
    "m130m": Mamba1Config("m130m", 2, 1536, 16, 2048, "f32", 0.0, 0.5,
                          delta_bias=True, gate=True),
    # Mamba-1.4B-shaped layer, bf16 inputs (the throughput workload).
    "m1p4b": Mamba1Config("m1p4b", 8, 4096, 16, 2048, "bf16", 0.0, 0.5,
                          delta_bias=True, gate=True),
    # Long-sequence stress, bf16, slow decay.
    "long": Mamba1Config("long", 16, 1536, 16, 16384, "bf16", -2.0, 1.0,
                         delta_bias=False, gate=True, sample_rows=64),
}

SSD_CONFIGS: Dict[str, SSDConfig] = {
    "ssd": SSDConfig("ssd", 4, 4096, 24, 64, 128, 1, 256, "bf16"),
}

# Extra small shapes from the exercise spec's correctness matrix
# ((batch, dim, seqlen) in {(2,4,8), (1,32,256), (8,128,64)}), fp32.
SPEC_SHAPES: Tuple[Tuple[int, int, int], ...] = ((2, 4, 8), (1, 32, 256), (8, 128, 64))


# ---------------------------------------------------------------------------
# Random streams and rounding
# ---------------------------------------------------------------------------

def _rng(seed: int, name: str) -> np.random.Generator:
    key = int.from_bytes(hashlib.sha256(name.encode()).digest()[:8], "little")
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([int(seed), key])))


def round_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns
    float32 holding the rounded values.  Inputs here are finite."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32)
    lsb = (bits >> np.uint32(16)) & np.uint32(1)
    rounded = (bits + np.uint32(0x7FFF) + lsb) & np.uint32(0xFFFF0000)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are already bf16-exact."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> np.uint32(16)).astype(np.uint16)


def normal(seed: int, name: str, shape, mean=0.0, std=1.0) -> np.ndarray:
    g = _rng(seed, name)
    out = g.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        out *= np.float32(std)
    if mean != 0.0:
        out += np.float32(mean)
    return out


def uniform(seed: int, name: str, shape, lo: float, hi: float) -> np.ndarray:
    g = _rng(seed, name)
    return (lo + (hi - lo) * g.random(size=shape)).astype(np.float32)


def inverse_softplus_dt_bias(seed: int, name: str, n: int) -> np.ndarray:
    """bias = log(expm1(dt0)) with dt0 ~ logUniform[1e-3, 1e-1], so that
    softplus(bias) = dt0 (the usual Mamba step-size initialisation)."""
    g = _rng(seed, name)
    dt0 = np.exp(g.uniform(math.log(1e-3), math.log(1e-1), size=n))
    return np.log(np.expm1(dt0)).astype(np.float32)


# ---------------------------------------------------------------------------
# Mamba-1 inputs
# ---------------------------------------------------------------------------

def mamba1_inputs(cfg: Mamba1Config, seed: int = 0, batch=None, dim=None,
                  dstate=None, seqlen=None) -> Dict[str, Optional[np.ndarray]]:
    """Inputs for ssm_selective_scan_fwd as float32 numpy arrays (bf16-exact
    when cfg.dtype == "bf16").  Sizes can be overridden for smaller cases.

    u, z ~ N(0,1); delta_raw ~ N(delta_mean, delta_std); B, C, D ~ N(0,1);
    A[d,n] = -(n+1) (the S4D-real pattern) in float32.
    """
    b = cfg.batch if batch is None else batch
    d = cfg.dim if dim is None else dim
    n = cfg.dstate if dstate is None else dstate
    L = cfg.seqlen if seqlen is None else seqlen
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)
    out: Dict[str, Optional[np.ndarray]] = {}
    out["u"] = rnd(normal(seed, "u", (b, d, L)))
    out["delta"] = rnd(normal(seed, "delta", (b, d, L), cfg.delta_mean, cfg.delta_std))
    out["z"] = rnd(normal(seed, "z", (b, d, L))) if cfg.gate else None
    out["B"] = rnd(normal(seed, "B", (b, n, L)))
    out["C"] = rnd(normal(seed, "C", (b, n, L)))
    out["D"] = normal(seed, "D", (d,)) if cfg.use_D else None
    out["A"] = np.ascontiguousarray(
        np.broadcast_to(-(np.arange(n, dtype=np.float32) + 1.0), (d, n)))
    out["delta_bias"] = inverse_softplus_dt_bias(seed, "dt0", d) if cfg.delta_bias else None
    return out


def sample_rows(seed: int, nrows_total: int, count: int) -> np.ndarray:
    """Seeded subset of flat row indices (sorted, distinct)."""
    g = _rng(seed, "rows")
    count = min(count, nrows_total)
    return np.sort(g.choice(nrows_total, size=count, replace=False)).astype(np.int64)


# ---------------------------------------------------------------------------
# SSD (Mamba-2) inputs
# ---------------------------------------------------------------------------

def ssd_inputs(cfg: SSDConfig, seed: int = 0, batch=None, seqlen=None,
               nheads=None, headdim=None, dstate=None, ngroups=None):
    """x ~ N(0,1) [b,L,h,P]; dt_raw ~ N(0,1) [b,L,h]; dt_bias = inverse
    softplus of logU[1e-3,1e-1] per head; A_h = -U[1,16]; B, C ~ N(0,1)/sqrt(N)
    [b,L,g,N]; D ~ N(0,1) per head."""
    b = cfg.batch if batch is None else batch
    L = cfg.seqlen if seqlen is None else seqlen
    h = cfg.nheads if nheads is None else nheads
    p = cfg.headdim if headdim is None else headdim
    n = cfg.dstate if dstate is None else dstate
    g = cfg.ngroups if ngroups is None else ngroups
    rnd = round_bf16 if cfg.dtype == "bf16" else (lambda a: a)
    scale = np.float32(1.0 / math.sqrt(n))
    return {
        "x": rnd(normal(seed, "x", (b, L, h, p))),
        "dt": rnd(normal(seed, "dt", (b, L, h))),
        "A": -uniform(seed, "A", (h,), 1.0, 16.0),
        "B": rnd(normal(seed, "B", (b, L, g, n)) * scale),
        "C": rnd(normal(seed, "C", (b, L, g, n)) * scale),
        "D": normal(seed, "D", (h,)),
        "dt_bias": inverse_softplus_dt_bias(seed, "dt0", h),
    }


# ---------------------------------------------------------------------------
# Upload helpers (plumbing: numpy -> torch device tensors)
# ---------------------------------------------------------------------------

def to_device(arr: Optional[np.ndarray], dtype: str, device="cuda"):
    """float32 numpy array -> torch tensor on `device` in "f32" or "bf16"
    (bf16 arrays must already be bf16-exact; the bits are copied as-is)."""
    if arr is None:
        return None
    import torch
    if dtype == "bf16":
        bits = bf16_bits(arr).view(np.int16)
        return torch.from_numpy(bits).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(device)


def to_host_f64(t) -> np.ndarray:
    """torch tensor (f32 or bf16, any device) -> float64 numpy array."""
    import torch
    return t.detach().to("cpu", torch.float32).numpy().astype(np.float64)
