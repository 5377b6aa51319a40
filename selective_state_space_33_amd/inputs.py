"""Seeded synthetic inputs for the selective scan (numpy only).

This module only draws random numbers and rounds them to the storage dtype;
it holds none of the scan's arithmetic, so both the GPU path and the CPU
oracle can be fed from it.

Workloads are named by what they are.  Every draw comes from one
``numpy.random.Generator(PCG64(seed))`` in a fixed order:
u (or the sinusoid parameters and noise), z (if gated), delta_raw, B, C, the
bias uniforms, and h0 (decode only).  Values are drawn in float32, and
rounded to bfloat16 (round to nearest, ties to even) where the workload
stores bf16, so both sides see the identical values.
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    op: str            # "scan" or "decode"
    batch: int
    L: int             # 1 for decode
    dim: int
    dstate: int
    dtype: str         # "f32" or "bf16": storage type of u, delta, z, B, C, y
    gate: bool         # z gate present
    u_kind: str = "gauss"                      # "gauss" or "sinusoids"
    bias_range: tuple = (1e-3, 0.1)            # softplus(bias) ~ U[lo, hi]
    h0_std: float = 0.1                        # decode prior state scale

    @property
    def updates(self) -> int:
        """State updates per call: batch * L * dim * dstate."""
        return self.batch * self.L * self.dim * self.dstate

    def scaled(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 scan, a bf16 decode step, a Mamba-130M-shaped
# and a Mamba-2.8B-shaped bf16 layer scan, and a long fp32 audio-style scan.
WORKLOADS = {
    "tiny_fp32": Workload("tiny_fp32", "scan", 1, 256, 16, 4, "f32", True),
    "decode_bf16": Workload("decode_bf16", "decode", 256, 1, 5120, 16, "bf16", True),
    "mamba130m_bf16": Workload("mamba130m_bf16", "scan", 8, 2048, 1536, 16, "bf16", True),
    "mamba2p8b_bf16": Workload("mamba2p8b_bf16", "scan", 4, 4096, 5120, 16, "bf16", True),
    "long_audio_fp32": Workload("long_audio_fp32", "scan", 1, 1 << 20, 64, 16, "f32", False,
                                u_kind="sinusoids", bias_range=(1e-4, 1e-2)),
}


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bfloat16 (ties to even); returns float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    lsb = (bits >> 16) & 1
    rounded = ((bits + 0x7FFF + lsb) & 0xFFFF0000).astype(np.uint32)
    return rounded.view(np.float32)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Upper 16 bits of float32 values that are already bf16-representable."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    return (x.view(np.uint32) >> 16).astype(np.uint16)


def _store(x: np.ndarray, dtype: str) -> np.ndarray:
    x = x.astype(np.float32, copy=False)
    return round_to_bf16(x) if dtype == "bf16" else x


def _sinusoids(rng: np.random.Generator, L: int, dim: int, batch: int) -> np.ndarray:
    """Sum of 4 seeded sinusoids per channel plus Gaussian noise, unit variance.

    Frequencies are log-uniform in [1e-4, 0.25] cycles/sample, phases uniform
    in [0, 2 pi), each amplitude sqrt(0.4) (variance 0.2 each, 0.8 in total),
    and the noise is N(0, 0.2), so the total variance is 1.
    """
    freqs = np.exp(rng.uniform(np.log(1e-4), np.log(0.25), size=(batch, dim, 4)))
    phases = rng.uniform(0.0, 2.0 * np.pi, size=(batch, dim, 4))
    amp = np.sqrt(0.4)
    out = np.empty((batch, L, dim), dtype=np.float32)
    t = np.arange(L, dtype=np.float64)
    for b in range(batch):
        for d in range(dim):
            s = np.zeros(L, dtype=np.float64)
            for k in range(4):
                s += amp * np.sin(2.0 * np.pi * freqs[b, d, k] * t + phases[b, d, k])
            out[b, :, d] = s
    out += rng.standard_normal(out.shape, dtype=np.float32) * np.float32(np.sqrt(0.2))
    return out


def make_inputs(w: Workload, seed: int = 0) -> dict:
    """Draw all inputs of a workload.

    Returns a dict of float32 numpy arrays (bf16-representable where the
    workload stores bf16): u, delta (the raw delta), z (or None), B, C, A,
    D, delta_bias, and for decode also h0.  Scan tensors are
    [batch, L, dim] / [batch, L, dstate]; decode drops the L axis.
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    bt, L, dim, N = w.batch, w.L, w.dim, w.dstate
    io_shape = (bt, dim) if w.op == "decode" else (bt, L, dim)
    bc_shape = (bt, N) if w.op == "decode" else (bt, L, N)

    if w.u_kind == "sinusoids":
        assert w.op == "scan"
        u = _sinusoids(rng, L, dim, bt)
    else:
        u = rng.standard_normal(io_shape, dtype=np.float32)
    z = rng.standard_normal(io_shape, dtype=np.float32) if w.gate else None
    delta = rng.standard_normal(io_shape, dtype=np.float32)
    B = rng.standard_normal(bc_shape, dtype=np.float32)
    C = rng.standard_normal(bc_shape, dtype=np.float32)
    lo, hi = w.bias_range
    # delta_bias = log(expm1(U)) is the inverse softplus of a uniform draw,
    # so that softplus(bias) is uniform in [lo, hi].
    bias = np.log(np.expm1(rng.uniform(lo, hi, size=dim))).astype(np.float32)
    A = np.broadcast_to(-(np.arange(N, dtype=np.float32) + 1.0), (dim, N)).copy()
    D = np.ones(dim, dtype=np.float32)
    out = {
        "u": _store(u, w.dtype),
        "z": _store(z, w.dtype) if z is not None else None,
        "delta": _store(delta, w.dtype),
        "B": _store(B, w.dtype),
        "C": _store(C, w.dtype),
        "A": A,
        "D": D,
        "delta_bias": bias,
    }
    if w.op == "decode":
        out["h0"] = (rng.standard_normal((bt, dim, N), dtype=np.float32) * np.float32(w.h0_std))
    return out


def random_scan_inputs(rng: np.random.Generator, batch: int, L: int, dim: int, dstate: int,
                       dtype: str = "f32", gate: bool = True, A: Optional[np.ndarray] = None) -> dict:
    """Small random scan inputs with a general (not structured) A, for edge-case tests.

    A[d, n] is drawn uniformly in [-2, -0.05] independently per (d, n) unless given.
    """
    u = rng.standard_normal((batch, L, dim), dtype=np.float32)
    z = rng.standard_normal((batch, L, dim), dtype=np.float32) if gate else None
    delta = rng.standard_normal((batch, L, dim), dtype=np.float32)
    B = rng.standard_normal((batch, L, dstate), dtype=np.float32)
    C = rng.standard_normal((batch, L, dstate), dtype=np.float32)
    bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, size=dim))).astype(np.float32)
    if A is None:
        A = rng.uniform(-2.0, -0.05, size=(dim, dstate)).astype(np.float32)
    D = rng.uniform(0.5, 1.5, size=dim).astype(np.float32)
    return {
        "u": _store(u, dtype), "z": _store(z, dtype) if z is not None else None,
        "delta": _store(delta, dtype), "B": _store(B, dtype), "C": _store(C, dtype),
        "A": np.ascontiguousarray(A, dtype=np.float32), "D": D, "delta_bias": bias,
    }


def packed_offsets(rng: np.random.Generator, total: int, mean_len: float, sigma: float = 1.0) -> list:
    """Seeded cut of `total` tokens into packed sequences: cumulative offsets [0, ..., total].

    Lengths are log-normal with median `mean_len` * exp(-sigma^2 / 2) (mean `mean_len`), at least 1 token,
    so a row mixes a few long sequences with many short ones; the last length is clipped to fit."""
    cu = [0]
    mu = np.log(mean_len) - sigma * sigma / 2
    while cu[-1] < total:
        n = max(1, int(round(rng.lognormal(mu, sigma))))
        cu.append(min(total, cu[-1] + n))
    return cu


# The Mamba-2 (SSD) layer shaped like the 2.7B model: d_inner 5120 as 80 heads of 64 channels, state 128
# (8x the two-term layer's 16), batch 4, L 4096, bf16.
SSD_WORKLOADS = {
    "mamba2_2p7b_bf16": dict(batch=4, L=4096, heads=80, headdim=64, dstate=128, dtype="bf16"),
    "ssd_small_bf16": dict(batch=2, L=300, heads=3, headdim=64, dstate=64, dtype="bf16"),
}


def random_ssd_inputs(rng: np.random.Generator, batch: int, L: int, heads: int, headdim: int, dstate: int,
                      dtype: str = "bf16", gate: bool = True, ngroups: int = 0) -> dict:
    """Seeded inputs of the SSD layer (float32 arrays, bf16-representable where stored as bf16).

    x, z: [batch, L, heads, headdim] ~ N(0, 1); delta (raw): [batch, L, heads] ~ N(0, 1); B, C: [batch, L, dstate]
    (ngroups = 0) or [batch, L, ngroups, dstate] ~ N(0, 1); A: [heads] = -U[1, 16] (a scalar per head); D = 1;
    delta_bias = log(expm1(U[1e-3, 0.1])), so softplus(bias) is uniform in [1e-3, 0.1]."""
    x = rng.standard_normal((batch, L, heads, headdim), dtype=np.float32)
    z = rng.standard_normal((batch, L, heads, headdim), dtype=np.float32) if gate else None
    delta = rng.standard_normal((batch, L, heads), dtype=np.float32)
    bc_shape = (batch, L, dstate) if ngroups == 0 else (batch, L, ngroups, dstate)
    B = rng.standard_normal(bc_shape, dtype=np.float32)
    C = rng.standard_normal(bc_shape, dtype=np.float32)
    A = -rng.uniform(1.0, 16.0, size=heads).astype(np.float32)
    bias = np.log(np.expm1(rng.uniform(1e-3, 0.1, size=heads))).astype(np.float32)
    return {
        "x": _store(x, dtype), "z": _store(z, dtype) if z is not None else None, "delta": _store(delta, dtype),
        "B": _store(B, dtype), "C": _store(C, dtype), "A": A, "D": np.ones(heads, dtype=np.float32),
        "delta_bias": bias,
    }
