"""Seeded synthetic inputs for the MATE core.

This module is the only code the GPU path and the CPU oracle have in common,
and it holds none of the method's arithmetic: it draws random tensors with the
distributions a workload names and rounds them to the storage dtype.

Recipe (reproducible, parallel):
  * each tensor is drawn flat, in canonical channels-last order, in blocks of
    2**22 elements; block j of tensor k uses ``numpy.random.default_rng([seed, k, j])``;
  * tensor ids: X=0, B=1, C=2, dt=3, A=4, D=5, Q=6, K=7, V=8;
  * X, B, C, Q, K, V ~ N(0, 1), divided by sqrt(last dim) for scaled workloads;
    dt = softplus(N(mu, sigma)); A = -exp(U(0, a_hi)); D ~ N(0, 1);
  * draws are float64, cast to float32, then rounded to bfloat16 (round to
    nearest even) for bf16 workloads; dt, A and D always stay float32.
The float32 view of a bf16 tensor holds exactly the rounded values, so the
oracle sees the same numbers the GPU does.
"""
from __future__ import annotations

import concurrent.futures as _cf
import os
from dataclasses import dataclass

import numpy as np

from .workloads import Workload

BLOCK = 1 << 22
TENSOR_IDS = {"x": 0, "B": 1, "C": 2, "dt": 3, "A": 4, "D": 5, "q": 6, "k": 7, "v": 8}


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except Exception:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _draw(seed: int, tid: int, n: int, kind: str, transform) -> np.ndarray:
    out = np.empty(n, dtype=np.float32)

    def blk(j):
        lo, hi = j * BLOCK, min(n, (j + 1) * BLOCK)
        rng = np.random.default_rng([seed, tid, j])
        z = rng.standard_normal(hi - lo) if kind == "normal" else rng.random(hi - lo)
        out[lo:hi] = transform(z)

    nblk = (n + BLOCK - 1) // BLOCK
    if nblk <= 1:
        for j in range(nblk):
            blk(j)
    else:
        with _cf.ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(blk, range(nblk)))
    return out


@dataclass
class Tensor:
    """One input tensor: float32 values and the bytes the device receives."""

    f32: np.ndarray | None      # exact values (None when not kept)
    dev: np.ndarray             # float32 array, or uint16 bf16 bit patterns

    @property
    def shape(self):
        return self.dev.shape


def _tensor(wl: Workload, name: str, shape, kind: str, transform, low_precision: bool, keep_f32: bool):
    n = int(np.prod(shape))
    vals = _draw(wl.seed, TENSOR_IDS[name], n, kind, transform).reshape(shape)
    if low_precision and wl.dtype == "bf16":
        bits = f32_to_bf16_bits(vals)
        del vals
        return Tensor(bf16_bits_to_f32(bits) if keep_f32 else None, bits)
    return Tensor(vals if keep_f32 else None, vals)


def make_ssd_inputs(wl: Workload, keep_f32: bool = True) -> dict:
    d = wl.dist
    b, T, H, W = wl.grid
    sx = 1.0 / np.sqrt(wl.headdim) if d.scaled else 1.0
    sb = 1.0 / np.sqrt(wl.d_state) if d.scaled else 1.0
    out = {}
    out["x"] = _tensor(wl, "x", (b, T, H, W, wl.nheads, wl.headdim), "normal", lambda z: z * sx, True, keep_f32)
    out["B"] = _tensor(wl, "B", (b, T, H, W, wl.ngroups, wl.d_state), "normal", lambda z: z * sb, True, keep_f32)
    out["C"] = _tensor(wl, "C", (b, T, H, W, wl.ngroups, wl.d_state), "normal", lambda z: z * sb, True, keep_f32)
    out["dt"] = _tensor(wl, "dt", (b, T, H, W, wl.nheads), "normal",
                        lambda z: np.logaddexp(0.0, d.dt_mu + d.dt_sigma * z), False, True)
    out["A"] = _tensor(wl, "A", (wl.nheads,), "uniform", lambda u: -np.exp(d.a_hi * u), False, True)
    out["D"] = _tensor(wl, "D", (wl.nheads,), "normal", lambda z: z, False, True)
    return out


def make_tesa_inputs(wl: Workload, keep_f32: bool = True) -> dict:
    d = wl.dist
    b, T, H, W = wl.grid
    s = 1.0 / np.sqrt(wl.t_dim) if d.scaled else 1.0
    shape = (b, T, H, W, wl.t_heads, wl.t_dim)
    return {name: _tensor(wl, name, shape, "normal", lambda z: z * s, True, keep_f32) for name in ("q", "k", "v")}
