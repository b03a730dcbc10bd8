"""The five synthetic MATE-core workloads (sizes, dtypes, input distributions).

Plain data: no arithmetic of the method lives here. Widths at the larger grids
follow LinGen-4B (xllm-io review "LinGen: Towards High-Resolution Minute-Length
Text-to-Video Generation ...", section 5.1: 20 heads, embedding 2560); the
pages give no latent grid, window, pooling or chunk sizes, so those are the
stated workload choices.
"""
from __future__ import annotations

from dataclasses import dataclass, field


@dataclass(frozen=True)
class Dist:
    """Input distributions. ``scaled`` divides X, B, C, Q, K, V by sqrt(last dim)."""

    dt_mu: float
    dt_sigma: float
    a_hi: float           # A = -exp(U(0, a_hi))
    scaled: bool


@dataclass(frozen=True)
class Workload:
    name: str
    seed: int
    dtype: str            # "f32" or "bf16" for x, B, C, y, q, k, v, o
    batch: int
    T: int
    H: int
    W: int
    # bidirectional SSD
    nheads: int
    headdim: int
    d_state: int
    ngroups: int
    chunk: int
    pool: tuple           # (pt, ph, pw) or (0, 0, 0)
    # TESA
    t_heads: int
    t_dim: int
    window: tuple
    shift: tuple          # the shift used on odd layers
    dist: Dist
    orders: tuple = (0, 1, 2, 3)
    # layer schedule: list of (order, shifted) pairs for one step
    schedule: tuple = field(default=())

    @property
    def N(self) -> int:
        return self.T * self.H * self.W

    @property
    def grid(self):
        return (self.batch, self.T, self.H, self.W)

    @property
    def R(self) -> int:
        if not any(self.pool):
            return 0
        pt, ph, pw = self.pool
        return (self.T // pt) * (self.H // ph) * (self.W // pw)

    def layer_shift(self, shifted: bool):
        return self.shift if shifted else (0, 0, 0)


_D01 = Dist(dt_mu=-1.0, dt_sigma=0.5, a_hi=1.0, scaled=False)
_D24 = Dist(dt_mu=-2.0, dt_sigma=0.5, a_hi=2.0, scaled=True)

_SCHED4 = ((0, False), (1, True), (2, False), (3, True))

WORKLOADS = {
    0: Workload("tiny-fp32 2x4x4", 0, "f32", 1, 2, 4, 4,
                nheads=2, headdim=16, d_state=8, ngroups=1, chunk=8, pool=(2, 2, 2),
                t_heads=2, t_dim=16, window=(2, 2, 2), shift=(1, 1, 1), dist=_D01,
                schedule=_SCHED4),
    1: Workload("small-bf16 8x16x16", 1, "bf16", 1, 8, 16, 16,
                nheads=16, headdim=64, d_state=64, ngroups=1, chunk=64, pool=(0, 0, 0),
                t_heads=8, t_dim=64, window=(4, 8, 8), shift=(2, 4, 4), dist=_D01,
                schedule=_SCHED4),
    2: Workload("lingen4b-layer 32x32x32", 2, "bf16", 1, 32, 32, 32,
                nheads=80, headdim=64, d_state=128, ngroups=1, chunk=128, pool=(0, 0, 0),
                t_heads=20, t_dim=128, window=(8, 8, 8), shift=(4, 4, 4), dist=_D24,
                orders=(0,), schedule=((0, True),)),
    3: Workload("lingen4b-review 64x32x32", 3, "bf16", 1, 64, 32, 32,
                nheads=80, headdim=64, d_state=128, ngroups=1, chunk=128, pool=(8, 8, 8),
                t_heads=20, t_dim=128, window=(8, 8, 8), shift=(4, 4, 4), dist=_D24,
                schedule=_SCHED4),
    4: Workload("long-grid 128x48x48", 4, "bf16", 1, 128, 48, 48,
                nheads=80, headdim=64, d_state=128, ngroups=1, chunk=128, pool=(8, 8, 8),
                t_heads=20, t_dim=128, window=(8, 8, 8), shift=(4, 4, 4), dist=_D24,
                schedule=_SCHED4),
}
