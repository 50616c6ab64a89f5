"""Layer configurations of the decode workloads (shapes, dtypes, value recipes).

Five layers: a tiny fp32 Mamba-2 head set, a Mamba-2 layer at batch 320 (the
timed workload), a Gated DeltaNet layer, a KDA layer, and a Mamba-2 stress
layer at batch 1024 with a ragged window phase swept over W and mean rank.
"""
from __future__ import annotations

from dataclasses import dataclass, replace
from typing import Optional

FAMILIES = ("mamba2", "gdn", "kda")


@dataclass(frozen=True)
class LayerConfig:
    name: str
    family: str            # "mamba2" | "gdn" | "kda"
    batch: int
    heads: int
    qk_groups: int         # Mamba-2: shared B/C groups; GDN/KDA: == heads
    dk: int                # key/query dim (Mamba-2 d_state)
    dv: int                # value dim (Mamba-2 headdim)
    window: int            # W: one flush every W steps
    mean_rank: int         # Gbar: sum of per-head ranks == mean_rank * heads
    fixed_rank: Optional[int]  # every head gets this rank (no draw) when set
    act: str               # "f32" | "bf16": dtype of q/k/v/o/dt and the ring
    sketch: str            # "f32" | "bf16": dtype of U
    steps: int
    ragged: bool           # per-sequence flush offset uniform in [0, W)
    seed: int
    rank_lo: int = 2
    rank_hi: int = 16
    dense_heads: tuple = ()   # heads set to rank 0 (dense fallback) after the draw

    @property
    def total_rank(self) -> int:
        return self.mean_rank * self.heads

    @property
    def heads_per_group(self) -> int:
        return self.heads // self.qk_groups

    def with_(self, **kw) -> "LayerConfig":
        return replace(self, **kw)


CONFIGS = {
    # Tiny Mamba-2-style layer, everything fp32, rank 4 per head.
    "tiny_m2": LayerConfig(
        name="tiny_m2", family="mamba2", batch=2, heads=4, qk_groups=4,
        dk=16, dv=32, window=4, mean_rank=4, fixed_rank=4, act="f32",
        sketch="f32", steps=32, ragged=False, seed=1),
    # Mamba-2 layer at batch 320: 128 heads, headdim 64, d_state 128,
    # 8 B/C groups, ranks in [2,16] with mean 8.  The timed workload.
    "m2_b320": LayerConfig(
        name="m2_b320", family="mamba2", batch=320, heads=128, qk_groups=8,
        dk=128, dv=64, window=16, mean_rank=8, fixed_rank=None, act="bf16",
        sketch="bf16", steps=256, ragged=False, seed=2),
    # Gated DeltaNet layer: 32 heads, dk = dv = 128, batch 256.
    "gdn_b256": LayerConfig(
        name="gdn_b256", family="gdn", batch=256, heads=32, qk_groups=32,
        dk=128, dv=128, window=16, mean_rank=8, fixed_rank=None, act="bf16",
        sketch="bf16", steps=256, ragged=False, seed=3),
    # KDA layer: as GDN with a per-channel decay g in (0.85, 1)^dk.
    "kda_b256": LayerConfig(
        name="kda_b256", family="kda", batch=256, heads=32, qk_groups=32,
        dk=128, dv=128, window=16, mean_rank=8, fixed_rank=None, act="bf16",
        sketch="bf16", steps=256, ragged=False, seed=4),
    # Mamba-2 stress layer at batch 1024, ragged window phase.  The sweep
    # over W in {8,16,32} x mean rank in {4,8,16} is made by sweep_configs.
    "m2_stress_b1024": LayerConfig(
        name="m2_stress_b1024", family="mamba2", batch=1024, heads=128,
        qk_groups=8, dk=128, dv=64, window=16, mean_rank=8, fixed_rank=None,
        act="bf16", sketch="bf16", steps=512, ragged=True, seed=5),
}

STRESS_WINDOWS = (8, 16, 32)
STRESS_RANKS = (4, 8, 16)


def sweep_configs():
    """The nine stress sweep points; seed = 5 + 100 * sweep index."""
    base = CONFIGS["m2_stress_b1024"]
    out = []
    idx = 0
    for w in STRESS_WINDOWS:
        for g in STRESS_RANKS:
            out.append(base.with_(name=f"m2_stress_b1024_w{w}_g{g}", window=w,
                                  mean_rank=g, seed=base.seed + 100 * idx))
            idx += 1
    return out


def get_config(name: str) -> LayerConfig:
    if name in CONFIGS:
        return CONFIGS[name]
    for c in sweep_configs():
        if c.name == name:
            return c
    raise KeyError(name)
