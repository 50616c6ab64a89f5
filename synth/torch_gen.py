"""The same counter-based generator and input recipes as ``synth.gen``,
evaluated with torch on any device (used to fill large device buffers).

Integer streams and uniforms are bit-identical to ``synth.gen``.  Normals go
through fp64 log/cos, which may differ from numpy's in the last fp64 bit, so
a stored (rounded) value can in rare cases differ by one unit in its last
place; callers that compare against the oracle overwrite the compared
sequences with ``synth.gen`` values.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from . import gen
from .configs import LayerConfig

_TWO64 = 1 << 64


def _s64(x: int) -> int:
    x &= _TWO64 - 1
    return x - _TWO64 if x >= (1 << 63) else x


_GAMMA = _s64(int(gen.GAMMA))
_M1 = _s64(0xBF58476D1CE4E5B9)
_M2 = _s64(0x94D049BB133111EB)


def _lsr(z: torch.Tensor, s: int) -> torch.Tensor:
    return (z >> s) & ((1 << (64 - s)) - 1)


def mix64(z: torch.Tensor) -> torch.Tensor:
    z = (z ^ _lsr(z, 30)) * _M1
    z = (z ^ _lsr(z, 27)) * _M2
    return z ^ _lsr(z, 31)


def uniform(seed: int, stream: int, counters: torch.Tensor) -> torch.Tensor:
    key = _s64(int(gen.stream_key(seed, stream)))
    x = mix64(key + (counters + 1) * _GAMMA)
    return _lsr(x, 11).to(torch.float64) * (2.0 ** -53)


def normal(seed: int, stream: int, counters: torch.Tensor) -> torch.Tensor:
    u1 = 1.0 - uniform(seed, stream, counters * 2)
    u2 = uniform(seed, stream, counters * 2 + 1)
    return torch.sqrt(-2.0 * torch.log(u1)) * torch.cos(2.0 * math.pi * u2)


def _store(x: torch.Tensor, dtype: str) -> torch.Tensor:
    x32 = x.to(torch.float32)
    return x32 if dtype == "f32" else x32.to(torch.bfloat16)


def initial_state(cfg: LayerConfig, b0: int, b1: int, device) -> torch.Tensor:
    """S0 of sequences b0..b1-1 (all heads), fp32 [b][H][dk][dv]."""
    per_b = cfg.heads * cfg.dk * cfg.dv
    cnt = torch.arange(b0 * per_b, b1 * per_b, dtype=torch.int64, device=device)
    S = 0.1 * normal(cfg.seed, gen.STREAM["S0"], cnt)
    return S.to(torch.float32).reshape(b1 - b0, cfg.heads, cfg.dk, cfg.dv)


def _counters(t: int, shape, device) -> torch.Tensor:
    numel = int(np.prod(shape))
    return torch.arange(t * numel, (t + 1) * numel, dtype=torch.int64, device=device).reshape(shape)


def step_inputs(cfg: LayerConfig, t: int, device):
    """Step t's inputs for every sequence as torch tensors in their storage
    dtypes: (q, k, v, gate, beta); recipes as ``synth.gen.make_step_inputs``."""
    B, H, G, dk, dv = cfg.batch, cfg.heads, cfg.qk_groups, cfg.dk, cfg.dv
    s = cfg.seed
    qn = normal(s, gen.STREAM["q"], _counters(t, (B, G, dk), device))
    kn = normal(s, gen.STREAM["k"], _counters(t, (B, G, dk), device))
    vn = normal(s, gen.STREAM["v"], _counters(t, (B, H, dv), device))
    if cfg.family == "mamba2":
        u = uniform(s, gen.STREAM["gate"], _counters(t, (B, H), device))
        gate = 0.001 + (0.1 - 0.001) * u
        return (_store(qn / math.sqrt(dk), cfg.act), _store(kn / math.sqrt(dk), cfg.act),
                _store(vn / math.sqrt(dk), cfg.act), _store(gate, cfg.act), None)
    q = qn / torch.linalg.norm(qn, dim=-1, keepdim=True)
    k = kn / torch.linalg.norm(kn, dim=-1, keepdim=True)
    v = vn / math.sqrt(dv)
    beta = uniform(s, gen.STREAM["beta"], _counters(t, (B, H), device))
    if cfg.family == "gdn":
        gate = 0.9 + 0.1 * uniform(s, gen.STREAM["gate"], _counters(t, (B, H), device))
    else:
        gate = 0.85 + 0.15 * uniform(s, gen.STREAM["gate"], _counters(t, (B, H, dk), device))
        gate = torch.where(gate <= 0.85, torch.full_like(gate, 0.85 + 0.15 * 2.0 ** -24), gate)
    return (_store(q, cfg.act), _store(k, cfg.act), _store(v, cfg.act),
            gate.to(torch.float32), beta.to(torch.float32))
