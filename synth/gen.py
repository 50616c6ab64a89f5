"""Counter-based generators and the layer/step input recipes.

All arrays returned here hold *stored* values: numbers exactly representable
in the dtype the layer stores them in (fp32, or bf16 reached by rounding to
nearest-even from fp32).  They are returned as float64 arrays (which hold
those values exactly) so that the fp64 oracle and the GPU path read the same
numbers; ``bf16_bits`` / ``float32`` views give the storage encoding.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

from .configs import LayerConfig

# SplitMix64 constants (Steele, Lea, Flood 2014).
GAMMA = np.uint64(0x9E3779B97F4A7C15)
_M1 = np.uint64(0xBF58476D1CE4E5B9)
_M2 = np.uint64(0x94D049BB133111EB)
_S30, _S27, _S31, _S11 = (np.uint64(s) for s in (30, 27, 31, 11))

# Stream ids: one per tensor so that no two tensors share random numbers.
STREAM = {
    "S0": 1, "A": 2, "basis": 3, "phase": 4,
    "q": 10, "k": 11, "v": 12, "gate": 13, "beta": 14,
}


def mix64(z: np.ndarray) -> np.ndarray:
    """SplitMix64 output function (wrapping uint64 arithmetic)."""
    z = np.asarray(z, dtype=np.uint64)
    with np.errstate(over="ignore"):
        z = (z ^ (z >> _S30)) * _M1
        z = (z ^ (z >> _S27)) * _M2
    return z ^ (z >> _S31)


def stream_key(seed: int, stream: int) -> np.uint64:
    with np.errstate(over="ignore"):
        s = mix64(np.array([np.uint64(stream) * GAMMA], dtype=np.uint64))[0]
        return mix64(np.array([np.uint64(seed) ^ s], dtype=np.uint64))[0]


def _raw(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    key = stream_key(seed, stream)
    c = np.asarray(counters, dtype=np.uint64)
    with np.errstate(over="ignore"):
        return mix64(key + (c + np.uint64(1)) * GAMMA)


_CHUNK = 1 << 18
_POOL = None


def _threads() -> int:
    n = int(os.environ.get("SYNTH_THREADS", "0") or 0)
    return n if n > 0 else min(16, os.cpu_count() or 1)


def _chunked(fn, counters: np.ndarray) -> np.ndarray:
    """Apply an elementwise generator to counters, split over threads for
    large arrays (numpy releases the GIL inside its loops).  The result is
    independent of the split."""
    global _POOL
    c = np.ascontiguousarray(np.asarray(counters, dtype=np.uint64))
    flat = c.reshape(-1)
    if flat.size <= 2 * _CHUNK or _threads() == 1:
        return fn(flat).reshape(c.shape)
    if _POOL is None:
        _POOL = ThreadPoolExecutor(max_workers=_threads())
    out = np.empty(flat.size, dtype=np.float64)

    def work(lo):
        out[lo:lo + _CHUNK] = fn(flat[lo:lo + _CHUNK])

    list(_POOL.map(work, range(0, flat.size, _CHUNK)))
    return out.reshape(c.shape)


def _uniform(seed, stream, c):
    return (_raw(seed, stream, c) >> _S11).astype(np.float64) * (2.0 ** -53)


def _normal(seed, stream, c):
    u1 = 1.0 - _uniform(seed, stream, c * np.uint64(2))          # (0, 1]
    u2 = _uniform(seed, stream, c * np.uint64(2) + np.uint64(1))
    return np.sqrt(-2.0 * np.log(u1)) * np.cos(2.0 * np.pi * u2)


def uniform(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """U[0,1) from the top 53 bits of the counter's SplitMix64 value."""
    return _chunked(lambda c: _uniform(seed, stream, c), counters)


def normal(seed: int, stream: int, counters: np.ndarray) -> np.ndarray:
    """N(0,1) by Box-Muller from uniforms at counters 2c and 2c+1."""
    return _chunked(lambda c: _normal(seed, stream, c), counters)


# ---------------------------------------------------------------- rounding
def round_f32(x: np.ndarray) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """bf16 encoding (uint16) of x: round to fp32, then nearest-even to bf16."""
    f = np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32))
    u = f.view(np.uint32).astype(np.uint64)
    u = u + np.uint64(0x7FFF) + ((u >> np.uint64(16)) & np.uint64(1))
    return ((u >> np.uint64(16)) & np.uint64(0xFFFF)).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    u = np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32)


def round_bf16(x: np.ndarray) -> np.ndarray:
    return bf16_bits_to_f32(bf16_bits(x)).astype(np.float64)


def round_to(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "f32":
        return round_f32(x)
    if dtype == "bf16":
        return round_bf16(x)
    raise ValueError(dtype)


# ------------------------------------------------------------ rank table
def draw_ranks(cfg: LayerConfig) -> np.ndarray:
    """Per-head sketch ranks r_h.

    Fixed-rank layers give every head ``fixed_rank``.  Otherwise: draw r_h
    i.i.d. uniform in {lo..hi} with default_rng(seed); while the sum differs
    from mean_rank*heads, pick a head uniformly and step it by +-1 toward the
    target when that stays inside [lo, hi].
    """
    H = cfg.heads
    if cfg.fixed_rank is not None:
        return np.full(H, cfg.fixed_rank, dtype=np.int32)
    lo, hi = cfg.rank_lo, cfg.rank_hi
    target = cfg.mean_rank * H
    if not (lo * H <= target <= hi * H):
        raise ValueError("mean rank outside the per-head rank range")
    rng = np.random.default_rng(cfg.seed)
    r = rng.integers(lo, hi + 1, size=H).astype(np.int64)
    while int(r.sum()) != target:
        i = int(rng.integers(0, H))
        step = 1 if int(r.sum()) < target else -1
        if lo <= r[i] + step <= hi:
            r[i] += step
    return r.astype(np.int32)


def rank_offsets(ranks: np.ndarray) -> np.ndarray:
    off = np.zeros(len(ranks) + 1, dtype=np.int32)
    off[1:] = np.cumsum(ranks, dtype=np.int64).astype(np.int32)
    return off


def make_basis(cfg: LayerConfig, ranks: np.ndarray) -> np.ndarray:
    """Pt [R][dk] float64 holding fp32 values: rows off_h..off_h+r_h-1 are the
    columns of P_h, the Q factor of the reduced QR of a seeded dk x r_h
    Gaussian (QR in fp64, stored in fp32)."""
    off = rank_offsets(ranks)
    Pt = np.zeros((int(off[-1]), cfg.dk), dtype=np.float64)
    for h, r in enumerate(ranks):
        r = int(r)
        if r == 0:
            continue
        cnt = (np.arange(cfg.dk * r, dtype=np.uint64)
               + np.uint64(h * cfg.dk * cfg.dk))
        G = normal(cfg.seed, STREAM["basis"], cnt).reshape(cfg.dk, r)
        Q, _ = np.linalg.qr(G, mode="reduced")
        Pt[off[h]:off[h] + r] = Q.T
    return round_f32(Pt)


def phase_offsets(cfg: LayerConfig) -> np.ndarray:
    """Flush offset o_b per sequence: sequence b flushes at steps t = o_b mod W.
    Aligned layers use o_b = W-1 (first flush at step W-1)."""
    W = cfg.window
    if not cfg.ragged:
        return np.full(cfg.batch, W - 1, dtype=np.int32)
    u = uniform(cfg.seed, STREAM["phase"], np.arange(cfg.batch, dtype=np.uint64))
    return np.minimum((u * W).astype(np.int64), W - 1).astype(np.int32)


def identity_gate(family: str) -> float:
    """Gate value of an identity ring entry (k = v = 0, beta = 0): Mamba-2
    dt = 0 (decay exp(0) = 1), GDN alpha = 1, KDA g = 1."""
    return 0.0 if family == "mamba2" else 1.0


# ------------------------------------------------------------- layer state
@dataclass
class LayerInputs:
    cfg: LayerConfig
    ranks: np.ndarray        # int32 [H]
    offsets: np.ndarray      # int32 [H+1]
    Pt: np.ndarray           # float64 (fp32 values) [R][dk]
    C: np.ndarray            # float64 (fp32 values) [R][dk]; C_h = P_h^T
    A: Optional[np.ndarray]  # Mamba-2: float64 (fp32 values) [H]
    phase: np.ndarray        # int32 [B] flush offsets
    count0: np.ndarray       # int32 [B][H] initial ring fill (identity pad)


def make_layer_inputs(cfg: LayerConfig) -> LayerInputs:
    ranks = draw_ranks(cfg)
    if cfg.dense_heads:                       # dense-fallback heads: rank 0
        ranks = ranks.copy()
        ranks[list(cfg.dense_heads)] = 0
    off = rank_offsets(ranks)
    Pt = make_basis(cfg, ranks)
    A = None
    if cfg.family == "mamba2":
        A = round_f32(uniform(cfg.seed, STREAM["A"],
                              np.arange(cfg.heads, dtype=np.uint64)))
    phase = phase_offsets(cfg)
    count0 = np.repeat((cfg.window - 1 - phase)[:, None], cfg.heads, axis=1)
    return LayerInputs(cfg=cfg, ranks=ranks, offsets=off, Pt=Pt, C=Pt.copy(),
                       A=A, phase=phase, count0=count0.astype(np.int32))


def initial_state(cfg: LayerConfig, b_idx: Optional[Sequence[int]] = None,
                  h_idx: Optional[Sequence[int]] = None) -> np.ndarray:
    """S0 ~ N(0, 0.1^2) in fp32 for the selected tiles: [len(b)][len(h)][dk][dv]
    (all sequences / heads by default).  Counter of S0[b][h][m][n] is the flat
    index in the full [B][H][dk][dv] tensor."""
    b_idx = np.arange(cfg.batch) if b_idx is None else np.asarray(b_idx)
    h_idx = np.arange(cfg.heads) if h_idx is None else np.asarray(h_idx)
    tile = cfg.dk * cfg.dv
    base = (b_idx[:, None].astype(np.uint64) * np.uint64(cfg.heads)
            + h_idx[None, :].astype(np.uint64)) * np.uint64(tile)
    cnt = base[:, :, None] + np.arange(tile, dtype=np.uint64)[None, None, :]
    S = 0.1 * normal(cfg.seed, STREAM["S0"], cnt)
    return round_f32(S).reshape(len(b_idx), len(h_idx), cfg.dk, cfg.dv)


# ------------------------------------------------------------- step inputs
@dataclass
class StepInputs:
    """Inputs of one decode step for the selected sequences (stored values).

    q, k: [b][G][dk]; v: [b][H][dv]; gate: Mamba-2 dt [b][H], GDN alpha
    [b][H], KDA g [b][H][dk]; beta: GDN/KDA [b][H] (None for Mamba-2)."""
    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    gate: np.ndarray
    beta: Optional[np.ndarray]


def _step_counters(t: int, full_shape, b_idx: np.ndarray) -> np.ndarray:
    per_b = int(np.prod(full_shape[1:]))
    numel = full_shape[0] * per_b
    base = np.uint64(t) * np.uint64(numel) + b_idx.astype(np.uint64) * np.uint64(per_b)
    cnt = base[:, None] + np.arange(per_b, dtype=np.uint64)[None, :]
    return cnt.reshape((len(b_idx),) + tuple(full_shape[1:]))


def make_step_inputs(cfg: LayerConfig, t: int,
                     b_idx: Optional[Sequence[int]] = None) -> StepInputs:
    """Inputs of decode step t (0-based).

    Mamba-2: q (C), k (B), v (x) ~ N(0,1)/sqrt(dk) in the activation dtype;
    dt ~ U[0.001, 0.1] in the activation dtype.
    GDN/KDA: q, k ~ N(0,1) normalised to unit L2 norm in fp64, then stored;
    v ~ N(0,1)/sqrt(dv); beta ~ U[0,1] fp32; GDN alpha ~ U[0.9,1] fp32; KDA
    g ~ U(0.85,1) per channel fp32.
    """
    b_idx = np.arange(cfg.batch) if b_idx is None else np.asarray(b_idx)
    B, H, G, dk, dv = cfg.batch, cfg.heads, cfg.qk_groups, cfg.dk, cfg.dv
    s = cfg.seed
    qn = normal(s, STREAM["q"], _step_counters(t, (B, G, dk), b_idx))
    kn = normal(s, STREAM["k"], _step_counters(t, (B, G, dk), b_idx))
    vn = normal(s, STREAM["v"], _step_counters(t, (B, H, dv), b_idx))
    if cfg.family == "mamba2":
        q = qn / np.sqrt(dk)
        k = kn / np.sqrt(dk)
        v = vn / np.sqrt(dk)
        u = uniform(s, STREAM["gate"], _step_counters(t, (B, H), b_idx))
        gate = 0.001 + (0.1 - 0.001) * u
        return StepInputs(q=round_to(q, cfg.act), k=round_to(k, cfg.act),
                          v=round_to(v, cfg.act), gate=round_to(gate, cfg.act),
                          beta=None)
    q = qn / np.linalg.norm(qn, axis=-1, keepdims=True)
    k = kn / np.linalg.norm(kn, axis=-1, keepdims=True)
    v = vn / np.sqrt(dv)
    beta = uniform(s, STREAM["beta"], _step_counters(t, (B, H), b_idx))
    if cfg.family == "gdn":
        u = uniform(s, STREAM["gate"], _step_counters(t, (B, H), b_idx))
        gate = 0.9 + 0.1 * u
    elif cfg.family == "kda":
        u = uniform(s, STREAM["gate"], _step_counters(t, (B, H, dk), b_idx))
        gate = 0.85 + 0.15 * u
        # the interval is open at 0.85: a draw of exactly 0 moves inward
        gate = np.where(gate <= 0.85, 0.85 + 0.15 * 2.0 ** -24, gate)
    else:
        raise ValueError(cfg.family)
    return StepInputs(q=round_to(q, cfg.act), k=round_to(k, cfg.act),
                      v=round_to(v, cfg.act), gate=round_f32(gate),
                      beta=round_f32(beta))
