"""Byte accounting of the decode path.

Two models:

* ``state_traffic_ratio`` -- the state-access traffic model of the paper's
  App. D ("State memory traffic reduction"): Standard reads and writes the
  full state D every step; ReplaySSM reads D every step and writes D/W;
  SketchSSM reads ((W-1) T_G + D) / W, where T_G is the bf16 sketch plus
  coefficient map, G (K + V) elements, and writes D/W.  Ring traffic and
  sketch writes are excluded, as the appendix states.
* ``window_bytes`` -- the algorithmic bytes the implemented path must move
  per sequence and window: every byte counted once at its minimum (state
  read and written at the flush, sketch written once and read at the W-1
  other steps, ring entries appended once and re-read by later steps of the
  window, step inputs read and outputs written once, basis / coefficient
  rows read once per launch and shared by all sequences).  With the
  state-dependent coefficient map each sequence's map (R x dk, sketch dtype)
  is written at the flush and read at the W-1 other steps, like the sketch,
  and only the basis remains shared.  A dense-fallback head (rank 0) has no
  sketch: its state copy (dk x dv, sketch dtype) is written at the flush and
  read at the W-1 other steps.
"""
from __future__ import annotations

from dataclasses import dataclass

ACT_BYTES = {"f32": 4, "bf16": 2}


def state_traffic_ratio(K: int, V: int, G: int, W: int, method: str = "sketch",
                        state_bytes: int = 4, sketch_bytes: int = 2) -> float:
    """Standard-to-method ratio of per-step state-access bytes (App. D)."""
    D = K * V * state_bytes
    std = 2.0 * D
    if method == "replay":
        return std / (D + D / W)
    if method == "sketch":
        TG = G * (K + V) * sketch_bytes
        return std / (((W - 1) * TG + D) / W + D / W)
    raise ValueError(method)


@dataclass(frozen=True)
class LayerBytes:
    per_window: int          # bytes per window over the whole batch (sketch path)
    per_step: float          # per_window / W
    flush_launch: int        # bytes of one flush launch (aligned phase, whole batch)
    read_launch_avg: float   # average bytes of one non-flush read launch
    full_step: int           # bytes of one standard full-state step
    replay_per_step: float   # ReplaySSM bytes per step, W-amortised
    basis: int               # shared basis rows read by a flush launch


def slot_bytes(family: str, H: int, G: int, dk: int, dv: int, act: str) -> int:
    """Bytes of one ring entry of one sequence (k per group, v, gate, beta)."""
    a = ACT_BYTES[act]
    k = G * dk * a
    v = H * dv * a
    if family == "mamba2":
        gate, beta = H * a, 0
    elif family == "gdn":
        gate, beta = H * 4, H * 4
    else:
        gate, beta = H * dk * 4, H * 4
    return k + v + gate + beta


def layer_bytes(family: str, B: int, H: int, G: int, dk: int, dv: int, W: int, R: int,
                act: str, sketch: str, coef: str = "fixed", dense: int = 0) -> LayerBytes:
    a, u = ACT_BYTES[act], ACT_BYTES[sketch]
    S = H * dk * dv * 4                   # state of one sequence
    Useq = R * dv * u                     # sketch of one sequence
    if coef == "state":                   # the sequence's own map travels with its sketch
        Useq += R * dk * u
    Useq += dense * dk * dv * u           # state copies of dense-fallback heads
    slot = slot_bytes(family, H, G, dk, dv, act)
    q = G * dk * a
    o = H * dv * a
    basis = R * dk * 4                    # Pt or C, shared by all sequences
    ring_reads = W * (W - 1) // 2         # reads of earlier entries over a window
    appends = W - 1                       # entries written to the ring
    per_seq = 2 * S + W * Useq + (ring_reads + appends) * slot + W * (q + slot + o)
    # shared rows: Pt at the flush, plus the fixed C at every read launch
    per_window = B * per_seq + (W if coef == "fixed" else 1) * basis
    # flush launch: S read + write, U write, W entries read, q read, o write, Pt
    flush = B * (2 * S + Useq + W * slot + q + o) + basis
    # the W-1 non-flush reads plus the read at the flush step (append only)
    read_total = per_window - flush
    full = B * (2 * S + q + slot + o)
    # ReplaySSM per window: W state reads, one state write, ring as above
    replay_window = B * (W * S + S + (ring_reads + appends) * slot + W * (q + slot + o))
    return LayerBytes(per_window=per_window, per_step=per_window / W, flush_launch=flush,
                      read_launch_avg=read_total / W, full_step=full,
                      replay_per_step=replay_window / W, basis=basis)


def config_bytes(cfg, R: int, coef: str = "fixed") -> LayerBytes:
    return layer_bytes(cfg.family, cfg.batch, cfg.heads, cfg.qk_groups, cfg.dk, cfg.dv,
                       cfg.window, R, cfg.act, cfg.sketch, coef, len(cfg.dense_heads))
