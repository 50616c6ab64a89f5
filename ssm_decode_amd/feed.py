"""Moves seeded synthetic inputs (``synth``) into a layer's device buffers.

Small layers are filled from the numpy generator; large ones from the same
generator evaluated with torch on the device (``synth.torch_gen``), with
chosen sequences overwritten by numpy values when they must match a host
reference exactly.
"""
from __future__ import annotations

from typing import Optional, Sequence

import numpy as np
import torch

import synth
from synth import torch_gen

from .layer import DecodeLayer, DeviceStep, TORCH_DTYPE


def to_device(x: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    """Stored values (float64 holding fp32 / bf16 numbers) -> device tensor;
    the conversion is exact."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, dtype=np.float64).astype(np.float32)))
    return t.to(device=device).to(TORCH_DTYPE[dtype])


def make_layer(cfg: synth.LayerConfig, li: synth.LayerInputs, device="cuda", coef: str = "fixed",
               ridge: float = 1e-4, pullback: str = "serial") -> DecodeLayer:
    lay = DecodeLayer(cfg.family, cfg.batch, cfg.heads, cfg.qk_groups, cfg.dk, cfg.dv,
                      cfg.window, cfg.act, cfg.sketch, li.offsets, device=device, coef=coef,
                      ridge=ridge, pullback=pullback)
    lay.Pt.copy_(to_device(li.Pt, "f32", device))
    lay.Cmap.copy_(to_device(li.C, "f32", device))
    if li.A is not None:
        lay.A.copy_(to_device(li.A, "f32", device))
    return lay


def fill_state(lay: DecodeLayer, cfg: synth.LayerConfig, exact_seqs: Optional[Sequence[int]] = None,
               numpy_all: bool = False, chunk: int = 32) -> None:
    """S0 for every sequence.  numpy_all: every sequence from the numpy
    generator; otherwise the device generator, then exact_seqs from numpy."""
    B = cfg.batch
    for b0 in range(0, B, chunk):
        b1 = min(B, b0 + chunk)
        if numpy_all:
            lay.S[b0:b1].copy_(to_device(synth.initial_state(cfg, b_idx=np.arange(b0, b1)), "f32", lay.device))
        else:
            lay.S[b0:b1].copy_(torch_gen.initial_state(cfg, b0, b1, lay.device))
    if not numpy_all and exact_seqs is not None:
        for b in exact_seqs:
            lay.S[b:b + 1].copy_(to_device(synth.initial_state(cfg, b_idx=[b]), "f32", lay.device))


def fill_step(step: DeviceStep, cfg: synth.LayerConfig, t: int,
              exact_seqs: Optional[Sequence[int]] = None, numpy_all: bool = False) -> None:
    """Step t's inputs into step (q, k, v, gate, beta)."""
    dev = step.q.device
    if numpy_all:
        si = synth.make_step_inputs(cfg, t)
        step.q.copy_(to_device(si.q, cfg.act, dev))
        step.k.copy_(to_device(si.k, cfg.act, dev))
        step.v.copy_(to_device(si.v, cfg.act, dev))
        gdt = cfg.act if cfg.family == "mamba2" else "f32"
        step.gate.copy_(to_device(si.gate, gdt, dev))
        if si.beta is not None:
            step.beta.copy_(to_device(si.beta, "f32", dev))
        return
    q, k, v, gate, beta = torch_gen.step_inputs(cfg, t, dev)
    step.q.copy_(q)
    step.k.copy_(k)
    step.v.copy_(v)
    step.gate.copy_(gate)
    if beta is not None:
        step.beta.copy_(beta)
    if exact_seqs is not None and len(exact_seqs):
        idx = np.asarray(sorted(set(int(b) for b in exact_seqs)))
        si = synth.make_step_inputs(cfg, t, b_idx=idx)
        ti = torch.from_numpy(idx).to(dev)
        step.q[ti] = to_device(si.q, cfg.act, dev)
        step.k[ti] = to_device(si.k, cfg.act, dev)
        step.v[ti] = to_device(si.v, cfg.act, dev)
        gdt = cfg.act if cfg.family == "mamba2" else "f32"
        step.gate[ti] = to_device(si.gate, gdt, dev)
        if si.beta is not None:
            step.beta[ti] = to_device(si.beta, "f32", dev)


def prime(lay: DecodeLayer, li: synth.LayerInputs) -> int:
    """Build U from the initial state (flush of every tile with an empty
    ring), then identity-pad the ring to each sequence's window phase."""
    from .abi import SKSSM_FLUSH_ALL
    lay.count.zero_()
    rc = lay.flush(None, SKSSM_FLUSH_ALL)
    lay.count.copy_(torch.from_numpy(li.count0).to(lay.device))
    return rc
