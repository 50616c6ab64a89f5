"""Device buffers of one decode layer, allocated with torch, and the argument
structs that describe them to the C ABI.  torch is used for device memory
and streams only; every step of the decode path runs in the HIP library."""
from __future__ import annotations

import ctypes as C
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

from . import abi

FAMILY = {"mamba2": abi.SKSSM_MAMBA2, "gdn": abi.SKSSM_GDN, "kda": abi.SKSSM_KDA}
DTYPE = {"f32": abi.SKSSM_F32, "bf16": abi.SKSSM_BF16}
TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else C.c_void_p(t.data_ptr())


def current_stream_handle() -> int:
    return torch.cuda.current_stream().cuda_stream


@dataclass
class DeviceStep:
    """One decode step's device tensors (layouts as in include/sketchssm.h)."""
    q: torch.Tensor
    k: torch.Tensor
    v: torch.Tensor
    gate: torch.Tensor
    beta: Optional[torch.Tensor]
    o: torch.Tensor

    def struct(self) -> abi.sketchssm_step:
        return abi.sketchssm_step(_ptr(self.q), _ptr(self.k), _ptr(self.v), _ptr(self.gate),
                                  _ptr(self.beta), _ptr(self.o))


COEF = {"fixed": abi.SKSSM_COEF_FIXED, "state": abi.SKSSM_COEF_STATE}
PULLBACK = {"serial": abi.SKSSM_PULLBACK_SERIAL, "wy": abi.SKSSM_PULLBACK_WY,
            "proj": abi.SKSSM_PULLBACK_PROJ}


class DecodeLayer:
    """All persistent buffers of one layer: S, U, Pt, C, rank offsets, the
    ring (k, v, gate, beta), the per-tile ring counts, A, the error word and
    the read's workspace.  coef = "fixed" reads the per-head map Cmap;
    coef = "state" has every flush write each tile's own map into Cstate
    ([B][R][dk], sketch dtype) with the relative ridge ``ridge``.
    pullback = "serial", "wy" or "proj" selects how a GDN/KDA read evaluates
    the effective query and the buffered term (Mamba-2 ignores it); "proj"
    keeps the ring's projected factors in ring_pc."""

    def __init__(self, family: str, batch: int, heads: int, qk_groups: int, dk: int, dv: int,
                 window: int, act: str, sketch: str, rank_offsets: np.ndarray,
                 device: str = "cuda", coef: str = "fixed", ridge: float = 1e-4,
                 pullback: str = "serial"):
        self.family, self.B, self.H, self.G = family, batch, heads, qk_groups
        self.dk, self.dv, self.W = dk, dv, window
        self.act, self.sketch = act, sketch
        self.device = device
        self.coef, self.ridge = coef, float(ridge)
        self.pullback = pullback
        self.offsets_host = np.ascontiguousarray(np.asarray(rank_offsets, dtype=np.int32))
        self.R = int(self.offsets_host[-1])
        at, ut = TORCH_DTYPE[act], TORCH_DTYPE[sketch]
        B, H, G, W = batch, heads, qk_groups, window
        z = lambda shape, dt: torch.zeros(shape, dtype=dt, device=device)
        self.S = z((B, H, dk, dv), torch.float32)
        self.U = z((B, self.R, dv), ut)
        self.Pt = z((self.R, dk), torch.float32)
        self.Cmap = z((self.R, dk), torch.float32)
        self.Cstate = z((B, self.R, dk), ut) if coef == "state" else None
        # state copies of the dense-fallback heads (rank 0), in head order
        self.dense_heads = np.nonzero(np.diff(self.offsets_host) == 0)[0]
        nd = len(self.dense_heads)
        self.Scopy = z((B, nd, dk, dv), ut) if nd else None
        self.offsets = torch.from_numpy(self.offsets_host.copy()).to(device)
        self.ring_k = z((B, G, W, dk), at)
        self.ring_v = z((B, H, W, dv), at)
        if family == "mamba2":
            self.ring_gate = z((B, H, W), at)
            self.ring_beta = None
            self.A = z((H,), torch.float32)
        elif family == "gdn":
            self.ring_gate = torch.ones((B, H, W), dtype=torch.float32, device=device)
            self.ring_beta = z((B, H, W), torch.float32)
            self.A = None
        else:
            self.ring_gate = torch.ones((B, H, W, dk), dtype=torch.float32, device=device)
            self.ring_beta = z((B, H, W), torch.float32)
            self.A = None
        # projected per-slot factors of the "proj" pull-back (GDN/KDA)
        self.ring_pc = z((B, H, W, 16), torch.float32) if (pullback == "proj" and family != "mamba2") else None
        self.count = z((B, H), torch.int32)
        self.err = z((4,), torch.int32)
        self._layer = abi.sketchssm_layer(
            FAMILY[family], B, H, G, dk, dv, W, DTYPE[act], DTYPE[sketch],
            self.offsets_host.ctypes.data_as(C.POINTER(C.c_int32)), COEF[coef],
            self.ridge if coef == "state" else 0.0, PULLBACK[pullback])
        nwork = abi.sketchssm_workspace_bytes(self._layer)
        if nwork < 0:
            raise ValueError(f"invalid layer description (code {nwork})")
        self.work = z((nwork,), torch.uint8) if nwork else None
        self._bufs = abi.sketchssm_buffers(
            _ptr(self.S), _ptr(self.U), _ptr(self.Pt), _ptr(self.Cmap), _ptr(self.offsets),
            _ptr(self.ring_k), _ptr(self.ring_v), _ptr(self.ring_gate), _ptr(self.ring_beta),
            _ptr(self.count), _ptr(self.A), _ptr(self.err), _ptr(self.work), _ptr(self.Cstate),
            _ptr(self.Scopy), _ptr(self.ring_pc))

    # -------------------------------------------------------------- structs
    @property
    def layer_struct(self) -> abi.sketchssm_layer:
        return self._layer

    @property
    def buffers_struct(self) -> abi.sketchssm_buffers:
        return self._bufs

    def new_step(self) -> DeviceStep:
        """Zeroed device tensors for one step's inputs and output."""
        at = TORCH_DTYPE[self.act]
        d, B, H, G = self.device, self.B, self.H, self.G
        gate = (torch.zeros((B, H), dtype=at, device=d) if self.family == "mamba2" else
                torch.zeros((B, H), dtype=torch.float32, device=d) if self.family == "gdn" else
                torch.zeros((B, H, self.dk), dtype=torch.float32, device=d))
        beta = None if self.family == "mamba2" else torch.zeros((B, H), dtype=torch.float32, device=d)
        return DeviceStep(q=torch.zeros((B, G, self.dk), dtype=at, device=d),
                          k=torch.zeros((B, G, self.dk), dtype=at, device=d),
                          v=torch.zeros((B, H, self.dv), dtype=at, device=d),
                          gate=gate, beta=beta,
                          o=torch.zeros((B, H, self.dv), dtype=at, device=d))

    # ---------------------------------------------------------------- calls
    def _stream(self, stream):
        return C.c_void_p(current_stream_handle() if stream is None else stream)

    def read(self, step: DeviceStep, stream=None) -> int:
        return abi.sketchssm_read(self._layer, self._bufs, step.struct(), self._stream(stream))

    def read_noalloc(self, step: DeviceStep, stream=None) -> int:
        """The read with the library's scratch array as its workspace."""
        return abi.sketchssm_read_noalloc(self._layer, self._bufs, step.struct(), self._stream(stream))

    def flush(self, step: Optional[DeviceStep], flags: int = abi.SKSSM_FLUSH_DUE, stream=None) -> int:
        st = None if step is None else step.struct()
        return abi.sketchssm_flush(self._layer, self._bufs, st, flags, self._stream(stream))

    def flush_seqs(self, step: Optional[DeviceStep], seqs, stream=None) -> int:
        """Due-only flush of the sequences in seqs (an int32 device tensor of
        distinct indices)."""
        st = None if step is None else step.struct()
        if seqs.dtype != torch.int32 or seqs.dim() != 1 or not seqs.is_contiguous():
            raise ValueError("seqs: a contiguous 1-d int32 tensor")
        n = int(seqs.numel())
        if n and seqs.device.type != "cuda":
            raise ValueError("seqs must be device memory")
        ptr = C.c_void_p(seqs.data_ptr()) if n else None
        return abi.sketchssm_flush_seqs(self._layer, self._bufs, st, ptr, n, self._stream(stream))

    def full_step(self, step: DeviceStep, stream=None) -> int:
        return abi.sketchssm_full_step(self._layer, self._bufs, step.struct(), self._stream(stream))

    def replay_step(self, step: DeviceStep, stream=None) -> int:
        return abi.sketchssm_replay_step(self._layer, self._bufs, step.struct(), self._stream(stream))

    def error_word(self) -> int:
        return int(self.err[0].item())
