"""ctypes binding of libsketchssm.so (argument marshalling only).

The four entry points keep the C names: ``sketchssm_read``,
``sketchssm_flush``, ``sketchssm_full_step``, ``sketchssm_replay_step``.
Each takes the three argument structs (or pointers to them) and a HIP stream
handle, and returns the library's status code.  Loading fails loudly when the
library has not been built: there is no fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libsketchssm.so")

# constants of include/sketchssm.h
SKSSM_MAMBA2, SKSSM_GDN, SKSSM_KDA = 0, 1, 2
SKSSM_F32, SKSSM_BF16 = 0, 1
SKSSM_FLUSH_DUE, SKSSM_FLUSH_ALL, SKSSM_FLUSH_DUE_SCAN, SKSSM_FLUSH_CLOSE = 0, 1, 2, 3
SKSSM_COEF_FIXED, SKSSM_COEF_STATE = 0, 1
SKSSM_PULLBACK_SERIAL, SKSSM_PULLBACK_WY, SKSSM_PULLBACK_PROJ = 0, 1, 2
SKSSM_OK, SKSSM_EINVAL, SKSSM_EDIM, SKSSM_EDTYPE, SKSSM_EFLAG, SKSSM_ELAUNCH = 0, -1, -2, -3, -4, -5
SKSSM_ESCRATCH = -6
SKSSM_NOALLOC_SCRATCH_BYTES = 16777216
SKSSM_ERRBIT_COUNT, SKSSM_ERRBIT_GROUP, SKSSM_ERRBIT_SEQ = 1, 2, 4

ENTRY_POINTS = ("sketchssm_read", "sketchssm_flush", "sketchssm_flush_seqs", "sketchssm_full_step",
                "sketchssm_replay_step", "sketchssm_workspace_bytes", "sketchssm_read_noalloc",
                "sketchssm_version")


class sketchssm_layer(C.Structure):
    _fields_ = [("family", C.c_int32), ("batch", C.c_int32), ("heads", C.c_int32),
                ("qk_groups", C.c_int32), ("dk", C.c_int32), ("dv", C.c_int32),
                ("window", C.c_int32), ("act_dtype", C.c_int32), ("sketch_dtype", C.c_int32),
                ("rank_offsets_host", C.POINTER(C.c_int32)), ("coef_map", C.c_int32),
                ("coef_ridge", C.c_float), ("pullback", C.c_int32)]


class sketchssm_buffers(C.Structure):
    _fields_ = [("S", C.c_void_p), ("U", C.c_void_p), ("Pt", C.c_void_p), ("C", C.c_void_p),
                ("rank_offsets", C.c_void_p), ("ring_k", C.c_void_p), ("ring_v", C.c_void_p),
                ("ring_gate", C.c_void_p), ("ring_beta", C.c_void_p), ("count", C.c_void_p),
                ("A", C.c_void_p), ("err", C.c_void_p), ("work", C.c_void_p),
                ("Cstate", C.c_void_p), ("Scopy", C.c_void_p), ("ring_pc", C.c_void_p)]


class sketchssm_step(C.Structure):
    _fields_ = [("q", C.c_void_p), ("k", C.c_void_p), ("v", C.c_void_p), ("gate", C.c_void_p),
                ("beta", C.c_void_p), ("o", C.c_void_p)]


_lib = None


def load(path: str = LIB_PATH) -> C.CDLL:
    """Load the HIP library; raises if it is missing (no CPU fallback)."""
    global _lib
    if _lib is None:
        # torch ships its own HIP runtime under the same soname as the
        # system's (libamdhip64.so.7); whichever is loaded first serves the
        # whole process.  Importing torch before the library keeps both on
        # torch's runtime, so that tensors allocated by torch are valid in
        # the library's launches whatever the caller imported first.
        try:
            import torch  # noqa: F401
        except ImportError:
            pass
        if not os.path.exists(path):
            raise RuntimeError(f"{path} is not built: run __graft_entry__.build() "
                               "(or python ssm_decode_amd/build.py) first")
        lib = C.CDLL(path)
        L, Bf, St = C.POINTER(sketchssm_layer), C.POINTER(sketchssm_buffers), C.POINTER(sketchssm_step)
        for name in ("sketchssm_read", "sketchssm_read_noalloc", "sketchssm_full_step",
                     "sketchssm_replay_step"):
            fn = getattr(lib, name)
            fn.argtypes = [L, Bf, St, C.c_void_p]
            fn.restype = C.c_int
        lib.sketchssm_flush.argtypes = [L, Bf, St, C.c_int32, C.c_void_p]
        lib.sketchssm_flush.restype = C.c_int
        lib.sketchssm_flush_seqs.argtypes = [L, Bf, St, C.c_void_p, C.c_int32, C.c_void_p]
        lib.sketchssm_flush_seqs.restype = C.c_int
        lib.sketchssm_workspace_bytes.argtypes = [L]
        lib.sketchssm_workspace_bytes.restype = C.c_int64
        lib.sketchssm_version.argtypes = []
        lib.sketchssm_version.restype = C.c_int
        _lib = lib
    return _lib


def _ref(x, ty):
    if x is None:
        return C.cast(None, C.POINTER(ty))
    if isinstance(x, ty):
        return C.byref(x)
    return x


def sketchssm_read(layer, bufs, step, stream=None) -> int:
    return load().sketchssm_read(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                 _ref(step, sketchssm_step), stream)


def sketchssm_read_noalloc(layer, bufs, step, stream=None) -> int:
    """sketchssm_read with the library's own scratch array as the workspace
    (bufs.work is ignored; nothing is allocated)."""
    return load().sketchssm_read_noalloc(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                         _ref(step, sketchssm_step), stream)


def sketchssm_flush(layer, bufs, step, flags, stream=None) -> int:
    return load().sketchssm_flush(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                  _ref(step, sketchssm_step), int(flags), stream)


def sketchssm_flush_seqs(layer, bufs, step, seqs, nseq, stream=None) -> int:
    """seqs: device address of nseq int32 sequence indices (or None with nseq = 0)."""
    return load().sketchssm_flush_seqs(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                       _ref(step, sketchssm_step), seqs, int(nseq), stream)


def sketchssm_full_step(layer, bufs, step, stream=None) -> int:
    return load().sketchssm_full_step(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                      _ref(step, sketchssm_step), stream)


def sketchssm_replay_step(layer, bufs, step, stream=None) -> int:
    return load().sketchssm_replay_step(_ref(layer, sketchssm_layer), _ref(bufs, sketchssm_buffers),
                                        _ref(step, sketchssm_step), stream)


def sketchssm_workspace_bytes(layer) -> int:
    return load().sketchssm_workspace_bytes(_ref(layer, sketchssm_layer))


def sketchssm_version() -> int:
    return load().sketchssm_version()
