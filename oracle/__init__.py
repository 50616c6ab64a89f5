"""SketchSSM decode oracle -- TEST INFRASTRUCTURE ONLY.

Python side of the fp64 CPU oracle in ``sketchssm_oracle.c``: it builds the
C file with gcc, gathers layer-shaped inputs into per-(sequence, head) tiles
and calls the four oracle procedures (standard step, ReplaySSM step,
sketched read, flush).  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It never imports
the HIP library and the HIP library never imports it; the two share only
the seeded inputs from ``synth``.
"""
from __future__ import annotations

import ctypes as C
import os
import subprocess
from typing import Optional, Sequence

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "sketchssm_oracle.c")
_LIB = os.path.join(_HERE, "_build", "libsketchssm_oracle.so")
# another build of the same source (the sanitizer test loads an instrumented one)
_LIB = os.environ.get("SKSSM_ORACLE_LIB", _LIB)

FAMILY = {"mamba2": 0, "gdn": 1, "kda": 2}
STORE = {"exact": 0, "f32": 1, "bf16": 2}
COEF = {"fixed": 0, "state": 1}
PULLBACK = {"serial": 0, "wy": 1, "proj": 2}
ERR_COUNT = 1


def build(force: bool = True, out: str = None, extra=()) -> str:
    """Compile the oracle with gcc (-O2, OpenMP, no fast-math); out and extra
    build another copy (e.g. with sanitizers) at another path."""
    out = out or _LIB
    if force or not os.path.exists(out):
        os.makedirs(os.path.dirname(out), exist_ok=True)
        tmp = out + ".tmp%d" % os.getpid()
        subprocess.check_call(["gcc", "-std=c11", "-O2", "-fopenmp", "-fPIC", "-shared",
                               "-Wall", "-Wno-unknown-pragmas"] + list(extra) + [_SRC, "-o", tmp, "-lm"])
        os.replace(tmp, out)
    return out


class _Layer(C.Structure):
    _fields_ = [("family", C.c_int), ("dk", C.c_int), ("dv", C.c_int), ("W", C.c_int),
                ("rmax", C.c_int), ("state_store", C.c_int), ("sketch_store", C.c_int),
                ("out_store", C.c_int), ("coef_mode", C.c_int), ("coef_ridge", C.c_double),
                ("pullback", C.c_int)]


_DP = C.POINTER(C.c_double)
_IP = C.POINTER(C.c_int)


class _Tiles(C.Structure):
    _fields_ = [("n", C.c_int), ("rank", _IP), ("S", _DP), ("U", _DP), ("Pt", _DP),
                ("C", _DP), ("A", _DP), ("rk", _DP), ("rv", _DP), ("rg", _DP),
                ("rb", _DP), ("count", _IP), ("Sc", _DP), ("rp", _DP)]


class _Step(C.Structure):
    _fields_ = [("q", _DP), ("k", _DP), ("v", _DP), ("g", _DP), ("b", _DP), ("o", _DP)]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build(force=True)
        _lib = C.CDLL(_LIB)
        for name in ("orc_full_step", "orc_read", "orc_replay_step"):
            getattr(_lib, name).argtypes = [C.POINTER(_Layer), C.POINTER(_Tiles), C.POINTER(_Step)]
            getattr(_lib, name).restype = C.c_int
        _lib.orc_flush.argtypes = [C.POINTER(_Layer), C.POINTER(_Tiles), C.POINTER(_Step), C.c_int]
        _lib.orc_flush.restype = C.c_int
        _lib.orc_set_mutation.argtypes = [C.c_int]
        _lib.orc_num_threads.restype = C.c_int
        _lib.orc_set_num_threads.argtypes = [C.c_int]
    return _lib


def set_mutation(m: int) -> None:
    lib().orc_set_mutation(int(m))


def num_threads() -> int:
    return int(lib().orc_num_threads())


def set_num_threads(n: int) -> None:
    lib().orc_set_num_threads(int(n))


def _p(a: Optional[np.ndarray], ty=_DP):
    if a is None:
        return C.cast(None, ty)
    assert a.flags.c_contiguous
    return a.ctypes.data_as(ty)


class OracleLayer:
    """The oracle's state for a set of (sequence, head) tiles of one layer.

    family, dk, dv, W: layer shape; ranks/Pt/C/A: per-head tables as produced
    by ``synth`` (Pt and C are [R][dk] with head h's rows at offsets[h]);
    tiles: [n, 2] array of (b, h); S0: [n][dk][dv] initial state of those
    tiles; stores: rounding at the state / sketch / output stores ("exact",
    "f32", "bf16"); qk_groups: heads per B/C group for the k/q gather.
    A head of rank 0 is a dense-fallback head: its flush stores the state in
    the sketch dtype (Sc) and its reads take S^T q~ from that copy.
    coef: "fixed" reads the per-head table Cmap; "state" makes every flush
    write each tile's own map from its new state (Cmap is then ignored) with
    the relative ridge ``ridge``; the map is stored in the sketch dtype.
    pullback: how the sketched read evaluates the effective query and the
    buffered term, "serial" (one transition at a time), "wy" (every slot's
    coefficient at once from a triangular system, paper App. C.1) or "proj"
    (the same coefficients, with C q~ formed from per-slot factors projected
    through the coefficient map when each slot is appended, paper App. C.2;
    self.rp holds them).
    """

    def __init__(self, family: str, dk: int, dv: int, W: int, ranks: np.ndarray,
                 offsets: np.ndarray, Pt: np.ndarray, Cmap: np.ndarray,
                 A: Optional[np.ndarray], tiles: np.ndarray, S0: np.ndarray,
                 heads: int, qk_groups: int, state_store="f32", sketch_store="f32",
                 out_store="f32", count0: Optional[np.ndarray] = None,
                 coef: str = "fixed", ridge: float = 0.0, pullback: str = "serial"):
        self.family, self.dk, self.dv, self.W = family, dk, dv, W
        self.tiles = np.ascontiguousarray(np.asarray(tiles, dtype=np.int64).reshape(-1, 2))
        n = len(self.tiles)
        self.n = n
        self.heads, self.qk_groups = heads, qk_groups
        self.hpg = heads // qk_groups
        hh = self.tiles[:, 1]
        self.rank = np.ascontiguousarray(np.asarray(ranks, dtype=np.int32)[hh])
        self.rmax = max(1, int(self.rank.max()) if n else 1)
        self.Pt = np.zeros((n, self.rmax, dk))
        self.C = np.zeros((n, self.rmax, dk))
        for i, h in enumerate(hh):
            r = int(ranks[h])
            self.Pt[i, :r] = Pt[offsets[h]:offsets[h] + r]
            if coef == "fixed":
                self.C[i, :r] = Cmap[offsets[h]:offsets[h] + r]
        self.A = None if A is None else np.ascontiguousarray(np.asarray(A, dtype=np.float64)[hh])
        self.S = np.ascontiguousarray(np.asarray(S0, dtype=np.float64).reshape(n, dk, dv)).copy()
        self.U = np.zeros((n, self.rmax, dv))
        self.Sc = np.zeros((n, dk, dv))          # state copies of rank-0 (dense-fallback) tiles
        self.gl = dk if family == "kda" else 1
        self.rk = np.zeros((n, W, dk))
        self.rv = np.zeros((n, W, dv))
        ident = 0.0 if family == "mamba2" else 1.0
        self.rg = np.full((n, W, self.gl), ident)
        self.rb = None if family == "mamba2" else np.zeros((n, W))
        self.rp = np.zeros((n, W, self.rmax))   # projected factors (pullback "proj")
        self.count = np.zeros(n, dtype=np.int32) if count0 is None else \
            np.ascontiguousarray(np.asarray(count0, dtype=np.int32).reshape(n)).copy()
        self.L = _Layer(FAMILY[family], dk, dv, W, self.rmax, STORE[state_store],
                        STORE[sketch_store], STORE[out_store], COEF[coef], float(ridge),
                        PULLBACK[pullback])

    # ------------------------------------------------------------------
    def _tiles_struct(self):
        return _Tiles(self.n, _p(self.rank, _IP), _p(self.S), _p(self.U), _p(self.Pt),
                      _p(self.C), _p(self.A), _p(self.rk), _p(self.rv), _p(self.rg),
                      _p(self.rb), _p(self.count, _IP), _p(self.Sc), _p(self.rp))

    def gather_step(self, step, seq_rows: Optional[np.ndarray] = None):
        """Per-tile arrays from a layer-shaped StepInputs (rows = sequences).
        seq_rows maps a tile's sequence b to its row in the step arrays (the
        identity when the step holds every sequence)."""
        b = self.tiles[:, 0] if seq_rows is None else seq_rows[self.tiles[:, 0]]
        h = self.tiles[:, 1]
        g = h // self.hpg
        q = np.ascontiguousarray(step.q[b, g], dtype=np.float64)
        k = np.ascontiguousarray(step.k[b, g], dtype=np.float64)
        v = np.ascontiguousarray(step.v[b, h], dtype=np.float64)
        gate = np.ascontiguousarray(step.gate[b, h], dtype=np.float64)
        beta = None if step.beta is None else np.ascontiguousarray(step.beta[b, h], dtype=np.float64)
        return q, k, v, gate, beta

    def _call(self, name, step, seq_rows, o, *extra):
        if o is None:
            o = np.zeros((self.n, self.dv))
        assert o.shape == (self.n, self.dv) and o.dtype == np.float64 and o.flags.c_contiguous
        keep = None
        if step is not None:
            keep = self.gather_step(step, seq_rows)
            q, k, v, gate, beta = keep
            st = _Step(_p(q), _p(k), _p(v), _p(gate), _p(beta), _p(o))
            stp = C.byref(st)
        else:
            stp = C.cast(None, C.POINTER(_Step))
        T = self._tiles_struct()
        rc = getattr(lib(), name)(C.byref(self.L), C.byref(T), stp, *extra)
        del keep
        return rc, o

    # Each call returns (status, o); o is written into the given array when
    # one is passed (a read and the flush of the same step share one output).
    def full_step(self, step, seq_rows=None, o=None):
        return self._call("orc_full_step", step, seq_rows, o)

    def read(self, step, seq_rows=None, o=None):
        return self._call("orc_read", step, seq_rows, o)

    def replay_step(self, step, seq_rows=None, o=None):
        return self._call("orc_replay_step", step, seq_rows, o)

    def flush(self, step=None, all_tiles: bool = False, seq_rows=None, o=None):
        return self._call("orc_flush", step, seq_rows, o, C.c_int(1 if all_tiles else 0))

    def set_ring(self, count: np.ndarray):
        """Identity-pad the ring: count entries with k = v = 0, beta = 0 and
        the family's identity gate (used for ragged window phases)."""
        self.count[:] = np.asarray(count, dtype=np.int32).reshape(self.n)
