"""Helpers that drive the oracle step by step (test infrastructure)."""
from __future__ import annotations

from types import SimpleNamespace

import numpy as np

import oracle


def single_tile(family, dk, dv, W, S0, Pt, Cm, A=0.0, store="exact", count0=0,
                coef="fixed", ridge=0.0, sketch_store=None, pullback="serial"):
    """An OracleLayer with one (sequence, head) tile; Pt, Cm: [r][dk]."""
    r = Pt.shape[0]
    return oracle.OracleLayer(
        family, dk, dv, W, ranks=np.array([r], np.int32), offsets=np.array([0, r], np.int32),
        Pt=np.asarray(Pt, float), Cmap=np.asarray(Cm, float),
        A=None if family != "mamba2" else np.array([A], float),
        tiles=np.array([[0, 0]]), S0=S0[None], heads=1, qk_groups=1,
        state_store=store, sketch_store=store if sketch_store is None else sketch_store,
        out_store=store, count0=np.array([count0], np.int32), coef=coef, ridge=ridge,
        pullback=pullback)


def entry_step(family, e):
    q, k, v, g, b = e
    gate = np.asarray(g, float).reshape(1, 1, -1) if family == "kda" else np.array([[float(g)]])
    return SimpleNamespace(q=np.asarray(q, float)[None, None], k=np.asarray(k, float)[None, None],
                           v=np.asarray(v, float)[None, None], gate=gate,
                           beta=None if family == "mamba2" else np.array([[float(b)]]))


def run_sketch(layer, steps):
    """Prime U from the initial state, then per step: read, and flush the
    tiles whose window the read filled.  Returns outputs [T][n][dv], the
    per-step flush masks and the count after each step."""
    saved = layer.count.copy()
    layer.count[:] = 0
    rc, _ = layer.flush(None, all_tiles=True)
    assert rc == 0
    layer.count[:] = saved
    outs, masks, counts = [], [], []
    for st in steps:
        o = np.zeros((layer.n, layer.dv))
        rc, _ = layer.read(st, o=o)
        assert rc == 0
        due = layer.count == layer.W
        if due.any():
            rc, _ = layer.flush(st, o=o)
            assert rc == 0
        outs.append(o)
        masks.append(due)
        counts.append(layer.count.copy())
    return outs, masks, counts


def run_replay(layer, steps):
    outs = []
    for st in steps:
        rc, o = layer.replay_step(st)
        assert rc == 0
        outs.append(o)
    return outs


def run_standard(layer, steps):
    outs = []
    for st in steps:
        rc, o = layer.full_step(st)
        assert rc == 0
        outs.append(o)
    return outs
