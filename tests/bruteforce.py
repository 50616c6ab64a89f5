"""Dense brute-force formulations used to pin the oracle.

Every transition M_t is built as an explicit dk x dk matrix and every
product is a dense numpy matmul, so these functions share nothing with the
oracle's structured loops (scalar decays, rank-1 erase updates, the
newest-first pull-back).  They follow the pages' definitions directly:
S_t = M_t S_{t-1} + B_t and o_t = S_t^T q_t (project page, full-state
equation); the effective query q~ = M_1^T ... M_n^T q and the sketched read
U (C q~) with U = S0^T P (project page, sketch and readout panels).
"""
from __future__ import annotations

import numpy as np


def dense_M(family, k, gate, beta, A=0.0):
    dk = len(k)
    eye = np.eye(dk)
    if family == "mamba2":
        return np.exp(-float(gate) * np.exp(A)) * eye
    E = eye - float(beta) * np.outer(k, k)
    if family == "gdn":
        return float(gate) * E
    if family == "kda":
        return E @ np.diag(gate)
    raise ValueError(family)


def dense_B(family, k, v, gate, beta):
    s = float(gate) if family == "mamba2" else float(beta)
    return s * np.outer(k, v)


def standard_run(family, S0, entries, A=0.0):
    """entries: list of (q, k, v, gate, beta). Returns outputs and states."""
    S = S0.copy()
    outs, states = [], []
    for (q, k, v, g, b) in entries:
        S = dense_M(family, k, g, b, A) @ S + dense_B(family, k, v, g, b)
        outs.append(S.T @ q)
        states.append(S.copy())
    return outs, states


def window_terms(family, ring, q, A=0.0):
    """For ring entries 1..n (oldest first): q~ = (M_n ... M_1)^T q and the
    buffered term sum_i (M_n ... M_{i+1} B_i)^T q, both by dense products."""
    dk = len(q)
    prod = np.eye(dk)                    # M_n ... M_1
    buf_state = np.zeros((dk, ring[0][1].shape[0])) if ring else None
    for (k, v, g, b) in ring:
        M = dense_M(family, k, g, b, A)
        prod = M @ prod
        buf_state = M @ buf_state + dense_B(family, k, v, g, b)
    qt = prod.T @ q
    obuf = buf_state.T @ q
    return qt, obuf, prod, buf_state


def sketch_run(family, S0, entries, W, Pt, Cm, A=0.0, phase_count=0):
    """SketchSSM over a stream of entries with one tile.

    The sketch is primed from S0, then each step appends its entry; when the
    window is full the flush applies the W entries to the state exactly,
    rebuilds U = S^T P and outputs S^T q; otherwise the output is
    U (C q~) + buffered term.  phase_count identity entries pre-fill the ring
    (ragged phase).  Returns outputs, flush flags and the state after each step.
    """
    dk = S0.shape[0]
    S = S0.copy()
    U = S.T @ Pt.T                    # [dv][r]: column j = S^T p_j
    ident = 0.0 if family == "mamba2" else 1.0
    gate_ident = np.full(dk, ident) if family == "kda" else ident
    ring = [(np.zeros(dk), np.zeros(S0.shape[1]), gate_ident, 0.0)] * phase_count
    outs, flushed, states = [], [], []
    for (q, k, v, g, b) in entries:
        ring = ring + [(k, v, g, b)]
        if len(ring) == W:
            _, _, prod, bstate = window_terms(family, ring, q, A)
            S = prod @ S + bstate
            U = S.T @ Pt.T
            outs.append(S.T @ q)
            flushed.append(True)
            ring = []
        else:
            qt, obuf, _, _ = window_terms(family, ring, q, A)
            outs.append(U @ (Cm @ qt) + obuf)
            flushed.append(False)
        states.append(S.copy())
    return outs, flushed, states, U


def replay_run(family, S0, entries, W, A=0.0):
    dk = S0.shape[0]
    S = S0.copy()
    ring = []
    outs = []
    for (q, k, v, g, b) in entries:
        ring = ring + [(k, v, g, b)]
        qt, obuf, prod, bstate = window_terms(family, ring, q, A)
        if len(ring) == W:
            S = prod @ S + bstate
            outs.append(S.T @ q)
            ring = []
        else:
            outs.append(S.T @ qt + obuf)
    return outs


def random_entries(rng, family, dk, dv, T, unit_k=False):
    ents = []
    for _ in range(T):
        q = rng.standard_normal(dk)
        k = rng.standard_normal(dk)
        if unit_k:
            k = k / np.linalg.norm(k)
        v = rng.standard_normal(dv)
        if family == "mamba2":
            g = rng.uniform(0.1, 1.0)
            b = 0.0
        elif family == "gdn":
            g = rng.uniform(0.5, 1.0)
            b = rng.uniform(0.0, 1.0)
        else:
            g = rng.uniform(0.5, 1.0, size=dk)
            b = rng.uniform(0.0, 1.0)
        ents.append((q, k, v, g, b))
    return ents
