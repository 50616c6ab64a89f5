"""Pins of the oracle's dense-fallback heads (rank 0).

Such a head keeps a copy of its state in the sketch dtype instead of a
sketch: the flush stores the updated state, the non-flush read takes
S^T q~ from the copy and adds the exact buffered term (paper App. D: dense
fallback heads read a bf16 state copy).  The pins check it against dense
brute force, against the copy's own rounding, and in a layer that mixes
dense and sketched heads; a mutation test plants a mistake.
"""
import numpy as np
import pytest

import oracle
from synth import round_bf16
from tests import bruteforce as bf
from tests.oracle_drive import single_tile, entry_step, run_sketch

FAMS = ("mamba2", "gdn", "kda")


def rel(x, y):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def _dense_tile(family, S0, W, store="exact", sketch_store=None, A=0.3):
    dk, dv = S0.shape
    return single_tile(family, dk, dv, W, S0, np.zeros((0, dk)), np.zeros((0, dk)), A,
                       store=store, sketch_store=sketch_store)


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("W", [1, 3, 5])
def test_exact_copy_reads_exactly(family, W):
    """With an exact copy, every output of a dense-fallback tile equals the
    plain recurrence's, computed with explicit dense transition matrices."""
    rng = np.random.default_rng(21 + W)
    dk, dv = 5, 4
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, 13)
    std, _ = bf.standard_run(family, S0, ents, 0.3)
    lay = _dense_tile(family, S0, W)
    outs, _, _ = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-12


@pytest.mark.parametrize("family", FAMS)
def test_bf16_copy_is_the_rounded_state(family):
    """The copy is the stored state rounded to bf16 (nearest even), and the
    read is that copy's S^T q~ plus the exact buffered term, both taken from
    dense products."""
    rng = np.random.default_rng(31)
    dk, dv, W = 6, 4, 4
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, 7)
    lay = _dense_tile(family, S0, W, store="f32", sketch_store="bf16")
    steps = [entry_step(family, e) for e in ents]
    outs, masks, _ = run_sketch(lay, steps[:W])      # one whole window: the copy is refreshed
    assert masks[W - 1][0]
    assert np.array_equal(lay.Sc[0], round_bf16(lay.S[0]))
    copy = lay.Sc[0].copy()
    ring = []
    for t in range(W, len(ents)):                     # reads of the next window
        q, k, v, g, b = ents[t]
        ring.append((k, v, g, b))
        o = np.zeros((1, dv))
        assert lay.read(steps[t], o=o)[0] == 0
        qt, obuf, _, _ = bf.window_terms(family, ring, q, 0.3)
        assert rel(o[0], copy.T @ qt + obuf) < 1e-6


def test_mixed_layer():
    """A layer with dense and sketched heads: each dense tile matches its own
    single-tile run, each sketched tile its own, so the two kinds do not
    interfere."""
    rng = np.random.default_rng(41)
    family, dk, dv, W, H = "gdn", 6, 4, 3, 4
    ranks = np.array([0, 2, 0, 3], np.int32)
    offsets = np.concatenate([[0], np.cumsum(ranks)]).astype(np.int32)
    Pt = np.zeros((int(offsets[-1]), dk))
    for h in range(H):
        if ranks[h]:
            Q, _ = np.linalg.qr(rng.standard_normal((dk, ranks[h])))
            Pt[offsets[h]:offsets[h + 1]] = Q.T
    S0 = rng.standard_normal((H, dk, dv))
    tiles = np.array([(0, h) for h in range(H)])
    lay = oracle.OracleLayer(family, dk, dv, W, ranks, offsets, Pt, Pt.copy(), None, tiles, S0,
                             heads=H, qk_groups=H, state_store="exact", sketch_store="exact",
                             out_store="exact")
    ents = [bf.random_entries(rng, family, dk, dv, 8) for _ in range(H)]
    from types import SimpleNamespace
    steps = []
    for t in range(8):
        q = np.stack([ents[h][t][0] for h in range(H)])[None]
        k = np.stack([ents[h][t][1] for h in range(H)])[None]
        v = np.stack([ents[h][t][2] for h in range(H)])[None]
        g = np.array([[ents[h][t][3] for h in range(H)]])
        b = np.array([[ents[h][t][4] for h in range(H)]])
        steps.append(SimpleNamespace(q=q, k=k, v=v, gate=g, beta=b))
    outs, _, _ = run_sketch(lay, steps)
    for h in range(H):
        r = int(ranks[h])
        one = single_tile(family, dk, dv, W, S0[h], Pt[offsets[h]:offsets[h + 1]],
                          Pt[offsets[h]:offsets[h + 1]].copy(), 0.0)
        o1, _, _ = run_sketch(one, [entry_step(family, ents[h][t]) for t in range(8)])
        for t in range(8):
            assert np.array_equal(outs[t][h], o1[t][0]), (h, r, t)
        if r == 0:
            std, _ = bf.standard_run(family, S0[h], ents[h], 0.0)
            assert max(rel(outs[t][h], std[t]) for t in range(8)) < 1e-12


def test_dense_pins_catch_planted_mistake():
    """Reading the copy with the raw query instead of the pulled-back one is
    caught (GDN: the two differ)."""
    test_exact_copy_reads_exactly("gdn", 3)
    oracle.set_mutation(14)
    try:
        with pytest.raises(AssertionError):
            test_exact_copy_reads_exactly("gdn", 3)
    finally:
        oracle.set_mutation(0)
    test_exact_copy_reads_exactly("gdn", 3)
