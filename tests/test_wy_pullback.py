"""Pins of the oracle's parallel evaluation of the effective query (paper
App. C.1, the WY-style form): every buffered slot's coefficient from one
upper-triangular system instead of one transition at a time.

The pins check it against dense products of the explicit transition
matrices (the query pulled back and the buffered term, each on its own),
against whole decode runs of the plain recurrence, and against the serial
form on random layers; a planted mistake in the system's decay products is
caught."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from tests.oracle_drive import single_tile, entry_step, run_sketch

FAMS = ("mamba2", "gdn", "kda")


def rel(x, y):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def _dense_tile(family, S0, W, pullback, A=0.3):
    """A dense-fallback tile (rank 0) with exact stores: its read is
    S0^T q~ + o_buf with S0 the exact copy."""
    dk = S0.shape[0]
    return single_tile(family, dk, S0.shape[1], W, S0, np.zeros((0, dk)), np.zeros((0, dk)), A,
                       store="exact", pullback=pullback)


def _read_after(family, S0, W, ring_entries, q, pullback, A=0.3):
    """Output of the read whose ring holds ring_entries and whose own entry
    is the last of them (its query q)."""
    lay = _dense_tile(family, S0, W, pullback, A)
    steps = [entry_step(family, e) for e in ring_entries]
    steps[-1].q = np.asarray(q, float)[None, None]
    outs, _, _ = run_sketch(lay, steps)
    return outs[-1][0]


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("n", [1, 2, 5, 8])
def test_query_and_buffer_terms_against_dense_products(family, n):
    """With a zero copy the read is the buffered term alone; with the
    identity copy it adds q~.  Both against (M_n..M_1)^T q and the buffered
    state's read, formed from explicit matrices."""
    rng = np.random.default_rng(100 + n)
    d = 6
    ents = bf.random_entries(rng, family, d, d, n)
    q = rng.standard_normal(d)
    ring = [(k, v, g, b) for (_, k, v, g, b) in ents]
    qt, obuf, _, _ = bf.window_terms(family, ring, q, 0.3)
    W = n + 1
    o0 = _read_after(family, np.zeros((d, d)), W, ents, q, "wy")
    oI = _read_after(family, np.eye(d), W, ents, q, "wy")
    assert rel(o0, obuf) < 1e-12
    assert rel(oI - o0, qt) < 1e-12


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("W", [1, 3, 5])
def test_decode_run_equals_plain_recurrence(family, W):
    """Every output of a dense-fallback tile with an exact copy, read with
    the parallel form, equals the plain recurrence's."""
    rng = np.random.default_rng(21 + W)
    dk, dv = 5, 4
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, 13)
    std, _ = bf.standard_run(family, S0, ents, 0.3)
    lay = _dense_tile(family, S0, W, "wy")
    outs, _, _ = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-12


@pytest.mark.parametrize("family", FAMS)
def test_parallel_form_matches_serial_on_random_layers(family):
    """A layer of sketched tiles at mixed ring fills: the parallel and the
    serial forms agree to rounding (exact stores), and to the f32 output
    store's rounding with f32 stores."""
    import synth
    from synth import LayerConfig
    cfg = LayerConfig(name="wy_" + family, family=family, batch=3, heads=4,
                      qk_groups=2 if family == "mamba2" else 4, dk=16, dv=32, window=6,
                      mean_rank=4, fixed_rank=None, act="f32", sketch="f32", steps=14,
                      ragged=True, seed=71)
    li = synth.make_layer_inputs(cfg)
    tiles = np.array([(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    for store, tol in (("exact", 1e-12), ("f32", 1e-6)):
        lays = [oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets,
                                   li.Pt, li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups,
                                   state_store=store, sketch_store=store, out_store=store,
                                   count0=li.count0[tiles[:, 0], tiles[:, 1]], pullback=pb)
                for pb in ("serial", "wy")]
        for lay in lays:
            assert lay.flush(None, all_tiles=True)[0] == 0
        worst = 0.0
        for t in range(cfg.steps):
            si = synth.make_step_inputs(cfg, t)
            os_ = []
            for lay in lays:
                o = np.zeros((len(tiles), cfg.dv))
                assert lay.read(si, o=o)[0] == 0
                if (lay.count == cfg.window).any():
                    assert lay.flush(si, o=o)[0] == 0
                os_.append(o)
            worst = max(worst, rel(os_[1], os_[0]))
        assert worst < tol, (store, worst)


def test_pins_catch_planted_mistake():
    """The decay products of the triangular system starting one slot early
    (D(j,l) taking slot j's own decay) is caught, for GDN and for KDA."""
    for fam in ("gdn", "kda"):
        test_query_and_buffer_terms_against_dense_products(fam, 5)
        oracle.set_mutation(15)
        try:
            with pytest.raises(AssertionError):
                test_query_and_buffer_terms_against_dense_products(fam, 5)
        finally:
            oracle.set_mutation(0)
