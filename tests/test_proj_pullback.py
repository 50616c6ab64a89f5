"""Pins of the oracle's coefficient computation with projected per-slot
factors (paper App. C.2): every appended slot keeps P_s = C (Gamma_s (.) k_s)
(r-dimensional), and a read forms C q~ = C (Gamma_{n-1} (.) q) -
sum_l beta_l d_l P_l with the coefficients d_l of the triangular system
(App. C.1).  Pinned against dense products of the explicit transition
matrices (whole decode runs with arbitrary bases and maps), against the
other two forms on random layers, and through the stored factors
themselves; a planted mistake in the factors' decay products is caught."""
import numpy as np
import pytest

import oracle
from tests import bruteforce as bf
from tests.oracle_drive import single_tile, entry_step, run_sketch

FAMS = ("gdn", "kda", "mamba2")


def rel(x, y):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("W", [2, 4, 7])
def test_decode_run_against_dense_products(family, W):
    """Arbitrary (non-orthonormal) basis and map, exact stores: every output
    of the projected form equals U (C q~) + o_buf (or S^T q at a flush), all
    formed from explicit matrices."""
    rng = np.random.default_rng(300 + W + 10 * FAMS.index(family))
    dk, dv, r = 6, 5, 4
    S0 = rng.standard_normal((dk, dv))
    Pt = rng.standard_normal((r, dk))
    Cm = rng.standard_normal((r, dk))
    ents = bf.random_entries(rng, family, dk, dv, 3 * W + 2)
    ref, _, _, _ = bf.sketch_run(family, S0, ents, W, Pt, Cm, 0.3)
    lay = single_tile(family, dk, dv, W, S0, Pt, Cm, 0.3, store="exact", pullback="proj")
    outs, _, _ = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], ref[t]) < 1e-11, t


@pytest.mark.parametrize("family", ("gdn", "kda"))
def test_stored_factors_are_the_projections(family):
    """After n appends the ring holds P_s = C (Gamma_s (.) k_s) with Gamma_s
    the cumulative product of the slots' decays, formed here with numpy."""
    rng = np.random.default_rng(77)
    dk, dv, r, W = 6, 5, 3, 8
    Cm = rng.standard_normal((r, dk))
    ents = bf.random_entries(rng, family, dk, dv, 5)
    lay = single_tile(family, dk, dv, W, rng.standard_normal((dk, dv)), rng.standard_normal((r, dk)),
                      Cm, store="exact", pullback="proj")
    run_sketch(lay, [entry_step(family, e) for e in ents])
    gam = np.ones(dk)
    for s, (_, k, _, g, _) in enumerate(ents):
        gam = gam * (np.full(dk, g) if family == "gdn" else np.asarray(g))
        assert rel(lay.rp[0, s, :r], Cm @ (gam * k)) < 1e-13, s


@pytest.mark.parametrize("family", FAMS)
def test_projected_form_matches_the_others_on_random_layers(family):
    """A layer of sketched tiles at mixed ring fills: the projected, parallel
    and serial forms agree to rounding with exact stores, and within the
    fp32 stores' rounding (factors, state, sketch, output) with f32 stores."""
    import synth
    from synth import LayerConfig
    cfg = LayerConfig(name="proj_" + family, family=family, batch=3, heads=4,
                      qk_groups=2 if family == "mamba2" else 4, dk=16, dv=32, window=6,
                      mean_rank=4, fixed_rank=None, act="f32", sketch="f32", steps=14,
                      ragged=True, seed=72)
    li = synth.make_layer_inputs(cfg)
    tiles = np.array([(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    for store, tol in (("exact", 1e-12), ("f32", 1e-6)):
        lays = [oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets,
                                   li.Pt, li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups,
                                   state_store=store, sketch_store=store, out_store=store,
                                   count0=li.count0[tiles[:, 0], tiles[:, 1]], pullback=pb)
                for pb in ("serial", "wy", "proj")]
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
            worst = max(worst, rel(os_[2], os_[0]), rel(os_[2], os_[1]))
        assert worst < tol, (store, worst)


def test_pins_catch_planted_mistake():
    """A factor formed with the decays of slots 0..s-1 instead of 0..s
    (slot s's own decay dropped) fails the dense pin, for GDN and KDA."""
    for fam in ("gdn", "kda"):
        test_decode_run_against_dense_products(fam, 4)
        oracle.set_mutation(16)
        try:
            with pytest.raises(AssertionError):
                test_decode_run_against_dense_products(fam, 4)
        finally:
            oracle.set_mutation(0)
