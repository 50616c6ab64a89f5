"""Pins of the oracle's state-dependent coefficient map.

The flush writes each tile's map C from its new state S and the sketch rows
u_j it just stored (the project page's per-window flush panel,
C = (U^T U)^+ U^T S0^T; the paper's App. A.2.1 derives it as the best
coefficients for reproducing S0^T q~ from the sketch vectors, App. A.2.2
names the regularised solve).  The pins check it against numpy's SVD-based
least squares and pseudoinverse, against exactness on states the sketch
spans, and against the store's rounding; a mutation test plants mistakes.
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


def _basis(rng, dk, r):
    Q, _ = np.linalg.qr(rng.standard_normal((dk, r)))
    return Q.T.copy()


def _primed(family, S0, Pt, ridge, store="exact", sketch_store=None, A=0.3):
    dk, dv = S0.shape
    lay = single_tile(family, dk, dv, 4, S0, Pt, np.zeros_like(Pt), A, store=store,
                      coef="state", ridge=ridge, sketch_store=sketch_store)
    rc, _ = lay.flush(None, all_tiles=True)
    assert rc == 0
    return lay


def _ridge_lstsq(Uh, S, ridge):
    """C from min |S^T x - Uh^T c|^2 + lambda |c|^2 for every x, as one
    stacked least-squares problem solved by numpy (SVD)."""
    r = Uh.shape[0]
    lam = ridge * np.trace(Uh @ Uh.T) / r
    A = np.vstack([Uh.T, np.sqrt(lam) * np.eye(r)])
    b = np.vstack([S.T, np.zeros((r, S.shape[0]))])
    return np.linalg.lstsq(A, b, rcond=None)[0]


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("ridge", [0.3, 1e-3])
def test_state_map_is_ridge_least_squares(family, ridge):
    """The stored map equals the ridge least-squares solution computed by
    numpy's SVD solver from the stored sketch and the state (dk != dv, so a
    transposed operand cannot pass)."""
    rng = np.random.default_rng(11)
    dk, dv, r = 7, 5, 3
    S0 = rng.standard_normal((dk, dv))
    lay = _primed(family, S0, _basis(rng, dk, r), ridge)
    ref = _ridge_lstsq(lay.U[0, :r], lay.S[0], ridge)
    assert rel(lay.C[0, :r], ref) < 1e-12


@pytest.mark.parametrize("family", FAMS)
def test_state_map_after_flush_uses_new_state(family):
    """After a window of updates the map follows the flushed state, not the
    state the window started from."""
    rng = np.random.default_rng(12)
    dk, dv, r, W = 6, 5, 3, 4
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, W)
    lay = single_tile(family, dk, dv, W, S0, _basis(rng, dk, r), np.zeros((r, dk)), 0.3,
                      coef="state", ridge=1e-2)
    run_sketch(lay, [entry_step(family, e) for e in ents])
    assert lay.count[0] == 0
    ref = _ridge_lstsq(lay.U[0, :r], lay.S[0], 1e-2)
    assert rel(lay.C[0, :r], ref) < 1e-12


def test_state_map_is_pseudoinverse_product():
    """As the ridge goes to zero the map is the pages' (U^T U)^+ U^T S^T,
    here numpy's pseudoinverse of the sketch matrix times S^T."""
    rng = np.random.default_rng(13)
    dk, dv, r = 8, 6, 4
    S0 = rng.standard_normal((dk, dv))
    lay = _primed("gdn", S0, _basis(rng, dk, r), 1e-14)
    Umat = lay.U[0, :r].T                     # dv x r, columns u_j
    ref = np.linalg.pinv(Umat) @ S0.T         # r x dk
    assert rel(lay.C[0, :r], ref) < 1e-9


@pytest.mark.parametrize("family", FAMS)
def test_low_rank_state_read_is_exact(family):
    """A state of rank 2 lies in the span of any rank-3 sketch of it, so with
    the state-dependent map every read of the first window equals the exact
    read; the fixed map C = P^T is not exact on the same inputs."""
    rng = np.random.default_rng(14)
    dk, dv, r, W = 6, 5, 3, 6
    S0 = rng.standard_normal((dk, 2)) @ rng.standard_normal((2, dv))
    Pt = _basis(rng, dk, r)
    ents = bf.random_entries(rng, family, dk, dv, W - 1)
    std, _ = bf.standard_run(family, S0, ents, 0.3)
    steps = [entry_step(family, e) for e in ents]
    lay = single_tile(family, dk, dv, W, S0, Pt, np.zeros((r, dk)), 0.3, coef="state", ridge=1e-14)
    outs, _, _ = run_sketch(lay, steps)
    fixed = single_tile(family, dk, dv, W, S0, Pt, Pt.copy(), 0.3)
    fouts, _, _ = run_sketch(fixed, steps)
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-9
    assert max(rel(fouts[t][0], std[t]) for t in range(len(ents))) > 1e-3


@pytest.mark.parametrize("family", FAMS)
def test_full_rank_state_map_is_exact(family):
    """With r = dk the sketch spans the state's rows at every flush, so every
    read of every window is exact (the counterpart of the full-rank pin of
    the fixed map)."""
    rng = np.random.default_rng(15)
    dk, dv, W = 4, 5, 4
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, 12)
    std, _ = bf.standard_run(family, S0, ents, 0.3)
    lay = single_tile(family, dk, dv, W, S0, _basis(rng, dk, dk), np.zeros((dk, dk)), 0.3,
                      coef="state", ridge=1e-14)
    outs, _, _ = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-9


def test_state_map_from_rounded_sketch():
    """With a bf16 sketch the map is solved from the sketch as stored and then
    rounded to bf16: nearly every entry equals the rounded numpy solution
    from the stored rows, and none is more than one bf16 step away."""
    rng = np.random.default_rng(16)
    dk, dv, r = 32, 24, 8
    S0 = rng.standard_normal((dk, dv))
    lay = _primed("kda", S0, _basis(rng, dk, r), 1e-4, sketch_store="bf16")
    Uh = lay.U[0, :r]
    assert np.array_equal(Uh, round_bf16(Uh))
    ref = round_bf16(_ridge_lstsq(Uh, lay.S[0], 1e-4))
    got = lay.C[0, :r]
    assert np.array_equal(got, round_bf16(got))
    same = np.mean(got == ref)
    assert same >= 0.99, same
    assert np.all(np.abs(got - ref) <= 2.0 ** -7 * np.abs(ref) + 1e-300)


def test_zero_state_gives_zero_map():
    lay = _primed("mamba2", np.zeros((5, 4)), _basis(np.random.default_rng(17), 5, 2), 1e-4)
    assert np.all(lay.C == 0.0)


# ------------------------------------------------------------- mutations
def _map_pins_pass():
    try:
        for fam in FAMS:
            test_state_map_is_ridge_least_squares(fam, 0.3)
            test_state_map_after_flush_uses_new_state(fam)
        test_state_map_from_rounded_sketch()
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutation", [11, 12, 13])
def test_map_pins_catch_planted_mistakes(mutation):
    """A dropped ridge, a map solved from the sketch before its rounding, and
    a map formed from the state the window started from each fail a pin."""
    assert _map_pins_pass()
    oracle.set_mutation(mutation)
    try:
        caught = not _map_pins_pass()
    finally:
        oracle.set_mutation(0)
    assert caught
    assert _map_pins_pass()
