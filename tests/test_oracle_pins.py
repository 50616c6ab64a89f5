"""Pins of the fp64 oracle against things other than itself.

Brute force with dense transition matrices (tests/bruteforce.py), closed
forms, algebraic special cases and numpy routines.  Each case runs the
three families.  A mutation test at the end plants known mistakes in the
oracle and checks that at least one of these pins fails for each.
"""
import numpy as np
import pytest

import oracle
from synth import round_bf16
from tests import bruteforce as bf
from tests.oracle_drive import single_tile, entry_step, run_sketch, run_replay, run_standard

FAMS = ("mamba2", "gdn", "kda")
TOL = 1e-12


def rel(x, y):
    x, y = np.asarray(x, float), np.asarray(y, float)
    return np.linalg.norm(x - y) / max(np.linalg.norm(y), 1e-300)


def _case(family, seed, dk=4, dv=3, W=4, T=12, r=2, unit_k=False):
    rng = np.random.default_rng(seed)
    S0 = rng.standard_normal((dk, dv))
    ents = bf.random_entries(rng, family, dk, dv, T, unit_k=unit_k)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, r)))
    Pt = Q.T.copy()
    Cm = rng.standard_normal((r, dk))          # any coefficient map
    A = rng.uniform(-0.5, 0.5)
    return S0, ents, Pt, Cm, A


# ------------------------------------------------- brute force (dense)
@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_standard_matches_dense_recurrence(family, seed):
    S0, ents, Pt, Cm, A = _case(family, seed)
    ref, _ = bf.standard_run(family, S0, [(q, k, v, g, b) for (q, k, v, g, b) in ents], A)
    lay = single_tile(family, 4, 3, 4, S0, Pt, Cm, A)
    outs = run_standard(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], ref[t]) < TOL, t


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("W", [1, 2, 3, 4])
def test_replay_matches_dense_and_standard(family, W):
    """P1/P2: ReplaySSM outputs equal the standard recurrence at every step;
    I-a: the state after a flush equals W naive per-step updates."""
    S0, ents, Pt, Cm, A = _case(family, 10 + W, W=W)
    ref, states = bf.standard_run(family, S0, ents, A)
    rep = bf.replay_run(family, S0, ents, W, A)
    lay = single_tile(family, 4, 3, W, S0, Pt, Cm, A)
    outs = run_replay(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], ref[t]) < TOL
        assert rel(rep[t], ref[t]) < TOL
    last_flush = (len(ents) // W) * W - 1
    assert rel(lay.S[0], states[last_flush]) < TOL


@pytest.mark.parametrize("family", FAMS)
@pytest.mark.parametrize("W,r", [(4, 2), (3, 1), (4, 4), (2, 3)])
def test_sketch_matches_dense_formulation(family, W, r):
    """I-d: sketched read U (C q~) + buffered term, with q~ and the buffered
    term from dense transition products; flush outputs exact (P2)."""
    S0, ents, Pt, Cm, A = _case(family, 20 + 7 * W + r, W=W, r=r)
    outs_ref, flushed, states, U = bf.sketch_run(family, S0, ents, W, Pt, Cm, A)
    std, _ = bf.standard_run(family, S0, ents, A)
    lay = single_tile(family, 4, 3, W, S0, Pt, Cm, A)
    outs, masks, counts = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert bool(masks[t][0]) == flushed[t]
        assert rel(outs[t][0], outs_ref[t]) < TOL, (t, outs[t][0], outs_ref[t])
        if flushed[t]:
            assert rel(outs[t][0], std[t]) < TOL
    assert rel(lay.S[0], states[-1]) < TOL
    assert rel(lay.U[0, :r].T, U) < TOL          # P7: U = S^T P


@pytest.mark.parametrize("family", FAMS)
def test_window_one_reduces_to_standard(family):
    """I-c: with W = 1 every step flushes; sketch == replay == standard,
    bitwise, in every store mode."""
    for store in ("exact", "f32"):
        S0, ents, Pt, Cm, A = _case(family, 33, W=1)
        S0 = S0.astype(np.float32).astype(np.float64)   # a stored fp32 state
        steps = [entry_step(family, e) for e in ents]
        a = run_standard(single_tile(family, 4, 3, 1, S0, Pt, Cm, A, store), steps)
        b = run_replay(single_tile(family, 4, 3, 1, S0, Pt, Cm, A, store), steps)
        c, masks, _ = run_sketch(single_tile(family, 4, 3, 1, S0, Pt, Cm, A, store), steps)
        for t in range(len(steps)):
            assert masks[t][0]
            assert np.array_equal(a[t], b[t]) and np.array_equal(a[t], c[t])


@pytest.mark.parametrize("family", FAMS)
def test_full_rank_sketch_is_exact(family):
    """I-b: r = dk, orthonormal P, C = P^T: the sketched read equals the
    exact read at every step."""
    dk, dv, W = 4, 3, 4
    S0, ents, _, _, A = _case(family, 44, W=W)
    Q, _ = np.linalg.qr(np.random.default_rng(5).standard_normal((dk, dk)))
    Pt = Q.T.copy()
    std, _ = bf.standard_run(family, S0, ents, A)
    lay = single_tile(family, dk, dv, W, S0, Pt, Pt.copy(), A)
    outs, _, _ = run_sketch(lay, [entry_step(family, e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-12


def test_mamba2_closed_form():
    """P3: S_T = (prod a) S0 + sum_i dt_i (prod_{t>i} a_t) k_i v_i^T."""
    dk, dv, W = 4, 3, 4
    S0, ents, Pt, Cm, A = _case("mamba2", 55, W=W, T=W)
    a = [np.exp(-g * np.exp(A)) for (_, _, _, g, _) in ents]
    ref = np.prod(a) * S0
    for i, (_, k, v, g, _) in enumerate(ents):
        ref = ref + g * np.prod(a[i + 1:]) * np.outer(k, v)
    lay = single_tile("mamba2", dk, dv, W, S0, Pt, Cm, A)
    run_sketch(lay, [entry_step("mamba2", e) for e in ents])
    assert rel(lay.S[0], ref) < TOL


def test_mamba2_decay_special_values():
    """The Mamba-2 decay at values known without its formula: with
    exp(A) = ln 2 a step of gate dt decays the state by 2^-dt, and gate 0
    leaves it unchanged and writes nothing.  S0 = I (2 x 2), one-hot keys
    and values, a window of three steps (dt = 1, 0, 2):
      after dt = 1, k = e0, v = e1:  S = [[1/2, 1], [0, 1/2]]
      after dt = 0:                  unchanged
      after dt = 2, k = e1, v = e0:  S = [[1/8, 1/4], [2, 1/8]]
    and the flush step's output for q = (1, 1) is S^T q = (17/8, 3/8)."""
    dk = dv = 2
    A = float(np.log(np.log(2.0)))
    e0, e1 = np.array([1.0, 0.0]), np.array([0.0, 1.0])
    q = np.array([1.0, 1.0])
    ents = [(q, e0, e1, 1.0, 0.0), (q, e0, e1, 0.0, 0.0), (q, e1, e0, 2.0, 0.0)]
    Pt = np.eye(2)
    lay = single_tile("mamba2", dk, dv, 3, np.eye(2), Pt, Pt.copy(), A)
    outs, _, _ = run_sketch(lay, [entry_step("mamba2", e) for e in ents])
    want = np.array([[0.125, 0.25], [2.0, 0.125]])
    assert np.abs(lay.S[0] - want).max() < 1e-14
    assert np.abs(outs[2][0] - np.array([2.125, 0.375])).max() < 1e-14


@pytest.mark.parametrize("r", [1, 2, 3])
def test_mamba2_span_pin(r):
    """P4: for Mamba-2 q~ is a scalar multiple of q, so if every query lies in
    span(P) the sketched read (C = P^T) is exact at any rank."""
    dk, dv, W = 6, 3, 4
    rng = np.random.default_rng(66 + r)
    S0, ents, _, _, A = _case("mamba2", 66 + r, dk=dk, dv=dv, W=W)
    Q, _ = np.linalg.qr(rng.standard_normal((dk, r)))
    ents = [(Q @ rng.standard_normal(r), k, v, g, b) for (q, k, v, g, b) in ents]
    std, _ = bf.standard_run("mamba2", S0, ents, A)
    lay = single_tile("mamba2", dk, dv, W, S0, Q.T.copy(), Q.T.copy(), A)
    outs, _, _ = run_sketch(lay, [entry_step("mamba2", e) for e in ents])
    for t in range(len(ents)):
        assert rel(outs[t][0], std[t]) < 1e-12
    # and a query off the span is not reproduced (the pin has teeth)
    if r < dk:
        off = [(rng.standard_normal(dk), k, v, g, b) for (q, k, v, g, b) in ents]
        std2, _ = bf.standard_run("mamba2", S0, off, A)
        lay2 = single_tile("mamba2", dk, dv, W, S0, Q.T.copy(), Q.T.copy(), A)
        outs2, masks2, _ = run_sketch(lay2, [entry_step("mamba2", e) for e in off])
        errs = [rel(outs2[t][0], std2[t]) for t in range(len(off)) if not masks2[t][0]]
        assert max(errs) > 1e-3


@pytest.mark.parametrize("family", ["gdn", "kda"])
def test_delta_rule_writes_value(family):
    """P5: alpha = 1 (g = 1), beta = 1, unit k: after the update S^T k = v."""
    dk, dv = 5, 4
    rng = np.random.default_rng(77)
    S0 = rng.standard_normal((dk, dv))
    k = rng.standard_normal(dk)
    k /= np.linalg.norm(k)
    v = rng.standard_normal(dv)
    g = np.ones(dk) if family == "kda" else 1.0
    e = (rng.standard_normal(dk), k, v, g, 1.0)
    lay = single_tile(family, dk, dv, 4, S0, np.eye(dk)[:1], np.eye(dk)[:1])
    run_standard(lay, [entry_step(family, e)])
    assert rel(lay.S[0].T @ k, v) < 1e-12


def test_kda_reduces_to_gdn_and_pure_decay():
    """P6: KDA with g = alpha 1 equals GDN; with beta = 0 both are pure decay."""
    dk, dv = 5, 4
    rng = np.random.default_rng(88)
    S0 = rng.standard_normal((dk, dv))
    Pt = np.eye(dk)[:2]
    ents = bf.random_entries(rng, "gdn", dk, dv, 6)
    kda_ents = [(q, k, v, np.full(dk, g), b) for (q, k, v, g, b) in ents]
    a = single_tile("gdn", dk, dv, 4, S0, Pt, Pt)
    b = single_tile("kda", dk, dv, 4, S0, Pt, Pt)
    oa = run_standard(a, [entry_step("gdn", e) for e in ents])
    ob = run_standard(b, [entry_step("kda", e) for e in kda_ents])
    for x, y in zip(oa, ob):
        assert rel(x, y) < 1e-12
    # beta = 0: pure decay
    gv = rng.uniform(0.5, 1.0, dk)
    e = (rng.standard_normal(dk), rng.standard_normal(dk), rng.standard_normal(dv), gv, 0.0)
    c = single_tile("kda", dk, dv, 4, S0, Pt, Pt)
    run_standard(c, [entry_step("kda", e)])
    assert rel(c.S[0], gv[:, None] * S0) < 1e-15
    e2 = (e[0], e[1], e[2], 0.7, 0.0)
    d = single_tile("gdn", dk, dv, 4, S0, Pt, Pt)
    run_standard(d, [entry_step("gdn", e2)])
    assert rel(d.S[0], 0.7 * S0) < 1e-15


def test_sketch_is_numpy_product():
    """P7: after the prime, U = S^T P equals numpy's S.T @ P."""
    rng = np.random.default_rng(99)
    dk, dv, r = 8, 5, 3
    S0 = rng.standard_normal((dk, dv))
    Pt = rng.standard_normal((r, dk))
    lay = single_tile("gdn", dk, dv, 4, S0, Pt, Pt)
    lay.flush(None, all_tiles=True)
    assert rel(lay.U[0, :r], (S0.T @ Pt.T).T) < 1e-14


def test_bf16_store_rounds_to_nearest_even():
    """Output stores round fp64 -> fp32 -> bf16 to nearest, ties to even:
    1 + 2^-8 is halfway between 1 and 1 + 2^-7 and rounds to 1;
    1 + 3*2^-8 is halfway between 1 + 2^-7 and 1 + 2^-6 and rounds up."""
    for val, want in [(1.0 + 2 ** -8, 1.0), (1.0 + 3 * 2 ** -8, 1.0 + 2 ** -6),
                      (1.0 + 2 ** -8 + 2 ** -20, 1.0 + 2 ** -7), (-(1.0 + 2 ** -8), -1.0)]:
        S0 = np.array([[val]])
        lay = oracle.OracleLayer("mamba2", 1, 1, 4, np.array([1], np.int32), np.array([0, 1], np.int32),
                                 np.ones((1, 1)), np.ones((1, 1)), np.array([0.0]), np.array([[0, 0]]),
                                 S0[None], 1, 1, state_store="exact", sketch_store="bf16", out_store="bf16")
        e = (np.array([1.0]), np.array([0.0]), np.array([0.0]), 0.0, 0.0)
        _, o = lay.full_step(entry_step("mamba2", e))
        assert o[0, 0] == want, (val, o[0, 0])
        lay.flush(None, all_tiles=True)
        assert lay.U[0, 0, 0] == want
        assert float(round_bf16(np.array([val]))[0]) == want


@pytest.mark.parametrize("family", FAMS)
def test_ragged_phase_closed_form(family):
    """P8: with flush offset o_b and an identity-padded ring of W-1-o_b
    entries, count_b(t) = (t - o_b) mod W after step t and sequence b flushes
    exactly at t = o_b (mod W); outputs match the dense formulation."""
    dk, dv, W, T = 3, 2, 4, 11
    rng = np.random.default_rng(123)
    ents = bf.random_entries(rng, family, dk, dv, T)
    Pt = np.eye(dk)[:2]
    for ob in range(W):
        S0 = rng.standard_normal((dk, dv))
        lay = single_tile(family, dk, dv, W, S0, Pt, Pt, 0.0, count0=W - 1 - ob)
        outs, masks, counts = run_sketch(lay, [entry_step(family, e) for e in ents])
        ref, flushed, _, _ = bf.sketch_run(family, S0, ents, W, Pt, Pt, 0.0, phase_count=W - 1 - ob)
        for t in range(T):
            assert int(counts[t][0]) == (t - ob) % W
            assert bool(masks[t][0]) == ((t - ob) % W == 0)
            assert flushed[t] == bool(masks[t][0])
            assert rel(outs[t][0], ref[t]) < 1e-12


def test_count_overflow_is_reported():
    """A ring already holding W entries is a skipped flush: read and replay
    report it and change nothing."""
    S0 = np.ones((2, 2))
    lay = single_tile("gdn", 2, 2, 2, S0, np.eye(2)[:1], np.eye(2)[:1], count0=2)
    e = (np.ones(2), np.ones(2), np.ones(2), 0.9, 0.5)
    rc, o = lay.read(entry_step("gdn", e))
    assert rc == oracle.ERR_COUNT and int(lay.count[0]) == 2
    rc, o = lay.replay_step(entry_step("gdn", e))
    assert rc == oracle.ERR_COUNT
    lay.count[0] = 3
    rc, _ = lay.flush(None, all_tiles=True)
    assert rc == oracle.ERR_COUNT


# ------------------------------------------------------------- mutations
def _all_pins_pass():
    try:
        for fam in FAMS:
            test_standard_matches_dense_recurrence(fam, 0)
            test_replay_matches_dense_and_standard(fam, 4)
            test_sketch_matches_dense_formulation(fam, 4, 2)
        test_mamba2_closed_form()
        test_delta_rule_writes_value("gdn")
    except AssertionError:
        return False
    return True


@pytest.mark.parametrize("mutation", list(range(1, 11)))
def test_pins_catch_planted_mistakes(mutation):
    """Each planted mistake (dropped buffered term, wrong erase sign, reversed
    pull-back, shifted sketch row, dropped decay, swapped KDA order, reversed
    flush order, wrong Mamba-2 write scale, un-pulled-back query, flush output
    from the old state) makes at least one pin fail."""
    assert _all_pins_pass()
    oracle.set_mutation(mutation)
    try:
        caught = not _all_pins_pass()
        if mutation == 6:       # KDA-only mistake
            try:
                test_standard_matches_dense_recurrence("kda", 1)
                caught = caught or False
            except AssertionError:
                caught = True
    finally:
        oracle.set_mutation(0)
    assert caught
    assert _all_pins_pass()
