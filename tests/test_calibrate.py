"""Pins of the offline calibration (basis and rank allocation).

The basis against closed forms on constructed state metrics and against
the objective evaluated by per-sample least squares; the allocation against
brute-force enumeration on small instances and against its own invariants
(feasibility, monotone error in the budget)."""
import itertools

import numpy as np
import pytest

from ssm_decode_amd import calibrate as cal


def _rot(rng, n):
    Q, _ = np.linalg.qr(rng.standard_normal((n, n)))
    return Q


def test_basis_closed_form_diagonal_metric():
    """E0 = diag(d), isotropic queries: E[z z^T] = E0, so the kept directions
    are the G largest entries of d and Omega* = e_i / sqrt(d_i)."""
    d = np.array([0.25, 4.0, 1.0, 9.0, 0.5, 2.0])
    b = cal.fit_basis(np.diag(d), np.eye(6), G=3)
    top = np.argsort(d)[::-1][:3]
    assert np.allclose(b.energy, np.sort(d)[::-1])
    for j, i in enumerate(top):
        col = b.omega[:, j]
        expect = np.zeros(6)
        expect[i] = 1.0 / np.sqrt(d[i])
        assert np.allclose(np.abs(col), np.abs(expect), atol=1e-12)
    assert b.residual == pytest.approx(np.sort(d)[:3].sum())


def test_basis_closed_form_rotated_metric_and_queries():
    """E0 = R diag(d) R^T with queries concentrated on chosen directions:
    E[z z^T] = E0^(1/2) Q E0^(1/2) has a known spectrum."""
    rng = np.random.default_rng(3)
    R = _rot(rng, 5)
    d = np.array([3.0, 2.0, 1.0, 0.5, 0.1])
    E0 = R @ np.diag(d) @ R.T
    s = np.array([0.1, 5.0, 1.0, 4.0, 0.2])          # query energy along R's columns
    Q = R @ np.diag(s) @ R.T
    b = cal.fit_basis(E0, Q, G=2)
    mu = np.sort(d * s)[::-1]
    assert np.allclose(b.energy, mu)
    keep = np.argsort(d * s)[::-1][:2]
    # Omega* spans E0^(-1/2) R[:, keep] = R[:, keep] / sqrt(d[keep])
    target = R[:, keep] / np.sqrt(d[keep])
    P = b.omega @ np.linalg.pinv(b.omega)
    assert np.allclose(P @ target, target, atol=1e-10)


@pytest.mark.parametrize("G", [1, 3, 5])
def test_basis_minimises_the_sampled_objective(G):
    """On a sample, L_G(Omega*) (each query solved by least squares) equals
    the residual energy, and random bases of the same size do worse."""
    rng = np.random.default_rng(10 + G)
    dk, dv, N, M = 8, 5, 40, 300
    scale = np.linspace(2.0, 0.1, dk)
    states = scale[None, :, None] * rng.standard_normal((N, dk, dv))
    qmix = rng.standard_normal((dk, dk)) * np.linspace(1.0, 0.2, dk)[None, :]
    queries = rng.standard_normal((M, dk)) @ qmix.T
    E0, Q = cal.moments(states, queries)
    b = cal.fit_basis(E0, Q, G)
    j = cal.objective(E0, queries, b.omega)
    assert j == pytest.approx(b.residual, rel=1e-9, abs=1e-12)
    for _ in range(20):
        assert cal.objective(E0, queries, rng.standard_normal((dk, G))) >= j - 1e-9


def test_basis_table_layout():
    rng = np.random.default_rng(4)
    bases = [cal.fit_basis(np.diag(rng.uniform(0.1, 2, 6)), np.eye(6), 4) for _ in range(3)]
    Pt = cal.basis_table(bases, [2, 0, 3])
    assert Pt.shape == (5, 6)
    assert np.array_equal(Pt[:2], bases[0].omega[:, :2].T)
    assert np.array_equal(Pt[2:], bases[2].omega[:, :3].T)


def _brute(err, traffic, budget):
    H, O = err.shape
    best = None
    for ch in itertools.product(range(O), repeat=H):
        ch = np.array(ch)
        if traffic[ch].sum() <= budget:
            e = err[np.arange(H), ch].sum()
            if best is None or e < best - 1e-15:
                best = e
    return best


def _instance(rng, H, r_max, dk=8, dv=4):
    err = np.stack([cal.rank_options(np.sort(rng.gamma(0.6, 1.0, dk))[::-1], r_max) for _ in range(H)])
    return err, cal.option_traffic(dk, dv, r_max)


@pytest.mark.parametrize("seed", range(12))
def test_allocation_against_brute_force(seed):
    """Feasible, never worse than the cheapest feasible uniform allocation,
    and within 2% of the brute-force optimum (equal on most instances)."""
    rng = np.random.default_rng(seed)
    H, r_max = 4, 4
    err, traffic = _instance(rng, H, r_max)
    budget = cal.mean_rank_budget(H, rng.uniform(1.0, 3.5), 8, 4)
    a = cal.allocate(err, traffic, budget)
    assert a.traffic <= budget
    assert a.error == pytest.approx(err[np.arange(H), a.choice].sum())
    opt = _brute(err, traffic, budget)
    assert a.error <= opt * 1.02 + 1e-12
    uni = [err[:, r].sum() for r in range(1, r_max + 1) if H * traffic[r] <= budget]
    assert a.error <= min(uni) + 1e-12


def test_allocation_exact_when_the_price_meets_the_budget():
    """Convex error curves and a budget that the price solution meets with
    no slack: the allocation is the brute-force optimum."""
    rng = np.random.default_rng(99)
    H, r_max = 5, 4
    err, traffic = _instance(rng, H, r_max)
    # the budget of the allocation at some price is met exactly by it
    ch = np.zeros(H, dtype=np.int64)
    for h in range(H):
        ch[h] = 1 + int(np.argmin(err[h, 1:] + 0.02 * traffic[1:]))
    budget = traffic[ch].sum()
    a = cal.allocate(err, traffic, budget)
    assert a.error == pytest.approx(_brute(err, traffic, budget), abs=1e-12)


def test_allocation_monotone_in_budget_and_takes_dense_when_affordable():
    rng = np.random.default_rng(7)
    H, r_max = 6, 4
    err, traffic = _instance(rng, H, r_max)
    prev = None
    for mean_rank in (1.0, 1.5, 2.0, 3.0, 4.0):
        a = cal.allocate(err, traffic, cal.mean_rank_budget(H, mean_rank, 8, 4))
        if prev is not None:
            assert a.error <= prev + 1e-12
        prev = a.error
    # a budget that pays for every head's state copy: everything dense, no error
    a = cal.allocate(err, traffic, H * traffic[cal.DENSE])
    assert a.error == 0.0 and (a.choice == cal.DENSE).all()
