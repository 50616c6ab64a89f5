"""Offline calibration of the sketch basis and the per-head ranks (host side).

Not on the decode path: it produces the inputs the path takes (the basis
P_h, written as the rows of Pt, and the rank table), once per model, from
calibration states and queries.  Everything here is float64 numpy.

Basis (project page "02 / How to Make a Sketch", offline sketching-matrix
panel; paper App. A.1).  The read reproduces S0^T q~ from the sketch
U = S0^T Omega, so the error of a query is the state-weighted distance of
q~ from the span of Omega.  Averaged over calibration states, the weight is
the state metric E0 = E[S0 S0^T], and with z = E0^(1/2) q~ the objective

    L_G(Omega) = E[ min_c | E0^(1/2) (q~ - Omega c) |^2 ]

is a projection error of z, minimised by the top-G eigenvectors P_G of the
uncentred second moment E[z z^T]:  Omega* = E0^(-1/2) P_G, with residual the
sum of the remaining eigenvalues.

Ranks (paper App. E).  Each head chooses among a dense fallback (exact, a
state copy read at every step) and the ranks r = 1..r_max, each with an
error score and a per-step traffic.  A traffic price makes the heads'
choices independent (each minimises error + price * traffic); the price is
set by bisection so that the total traffic meets the budget, the best
feasible allocation seen is kept, and the remaining slack is spent on
single-head substitutions that lower the total error.
"""
from __future__ import annotations

from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np


# ------------------------------------------------------------------ basis
def moments(states: np.ndarray, queries: np.ndarray):
    """Second moments of one head's calibration set.

    states [N][dk][dv]: full states at window boundaries; queries [M][dk]:
    effective queries.  Returns E0 = mean S S^T and Q = mean q~ q~^T (dk x dk)."""
    S = np.asarray(states, dtype=np.float64)
    q = np.asarray(queries, dtype=np.float64)
    E0 = np.einsum("nij,nkj->ik", S, S) / len(S)
    Q = q.T @ q / len(q)
    return E0, Q


@dataclass
class Basis:
    omega: np.ndarray        # [dk][G]: Omega* = E0^(-1/2) P_G
    energy: np.ndarray       # [dk] eigenvalues of E[z z^T], descending
    E0: np.ndarray           # the state metric used

    @property
    def residual(self) -> float:
        """L_G(Omega*): the energy in the eigen-directions not kept."""
        return float(self.energy[self.omega.shape[1]:].sum())

    def captured(self, g: Optional[int] = None) -> float:
        """Fraction of the output energy the first g directions keep."""
        g = self.omega.shape[1] if g is None else g
        tot = float(self.energy.sum())
        return float(self.energy[:g].sum()) / tot if tot > 0 else 1.0


def _sym_pow(M: np.ndarray, p: float, floor: float) -> np.ndarray:
    w, V = np.linalg.eigh((M + M.T) / 2)
    w = np.maximum(w, floor)
    return (V * w ** p) @ V.T


def fit_basis(E0: np.ndarray, Q: np.ndarray, G: int, rel_floor: float = 1e-9) -> Basis:
    """Omega* = E0^(-1/2) P_G from the state metric E0 and the query second
    moment Q = E[q~ q~^T]; E[z z^T] = E0^(1/2) Q E0^(1/2).  A singular E0
    has its eigenvalues floored at rel_floor times the largest, so that
    E0^(-1/2) exists (directions the states never excite cost no error)."""
    E0 = np.asarray(E0, dtype=np.float64)
    dk = E0.shape[0]
    if not 1 <= G <= dk:
        raise ValueError("G must lie in [1, dk]")
    floor = rel_floor * max(float(np.linalg.eigvalsh(E0).max()), 1e-300)
    half = _sym_pow(E0, 0.5, floor)
    Mz = half @ np.asarray(Q, dtype=np.float64) @ half
    w, V = np.linalg.eigh((Mz + Mz.T) / 2)
    order = np.argsort(w)[::-1]
    w, V = np.maximum(w[order], 0.0), V[:, order]
    omega = _sym_pow(E0, -0.5, floor) @ V[:, :G]
    return Basis(omega=omega, energy=w, E0=E0)


def objective(E0: np.ndarray, queries: np.ndarray, omega: np.ndarray) -> float:
    """L_G(Omega) on a sample of queries, each solved by least squares."""
    w, V = np.linalg.eigh(E0)
    half = (V * np.sqrt(np.maximum(w, 0.0))) @ V.T
    A = half @ omega
    Z = half @ np.asarray(queries, dtype=np.float64).T          # [dk][M]
    c, *_ = np.linalg.lstsq(A, Z, rcond=None)
    R = Z - A @ c
    return float((R * R).sum() / Z.shape[1])


def basis_table(bases: Sequence[Basis], ranks: Sequence[int]) -> np.ndarray:
    """The rows of Pt ([R][dk], the layout the decode path takes) for the
    heads' ranks: head h contributes the first r_h columns of its Omega*
    (none for a dense-fallback head, r_h = 0)."""
    rows = [b.omega[:, :r].T for b, r in zip(bases, ranks) if r > 0]
    dk = bases[0].omega.shape[0]
    return np.concatenate(rows) if rows else np.zeros((0, dk))


# ------------------------------------------------------------------ ranks
DENSE = 0          # option 0 of every head is the dense fallback


@dataclass
class Allocation:
    choice: np.ndarray       # [H] option per head: 0 dense, r >= 1 the rank
    error: float
    traffic: float
    price: float


def rank_options(energy: np.ndarray, r_max: int) -> np.ndarray:
    """Error of each option of one head from its energy spectrum: the dense
    fallback is exact (0); rank r leaves the energy beyond the first r
    directions, as a fraction of the total."""
    e = np.asarray(energy, dtype=np.float64)
    tot = e.sum()
    err = np.zeros(r_max + 1)
    for r in range(1, r_max + 1):
        err[r] = e[r:].sum() / tot if tot > 0 else 0.0
    return err


def option_traffic(dk: int, dv: int, r_max: int, elem_bytes: int = 2) -> np.ndarray:
    """Per-step read bytes of each option (paper App. D): the dense fallback
    reads its state copy, dk dv elements; rank r reads r (dk + dv) elements
    of sketch and map."""
    t = np.array([r * (dk + dv) for r in range(r_max + 1)], dtype=np.float64) * elem_bytes
    t[DENSE] = dk * dv * elem_bytes
    return t


def _choose(err: np.ndarray, traffic: np.ndarray, price: float) -> np.ndarray:
    cost = err + price * traffic[None, :]
    # ties go to the option with less traffic
    best = np.zeros(len(err), dtype=np.int64)
    for h in range(len(err)):
        c = cost[h]
        m = c.min()
        cand = np.nonzero(c <= m + 1e-15 * max(1.0, abs(m)))[0]
        best[h] = cand[np.argmin(traffic[cand])]
    return best


def allocate(err: np.ndarray, traffic: np.ndarray, budget: float,
             iters: int = 100) -> Allocation:
    """Per-head options under a total traffic budget.

    err [H][O]: error score of option o of head h; traffic [O]: its per-step
    bytes (the same for every head); budget: total bytes per step."""
    err = np.asarray(err, dtype=np.float64)
    traffic = np.asarray(traffic, dtype=np.float64)
    H = len(err)
    tot = lambda ch: float(traffic[ch].sum())
    toterr = lambda ch: float(err[np.arange(H), ch].sum())
    if tot(np.full(H, int(np.argmin(traffic)))) > budget:
        raise ValueError("budget below the cheapest allocation")
    best = None

    def consider(ch, price):
        nonlocal best
        if tot(ch) <= budget and (best is None or toterr(ch) < best.error - 1e-15):
            best = Allocation(ch.copy(), toterr(ch), tot(ch), price)

    # the price range: at hi every head takes its cheapest option
    spread = float((err.max(axis=1) - err.min(axis=1)).max()) if err.size else 0.0
    dt = np.diff(np.unique(traffic))
    hi = (spread + 1.0) / (dt.min() if dt.size else 1.0)
    lo = 0.0
    consider(_choose(err, traffic, lo), lo)
    consider(_choose(err, traffic, hi), hi)
    for _ in range(iters):
        mid = 0.5 * (lo + hi)
        ch = _choose(err, traffic, mid)
        consider(ch, mid)
        if tot(ch) > budget:
            lo = mid
        else:
            hi = mid
    # spend the slack: single-head substitutions that lower the error
    ch = best.choice.copy()
    while True:
        cur_t, cur_e = tot(ch), toterr(ch)
        gain, move = 0.0, None
        for h in range(H):
            for o in range(traffic.size):
                if o == ch[h]:
                    continue
                nt = cur_t - traffic[ch[h]] + traffic[o]
                de = err[h, ch[h]] - err[h, o]
                if nt <= budget and de > gain + 1e-15:
                    gain, move = de, (h, o)
        if move is None:
            break
        ch[move[0]] = move[1]
    return Allocation(ch, toterr(ch), tot(ch), best.price)


def mean_rank_budget(heads: int, mean_rank: float, dk: int, dv: int, elem_bytes: int = 2) -> float:
    """The traffic budget of a mean sketch rank: heads x mean_rank x (dk + dv)
    elements per step."""
    return heads * mean_rank * (dk + dv) * elem_bytes
