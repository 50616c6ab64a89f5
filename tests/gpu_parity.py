"""Drives the HIP path (through the C ABI) and the oracle side by side on the
same seeded inputs and compares them step by step (test infrastructure)."""
from __future__ import annotations

import sys
import time
from dataclasses import dataclass, field

import numpy as np
import torch

import oracle
import synth
from ssm_decode_amd import abi, feed

TOL_F32 = 1e-5
TOL_BF16 = 1e-2


def rel_l2(x, ref) -> float:
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / den) if den > 0 else float(np.linalg.norm(x))


def rel_l2_rows(x, ref):
    """Relative L2 error of every row (one tile's values per row): the
    per-tile gate.  A row whose reference is zero reports its absolute norm."""
    x = np.asarray(x, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    x = x.reshape(len(x), -1)
    ref = ref.reshape(len(ref), -1)
    num = np.linalg.norm(x - ref, axis=1)
    den = np.linalg.norm(ref, axis=1)
    return np.where(den > 0, num / np.where(den > 0, den, 1.0), num)


def tol_out(cfg) -> float:
    return TOL_F32 if cfg.act == "f32" else TOL_BF16


def tol_sketch(cfg) -> float:
    return TOL_F32 if cfg.sketch == "f32" else TOL_BF16


@dataclass
class ParityReport:
    name: str
    method: str
    steps: int
    tiles: int
    max_o: float = 0.0
    max_S: float = 0.0
    max_U: float = 0.0
    max_C: float = 0.0
    max_Sc: float = 0.0
    tile_o: float = 0.0              # worst per-tile relative L2 (o per step; S, U, C per flush)
    tile_S: float = 0.0
    tile_U: float = 0.0
    tile_C: float = 0.0
    worst_o_tile: tuple = ()         # (step, b, h) of tile_o
    flushes: int = 0
    count_mismatch: int = 0
    err_word: int = 0
    seconds: float = 0.0
    per_step_o: list = field(default_factory=list)

    def line(self) -> str:
        return (f"{self.name} {self.method}: steps={self.steps} tiles={self.tiles} "
                f"max rel-L2 o={self.max_o:.3e} S={self.max_S:.3e} U={self.max_U:.3e} C={self.max_C:.3e} "
                f"Scopy={self.max_Sc:.3e}; worst tile o={self.tile_o:.3e} at (t,b,h)={self.worst_o_tile} "
                f"S={self.tile_S:.3e} U={self.tile_U:.3e} C={self.tile_C:.3e}; "
                f"flush-steps={self.flushes} count-mismatch={self.count_mismatch} "
                f"err={self.err_word} ({self.seconds:.1f}s)")


def sample_tiles(cfg, n_seq: int, n_head: int, seed: int = 0) -> np.ndarray:
    """Sequences spread over the batch (first, last, random) x heads spread
    over the head range (first, last, random)."""
    rng = np.random.default_rng(1000 + seed)
    bs = {0, cfg.batch - 1} | set(rng.choice(cfg.batch, size=min(cfg.batch, n_seq), replace=False).tolist())
    hs = {0, cfg.heads - 1} | set(rng.choice(cfg.heads, size=min(cfg.heads, n_head), replace=False).tolist())
    return np.array([(b, h) for b in sorted(bs) for h in sorted(hs)], dtype=np.int64)


def all_tiles(cfg) -> np.ndarray:
    return np.array([(b, h) for b in range(cfg.batch) for h in range(cfg.heads)], dtype=np.int64)


def run_parity(cfg, method: str = "sketch", steps: int = None, tiles: np.ndarray = None,
               numpy_all: bool = True, li: synth.LayerInputs = None, log=True,
               coef: str = "fixed", ridge: float = 1e-4, pullback: str = "serial",
               flush: str = "due", plant: dict = None) -> ParityReport:
    """coef = "state": the flush forms each tile's own coefficient map with the
    relative ridge ``ridge`` (both sides use its fp32 value) and the maps of
    the flushed tiles are compared too.  pullback = "wy": both sides evaluate
    the effective query of a GDN/KDA read from the triangular system over
    the buffered slots.  flush = "list": the sketch path flushes through
    sketchssm_flush_seqs with each step's due sequences (from the window
    phases) instead of the due-flag flush; flush = "scan": through
    sketchssm_flush with SKSSM_FLUSH_DUE_SCAN (the due sequences listed on the
    device); flush = "close" (aligned phases): the step that closes every
    window runs sketchssm_flush with SKSSM_FLUSH_CLOSE instead of the read and
    the due-flag flush (the oracle still reads, then flushes).

    Gates: the relative L2 error pooled over the compared tiles, and the same
    error of every tile on its own (o per step; S, U and C per flush).

    plant: a mistake planted in the oracle's expected values on the CPU, to
    show that the checker catches it: {"o": (step, tile, rel)} scales one
    tile's expected output at one step by (1 + rel); {"S": (flush, tile,
    rel)} and {"U": (flush, tile, rel)} do the same to one tile's expected
    state or sketch at the given flush step (counted from 0)."""
    plant = plant or {}
    t0 = time.time()
    steps = cfg.steps if steps is None else steps
    li = synth.make_layer_inputs(cfg) if li is None else li
    tiles = all_tiles(cfg) if tiles is None else tiles
    seqs = np.unique(tiles[:, 0])
    seq_rows = np.full(cfg.batch, -1, dtype=np.int64)
    seq_rows[seqs] = np.arange(len(seqs))
    W = cfg.window

    # --- HIP side
    lay = feed.make_layer(cfg, li, coef=coef, ridge=ridge, pullback=pullback)
    feed.fill_state(lay, cfg, exact_seqs=seqs, numpy_all=numpy_all)
    # --- oracle side
    S0s = synth.initial_state(cfg, b_idx=seqs)
    S0_t = S0s[seq_rows[tiles[:, 0]], tiles[:, 1]]
    orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, W, li.ranks, li.offsets, li.Pt, li.C, li.A,
                             tiles, S0_t, cfg.heads, cfg.qk_groups, state_store="f32",
                             sketch_store=cfg.sketch, out_store=cfg.act, coef=coef,
                             ridge=float(np.float32(ridge)), pullback=pullback)
    count0_t = li.count0[tiles[:, 0], tiles[:, 1]]
    if method == "sketch":
        assert feed.prime(lay, li) == 0
        rc, _ = orc.flush(None, all_tiles=True)
        assert rc == 0
    else:
        lay.count.copy_(torch.from_numpy(li.count0).to(lay.device))
    orc.count[:] = count0_t if method != "standard" else 0

    rep = ParityReport(cfg.name, method + ("" if coef == "fixed" else "/state-map")
                       + ("" if pullback == "serial" else "/wy"), steps, len(tiles))

    def compare_maps(sel):
        C_gpu = lay.Cstate[tiles[sel, 0]].float().cpu().numpy().astype(np.float64)
        Cg, Co = [], []
        for i, ti in enumerate(sel):
            h = tiles[ti, 1]
            off, r = li.offsets[h], li.ranks[h]
            Cg.append(C_gpu[i, off:off + r])
            Co.append(orc.C[ti, :r])
            if r:
                rep.tile_C = max(rep.tile_C, rel_l2(Cg[-1], Co[-1]))
        if Cg and sum(c.size for c in Cg):
            rep.max_C = max(rep.max_C, rel_l2(np.concatenate(Cg), np.concatenate(Co)))

    if method == "sketch" and coef == "state":
        torch.cuda.synchronize()
        compare_maps(np.arange(len(tiles)))
    step = lay.new_step()
    tb = torch.from_numpy(tiles[:, 0]).to(lay.device)
    th = torch.from_numpy(tiles[:, 1]).to(lay.device)
    t_o, t_s = tol_out(cfg), tol_sketch(cfg)

    def due_list(t):
        # sequences whose window closes at step t: count after the read == W
        due = np.nonzero((t - li.phase) % W == 0)[0].astype(np.int32)
        return torch.from_numpy(due).to(lay.device)

    for t in range(steps):
        feed.fill_step(step, cfg, t, exact_seqs=seqs, numpy_all=numpy_all)
        si = synth.make_step_inputs(cfg, t, b_idx=seqs)
        o_ref = np.zeros((len(tiles), cfg.dv))
        if method == "sketch":
            if flush == "close":
                assert (li.phase == li.phase[0]).all(), "the closing flush needs an aligned phase"
                if (t - int(li.phase[0])) % W == 0:    # every window closes at this step
                    assert lay.flush(step, abi.SKSSM_FLUSH_CLOSE) == 0
                else:
                    assert lay.read(step) == 0
            else:
                assert lay.read(step) == 0
                if flush == "list":
                    assert lay.flush_seqs(step, due_list(t)) == 0
                elif flush == "scan":
                    assert lay.flush(step, abi.SKSSM_FLUSH_DUE_SCAN) == 0
                else:
                    assert lay.flush(step, abi.SKSSM_FLUSH_DUE) == 0
            # (the oracle's window: read, then flush, whatever the HIP path ran)
            rc, _ = orc.read(si, seq_rows=seq_rows, o=o_ref)
            assert rc == 0
            due = orc.count == W
            if due.any():
                rc, _ = orc.flush(si, seq_rows=seq_rows, o=o_ref)
                assert rc == 0
        elif method == "replay":
            assert lay.replay_step(step) == 0
            rc, _ = orc.replay_step(si, seq_rows=seq_rows, o=o_ref)
            assert rc == 0
            due = orc.count == 0
        elif method == "standard":
            assert lay.full_step(step) == 0
            rc, _ = orc.full_step(si, seq_rows=seq_rows, o=o_ref)
            assert rc == 0
            due = np.ones(len(tiles), dtype=bool)
        else:
            raise ValueError(method)
        torch.cuda.synchronize()
        o_gpu = step.o[tb, th].float().cpu().numpy().astype(np.float64)
        if "o" in plant and plant["o"][0] == t:
            o_ref = o_ref.copy()
            o_ref[plant["o"][1]] *= 1.0 + plant["o"][2]
        e = rel_l2(o_gpu, o_ref)
        rep.per_step_o.append(e)
        rep.max_o = max(rep.max_o, e)
        et = rel_l2_rows(o_gpu, o_ref)
        if et.max() > rep.tile_o:
            i = int(et.argmax())
            rep.tile_o = float(et[i])
            rep.worst_o_tile = (t, int(tiles[i, 0]), int(tiles[i, 1]))
        if method != "standard":
            cnt = lay.count.cpu().numpy()
            want = (t - li.phase[:, None]) % W
            rep.count_mismatch += int((cnt != np.broadcast_to(want, cnt.shape)).sum())
            rep.count_mismatch += int((cnt[tiles[:, 0], tiles[:, 1]] != orc.count).sum())
        if due.any():
            fi = rep.flushes
            rep.flushes += 1
            sel = np.nonzero(due)[0]
            sb = torch.from_numpy(tiles[sel, 0]).to(lay.device)
            sh = torch.from_numpy(tiles[sel, 1]).to(lay.device)
            S_gpu = lay.S[sb, sh].cpu().numpy().astype(np.float64)
            S_ref = orc.S[sel]
            if "S" in plant and plant["S"][0] == fi and plant["S"][1] in sel:
                S_ref = S_ref.copy()
                S_ref[int(np.nonzero(sel == plant["S"][1])[0][0])] *= 1.0 + plant["S"][2]
            rep.max_S = max(rep.max_S, rel_l2(S_gpu, S_ref))
            rep.tile_S = max(rep.tile_S, float(rel_l2_rows(S_gpu, S_ref).max()))
            if method == "sketch":
                U_gpu = lay.U[tiles[sel, 0]].float().cpu().numpy().astype(np.float64)
                Ug, Uo = [], []
                for i, ti in enumerate(sel):
                    h = tiles[ti, 1]
                    off, r = li.offsets[h], li.ranks[h]
                    Ug.append(U_gpu[i, off:off + r])
                    uo = orc.U[ti, :r]
                    if "U" in plant and plant["U"][0] == fi and plant["U"][1] == ti:
                        uo = uo * (1.0 + plant["U"][2])
                    Uo.append(uo)
                    if r:
                        rep.tile_U = max(rep.tile_U, rel_l2(Ug[-1], Uo[-1]))
                if Ug and sum(u.size for u in Ug):
                    rep.max_U = max(rep.max_U, rel_l2(np.concatenate(Ug), np.concatenate(Uo)))
                if coef == "state":
                    compare_maps(sel)
                dense = [ti for ti in sel if li.ranks[tiles[ti, 1]] == 0]
                if dense:                           # dense-fallback tiles: their state copies
                    slot = {int(hd): i for i, hd in enumerate(lay.dense_heads)}
                    db = torch.from_numpy(tiles[dense, 0]).to(lay.device)
                    dh = torch.tensor([slot[int(tiles[ti, 1])] for ti in dense], device=lay.device)
                    Sc_gpu = lay.Scopy[db, dh].float().cpu().numpy().astype(np.float64)
                    rep.max_Sc = max(rep.max_Sc, rel_l2(Sc_gpu, orc.Sc[dense]))
        if log and (t % 16 == 15 or t == steps - 1):
            print(f"  [{cfg.name} {rep.method}] step {t + 1}/{steps} max o={rep.max_o:.2e} "
                  f"S={rep.max_S:.2e} U={rep.max_U:.2e} C={rep.max_C:.2e}", flush=True)
        assert e <= t_o, f"{cfg.name} {method} step {t}: rel-L2(o) = {e:.3e} > {t_o}"
        assert rep.tile_o <= t_o, (f"{cfg.name} {method} step {t}: per-tile rel-L2(o) = "
                                   f"{rep.tile_o:.3e} > {t_o} at (t,b,h)={rep.worst_o_tile}")
    rep.err_word = lay.error_word()
    rep.seconds = time.time() - t0
    assert rep.count_mismatch == 0, rep.line()
    assert rep.max_S <= TOL_F32, rep.line()
    assert rep.max_U <= t_s, rep.line()
    assert rep.max_C <= t_s, rep.line()
    assert rep.max_Sc <= t_s, rep.line()
    assert rep.tile_S <= TOL_F32, "per-tile S: " + rep.line()
    assert rep.tile_U <= t_s, "per-tile U: " + rep.line()
    assert rep.tile_C <= t_s, "per-tile C: " + rep.line()
    assert rep.err_word == 0, rep.line()
    if log:
        print("  " + rep.line(), flush=True)
        sys.stdout.flush()
    return rep
