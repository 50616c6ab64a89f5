"""A calibrated basis on the decode path (needs a GPU).

Synthetic states with a decaying spectrum (no model, no data set): the
basis fitted offline from calibration states and queries (Omega* =
E0^(-1/2) P_G) gives the GPU's sketched reads, with the state-dependent map,
a smaller error against the exact read than a random orthonormal basis of
the same rank; the GPU outputs also match the oracle run with the same
calibrated basis."""
import numpy as np
import pytest

from synth import LayerConfig

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_decode_amd import abi
    abi.load()


def _structured_states(rng, B, H, dk, dv):
    """Per head a shared column space with a decaying spectrum, per sequence
    its own mixing, plus a little isotropic noise."""
    S = np.zeros((B, H, dk, dv))
    for h in range(H):
        Qk, _ = np.linalg.qr(rng.standard_normal((dk, dk)))
        sig = 0.5 * np.exp(-np.arange(dk) / 4.0)
        for b in range(B):
            S[b, h] = (Qk * sig) @ rng.standard_normal((dk, dv)) / np.sqrt(dv) \
                + 0.002 * rng.standard_normal((dk, dv))
    return S.astype(np.float32).astype(np.float64)


def _run(cfg, li, S0, Pt, steps, coef):
    """GPU sketch path and the exact ReplaySSM path on the same inputs; the
    oracle sketch path for parity.  Returns (relative errors vs exact, max
    parity error vs oracle)."""
    import oracle
    import synth
    from ssm_decode_amd import abi, feed
    from tests.gpu_parity import rel_l2
    Pt = Pt.astype(np.float32).astype(np.float64)     # the basis as the device stores it
    li = synth.LayerInputs(cfg=cfg, ranks=li.ranks, offsets=li.offsets, Pt=Pt, C=Pt.copy(), A=li.A,
                           phase=li.phase, count0=li.count0)
    ls = feed.make_layer(cfg, li, coef=coef, ridge=1e-4)
    lr = feed.make_layer(cfg, li)
    for lay in (ls, lr):
        lay.S.copy_(torch.from_numpy(S0).float().cuda())
    assert feed.prime(ls, li) == 0
    lr.count.copy_(torch.from_numpy(li.count0).cuda())
    tiles = np.array([(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])
    orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets, Pt, Pt.copy(),
                             li.A, tiles, S0.reshape(-1, cfg.dk, cfg.dv), cfg.heads, cfg.qk_groups,
                             state_store="f32", sketch_store=cfg.sketch, out_store=cfg.act, coef=coef,
                             ridge=float(np.float32(1e-4)))
    assert orc.flush(None, all_tiles=True)[0] == 0
    ss, sr = ls.new_step(), lr.new_step()
    errs, par = [], 0.0
    for t in range(steps):
        feed.fill_step(ss, cfg, t, numpy_all=True)
        feed.fill_step(sr, cfg, t, numpy_all=True)
        assert ls.read(ss) == 0 and ls.flush(ss, abi.SKSSM_FLUSH_DUE) == 0
        assert lr.replay_step(sr) == 0
        si = synth.make_step_inputs(cfg, t)
        o = np.zeros((len(tiles), cfg.dv))
        assert orc.read(si, o=o)[0] == 0
        if (orc.count == cfg.window).any():
            assert orc.flush(si, o=o)[0] == 0
        torch.cuda.synchronize()
        og = ss.o.reshape(-1, cfg.dv).double().cpu().numpy()
        par = max(par, rel_l2(og, o))
        if (t + 1) % cfg.window:                       # non-flush steps only
            errs.append(rel_l2(og, sr.o.reshape(-1, cfg.dv).double().cpu().numpy()))
    return np.array(errs), par


def test_calibrated_basis_beats_random():
    import synth
    from ssm_decode_amd import calibrate as cal
    cfg = LayerConfig(name="calib_m2", family="mamba2", batch=8, heads=4, qk_groups=1, dk=64, dv=64,
                      window=8, mean_rank=8, fixed_rank=8, act="f32", sketch="f32", steps=24,
                      ragged=False, seed=77)
    li = synth.make_layer_inputs(cfg)
    rng = np.random.default_rng(5)
    S0 = _structured_states(rng, cfg.batch, cfg.heads, cfg.dk, cfg.dv)
    # calibration set: the layer's own states and independent isotropic
    # queries (a Mamba-2 effective query is a multiple of the query)
    bases = []
    for h in range(cfg.heads):
        E0, Q = cal.moments(S0[:, h], rng.standard_normal((512, cfg.dk)))
        bases.append(cal.fit_basis(E0, Q, 8))
    Pt_cal = cal.basis_table(bases, li.ranks)
    Pt_rnd = np.concatenate([np.linalg.qr(rng.standard_normal((cfg.dk, 8)))[0].T
                             for _ in range(cfg.heads)])
    e_cal, p_cal = _run(cfg, li, S0, Pt_cal, cfg.steps, "state")
    e_rnd, p_rnd = _run(cfg, li, S0, Pt_rnd, cfg.steps, "state")
    print(f"\n  sketched-read error vs exact: calibrated {e_cal.mean():.4f}, random {e_rnd.mean():.4f}; "
          f"captured energy {np.mean([b.captured() for b in bases]):.3f}; "
          f"parity vs oracle {p_cal:.2e} / {p_rnd:.2e}", flush=True)
    assert p_cal <= 1e-5 and p_rnd <= 1e-5
    assert e_cal.mean() < 0.8 * e_rnd.mean()
