"""The seeded input generators: the published SplitMix64 outputs, the
distributions, the rank table rule (bit-exact properties), the bases and the
window phases."""
import numpy as np
import pytest

import synth
from synth import CONFIGS, gen, sweep_configs


def test_splitmix64_reference_outputs():
    """SplitMix64 with state 1234567 (the published test sequence): the first
    outputs are mix64(1234567 + k*gamma), k = 1, 2, 3."""
    want = [6457827717110365317, 3203168211198807973, 9817491932198370423]
    got = [int(gen.mix64(np.array([(1234567 + k * int(gen.GAMMA)) % (1 << 64)], dtype=np.uint64))[0])
           for k in (1, 2, 3)]
    assert got == want


def test_uniform_and_normal_moments():
    c = np.arange(200000, dtype=np.uint64)
    u = synth.uniform(7, 3, c)
    assert u.min() >= 0.0 and u.max() < 1.0
    assert abs(u.mean() - 0.5) < 0.005 and abs(u.var() - 1 / 12) < 0.002
    z = synth.normal(7, 3, c)
    assert abs(z.mean()) < 0.01 and abs(z.std() - 1.0) < 0.01
    # addressable: a slice equals the same counters generated alone
    assert np.array_equal(synth.normal(7, 3, c[1000:1010]), z[1000:1010])
    # threaded chunks do not change values
    big = np.arange(3 << 18, dtype=np.uint64)
    assert np.array_equal(synth.normal(9, 1, big)[-5:], synth.normal(9, 1, big[-5:]))


@pytest.mark.parametrize("cfg", [CONFIGS[n] for n in ("m2_b320", "gdn_b256", "kda_b256")]
                         + sweep_configs())
def test_rank_table(cfg):
    """P9: sum r_h = mean_rank * H, 2 <= r_h <= 16, offsets = exclusive prefix
    sum; the draw is deterministic; mean rank 16 forces every r_h = 16."""
    r = synth.draw_ranks(cfg)
    assert r.dtype == np.int32 and len(r) == cfg.heads
    assert int(r.sum()) == cfg.mean_rank * cfg.heads
    assert r.min() >= 2 and r.max() <= 16
    off = synth.rank_offsets(r)
    assert off[0] == 0 and np.array_equal(np.diff(off), r)
    assert np.array_equal(r, synth.draw_ranks(cfg))
    if cfg.mean_rank == 16:
        assert (r == 16).all()


def test_basis_is_orthonormal_per_head():
    cfg = CONFIGS["m2_b320"]
    li = synth.make_layer_inputs(cfg)
    for h in range(0, cfg.heads, 17):
        P = li.Pt[li.offsets[h]:li.offsets[h + 1]]
        assert np.abs(P @ P.T - np.eye(len(P))).max() < 1e-6
        assert np.array_equal(P, P.astype(np.float32).astype(np.float64))
    assert np.array_equal(li.C, li.Pt)


def test_phase_offsets():
    cfg = CONFIGS["m2_stress_b1024"]
    ph = synth.phase_offsets(cfg)
    assert ph.min() >= 0 and ph.max() < cfg.window and len(set(ph.tolist())) == cfg.window
    li = synth.make_layer_inputs(cfg.with_(batch=8))
    assert np.array_equal(li.count0, np.repeat((cfg.window - 1 - li.phase)[:, None], cfg.heads, 1))
    aligned = synth.phase_offsets(CONFIGS["m2_b320"])
    assert (aligned == 15).all()


@pytest.mark.parametrize("name", ["tiny_m2", "m2_b320", "gdn_b256", "kda_b256"])
def test_step_inputs_recipe(name):
    cfg = CONFIGS[name]
    si = synth.make_step_inputs(cfg, 3, b_idx=[0, 1])
    rnd = synth.round_f32 if cfg.act == "f32" else synth.round_bf16
    for x in (si.q, si.k, si.v):
        assert np.array_equal(x, rnd(x))
    if cfg.family == "mamba2":
        assert si.beta is None and si.gate.min() >= 0.0009 and si.gate.max() <= 0.1001
        assert np.array_equal(si.gate, rnd(si.gate))
    else:
        n = np.linalg.norm(si.q, axis=-1)
        assert np.abs(n - 1).max() < 1e-2
        assert si.beta.min() >= 0 and si.beta.max() < 1
        lo = 0.9 if cfg.family == "gdn" else 0.85
        assert si.gate.min() > lo - 1e-7 and si.gate.max() <= 1.0
    # a sequence subset equals the same rows of the full step
    full = synth.make_step_inputs(cfg, 3) if cfg.batch <= 8 else None
    if full is not None:
        assert np.array_equal(full.v[[0, 1]], si.v)


def test_torch_generator_matches_numpy():
    torch = pytest.importorskip("torch")
    from synth import torch_gen
    c = np.arange(100000, dtype=np.uint64)
    ct = torch.arange(100000, dtype=torch.int64)
    assert np.array_equal(synth.uniform(5, 12, c), torch_gen.uniform(5, 12, ct).numpy())
    zn = synth.normal(5, 12, c)
    zt = torch_gen.normal(5, 12, ct).numpy()
    assert np.abs(zn - zt).max() <= 4 * np.spacing(np.abs(zn).max())
    for name in ("m2_b320", "kda_b256"):
        cfg = CONFIGS[name].with_(batch=3)
        si = synth.make_step_inputs(cfg, 5)
        q, k, v, gate, beta = torch_gen.step_inputs(cfg, 5, "cpu")
        assert np.array_equal(si.q, q.float().numpy().astype(np.float64))
        assert np.array_equal(si.v, v.float().numpy().astype(np.float64))
        assert np.array_equal(si.gate, gate.float().numpy().astype(np.float64))
        S = torch_gen.initial_state(cfg, 1, 2, "cpu").numpy().astype(np.float64)
        assert np.array_equal(S, synth.initial_state(cfg, b_idx=[1]))
