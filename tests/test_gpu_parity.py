"""HIP path vs oracle, element by element, through the C ABI (needs a GPU).

Tolerances (relative L2 over the compared tiles, per step for o, per flush
for S and U): 1e-5 for fp32 states, and for fp32 outputs / sketches; 1e-2
where q/k/v/o and U are bf16.  Ring counts are compared exactly for every
tile at every step, against the oracle and the closed form
count_b(t) = (t - o_b) mod W.
"""
import numpy as np
import pytest

from synth import CONFIGS, LayerConfig, sweep_configs

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _tiny(family, seed, **kw):
    base = dict(name=f"tiny_{family}", family=family, batch=2, heads=4, qk_groups=4, dk=16, dv=32,
                window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=32,
                ragged=False, seed=seed)
    base.update(kw)
    return LayerConfig(**base)


def _small(name, **kw):
    return CONFIGS[name].with_(name=name + "_small", **kw)


@pytest.fixture(scope="module", autouse=True)
def _lib():
    _need_gpu()
    from ssm_decode_amd import abi
    abi.load()


def run(cfg, method, **kw):
    from tests.gpu_parity import run_parity
    print(f"\n[parity] {cfg.name} {method} B={cfg.batch} H={cfg.heads} W={cfg.window} "
          f"Gbar={cfg.mean_rank} ragged={cfg.ragged}", flush=True)
    return run_parity(cfg, method, **kw)


# ------------------------------------------------------------- tiny, fp32
@pytest.mark.parametrize("method", ["sketch", "replay", "standard"])
def test_tiny_m2(method):
    run(CONFIGS["tiny_m2"], method)


@pytest.mark.parametrize("family,seed", [("gdn", 11), ("kda", 12)])
@pytest.mark.parametrize("method", ["sketch", "replay", "standard"])
def test_tiny_deltanet(family, seed, method):
    run(_tiny(family, seed), method)


@pytest.mark.parametrize("family,seed", [("mamba2", 1), ("gdn", 13), ("kda", 14)])
def test_tiny_ragged(family, seed):
    run(_tiny(family, seed, ragged=True, steps=19, batch=5), "sketch")


def test_full_rank_sketch_equals_standard():
    """r_h = dk, orthonormal P, C = P^T, fp32 sketch: the sketched read equals
    the exact read, so the GPU sketch path matches the oracle's standard path."""
    from tests.gpu_parity import rel_l2
    import synth
    import oracle
    from ssm_decode_amd import abi, feed
    cfg = CONFIGS["tiny_m2"].with_(name="tiny_m2_r16", fixed_rank=16, mean_rank=16)
    li = synth.make_layer_inputs(cfg)
    lay = feed.make_layer(cfg, li)
    feed.fill_state(lay, cfg, numpy_all=True)
    assert feed.prime(lay, li) == 0
    tiles = np.array([(b, h) for b in range(cfg.batch) for h in range(cfg.heads)])
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    std = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets, li.Pt,
                             li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups)
    step = lay.new_step()
    worst = 0.0
    for t in range(cfg.steps):
        feed.fill_step(step, cfg, t, numpy_all=True)
        assert lay.read(step) == 0 and lay.flush(step, abi.SKSSM_FLUSH_DUE) == 0
        _, o_ref = std.full_step(synth.make_step_inputs(cfg, t))
        torch.cuda.synchronize()
        e = rel_l2(step.o.reshape(-1, cfg.dv).cpu().numpy(), o_ref)
        worst = max(worst, e)
        assert e < 1e-5, (t, e)
    print(f"  rank-16 sketch vs standard: max rel-L2 {worst:.2e}")


# ------------------------- real head shapes, reduced batch, every tile, bf16
@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_small_batch_ragged(name):
    cfg = _small(name, batch=3, ragged=True, steps=40)
    run(cfg, "sketch")


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
@pytest.mark.parametrize("method", ["replay", "standard"])
def test_small_batch_baselines(name, method):
    cfg = _small(name, batch=2, ragged=True, steps=20)
    run(cfg, method)


@pytest.mark.parametrize("W,G", [(8, 4), (32, 16), (16, 4)])
def test_small_stress_points(W, G):
    base = CONFIGS["m2_stress_b1024"]
    cfg = base.with_(name=f"stress_w{W}_g{G}_small", batch=4, window=W, mean_rank=G,
                     steps=2 * W + 5)
    run(cfg, "sketch")


# -------------------- full batch (launch configuration of the benchmark),
# sampled tiles; the device generator fills the other sequences
def _full(name, steps=None, n_seq=4, n_head=4):
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS[name]
    tiles = sample_tiles(cfg, n_seq, n_head, seed=cfg.seed)
    return run(cfg, "sketch", steps=steps, tiles=tiles, numpy_all=False)


def test_full_m2_b320():
    _full("m2_b320")


def test_full_gdn_b256():
    _full("gdn_b256")


def test_full_kda_b256():
    _full("kda_b256")


@pytest.mark.parametrize("idx", list(range(9)))
def test_full_stress_sweep(idx):
    from tests.gpu_parity import sample_tiles
    cfg = sweep_configs()[idx]
    steps = cfg.steps if (cfg.window, cfg.mean_rank) == (16, 8) else 2 * cfg.window + 7
    tiles = sample_tiles(cfg, 4, 3, seed=cfg.seed)
    run(cfg, "sketch", steps=steps, tiles=tiles, numpy_all=False)


@pytest.mark.parametrize("name,W", [("m2_b320", 16), ("m2_b320", 32), ("gdn_b256", 16), ("kda_b256", 32)])
def test_read_at_every_ring_fill(name, W):
    """One sketched read from every ring fill n0 = 0..W-2 (identity-padded
    ring), so every lane position of the slot scans and broadcasts holds the
    step's own entry once."""
    import synth
    import oracle
    from ssm_decode_amd import feed
    from tests.gpu_parity import rel_l2, all_tiles, tol_out
    cfg = CONFIGS[name].with_(name=f"{name}_fill", batch=1, window=W)
    li = synth.make_layer_inputs(cfg)
    tiles = all_tiles(cfg)
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    worst = 0.0
    for n0 in range(W - 1):
        lay = feed.make_layer(cfg, li)
        feed.fill_state(lay, cfg, numpy_all=True)
        assert feed.prime(lay, li) == 0
        orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, W, li.ranks, li.offsets, li.Pt, li.C,
                                 li.A, tiles, S0, cfg.heads, cfg.qk_groups, state_store="f32",
                                 sketch_store=cfg.sketch, out_store=cfg.act)
        orc.flush(None, all_tiles=True)
        lay.count.fill_(n0)
        orc.count[:] = n0
        step = lay.new_step()
        feed.fill_step(step, cfg, 0, numpy_all=True)
        assert lay.read(step) == 0
        torch.cuda.synchronize()
        o_ref = np.zeros((len(tiles), cfg.dv))
        orc.read(synth.make_step_inputs(cfg, 0), o=o_ref)
        e = rel_l2(step.o.float().cpu().numpy().reshape(-1, cfg.dv), o_ref)
        worst = max(worst, e)
        assert e <= tol_out(cfg), (n0, e)
        assert (lay.count.cpu().numpy() == n0 + 1).all()
    print(f"  {name} W={W}: every ring fill, max rel-L2 {worst:.2e}")
