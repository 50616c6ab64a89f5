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


@pytest.mark.parametrize("dk,dv", [(64, 64), (128, 128)])
@pytest.mark.parametrize("W", [16, 32])
def test_m2_other_head_shapes(dk, dv, W):
    """Mamba-2 at the other supported head shapes, both ring capacities,
    every tile, ragged: the read splits a head's columns over two or four
    16-lane rows where its loads would not fit five waves per SIMD (128
    columns, or a 32-slot ring)."""
    cfg = _small("m2_b320", batch=3, ragged=True, steps=2 * W + 5, dk=dk, dv=dv, window=W)
    run(cfg, "sketch")


@pytest.mark.parametrize("W", [16, 32])
def test_m2_group_not_a_multiple_of_the_wave(W):
    """Five heads per B/C group at the real head shape: the last read wave
    of every group holds one head of the group (four heads a wave at W = 16,
    two at W = 32) and lanes past it take no rows; every tile, ragged,
    2W + 5 steps."""
    cfg = CONFIGS["m2_b320"].with_(name=f"m2_hpg5_w{W}", heads=20, qk_groups=4, batch=3, window=W,
                                   ragged=True, steps=2 * W + 5)
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
    """Every sweep point at batch 1024 for the workload's full 512 steps
    (16 to 64 windows), on sampled tiles."""
    from tests.gpu_parity import sample_tiles
    cfg = sweep_configs()[idx]
    tiles = sample_tiles(cfg, 4, 3, seed=cfg.seed)
    rep = run(cfg, "sketch", steps=cfg.steps, tiles=tiles, numpy_all=False)
    assert rep.steps == 512 and rep.flushes >= cfg.steps // cfg.window


# ------------- the flush of listed sequences (sketchssm_flush_seqs) vs oracle
@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_flush_list_small_batch(name):
    cfg = CONFIGS[name].with_(name=name + "_list", batch=5, ragged=True, steps=40)
    run(cfg, "sketch", flush="list")


def test_flush_list_stress_w32():
    """The batch-1024 W = 32 stress point, flushed through the caller's
    list of due sequences, for the full 512 steps on sampled tiles."""
    from tests.gpu_parity import sample_tiles
    cfg = [c for c in sweep_configs() if (c.window, c.mean_rank) == (32, 8)][0]
    tiles = sample_tiles(cfg, 4, 3, seed=cfg.seed + 1)
    run(cfg, "sketch", steps=cfg.steps, tiles=tiles, numpy_all=False, flush="list")


# ------------- the flush over a device-side list of due sequences vs oracle
@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_flush_scan_small_batch(name):
    cfg = CONFIGS[name].with_(name=name + "_scan", batch=5, ragged=True, steps=40)
    run(cfg, "sketch", flush="scan")


def test_flush_scan_state_map_and_dense_heads():
    """The scan flush's other instantiations: the state-dependent map (KDA)
    and layers with dense-fallback heads (Mamba-2, GDN), ragged, every
    tile."""
    run(CONFIGS["kda_b256"].with_(name="kda_scan_map", batch=3, ragged=True, steps=36), "sketch",
        coef="state", flush="scan")
    run(CONFIGS["m2_b320"].with_(name="m2_scan_dense", batch=3, ragged=True, steps=36,
                                 dense_heads=(0, 77)), "sketch", flush="scan")
    run(CONFIGS["gdn_b256"].with_(name="gdn_scan_dense", batch=3, ragged=True, steps=36,
                                  dense_heads=(5,)), "sketch", flush="scan")


def test_flush_scan_batch_over_one_scan_chunk():
    """A batch of 2,500 sequences: the scan lists the due sequences over
    three chunks of 1,024 (a running base carried between chunks); small
    heads, ragged, W = 4, sampled tiles in every chunk."""
    import numpy as np
    from synth import LayerConfig
    cfg = LayerConfig(name="tiny_m2_b2500_scan", family="mamba2", batch=2500, heads=4, qk_groups=4, dk=16,
                      dv=32, window=4, mean_rank=4, fixed_rank=4, act="bf16", sketch="bf16", steps=14,
                      ragged=True, seed=91)
    tiles = np.array([(b, h) for b in (0, 1, 1023, 1024, 1500, 2047, 2048, 2499) for h in (0, 3)],
                     dtype=np.int64)
    run(cfg, "sketch", tiles=tiles, numpy_all=False, flush="scan")


@pytest.mark.parametrize("W,G", [(32, 8), (8, 16)])
def test_flush_scan_stress(W, G):
    """Batch 1024, ragged, flushed through SKSSM_FLUSH_DUE_SCAN for the full
    512 steps on sampled tiles."""
    from tests.gpu_parity import sample_tiles
    cfg = [c for c in sweep_configs() if (c.window, c.mean_rank) == (W, G)][0]
    tiles = sample_tiles(cfg, 4, 3, seed=cfg.seed + 2)
    run(cfg, "sketch", steps=cfg.steps, tiles=tiles, numpy_all=False, flush="scan")


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_flush_scan_aligned_full_batch(name):
    """The aligned full-batch layers (every tile due at once: the scan
    flush's workgroups each take several tiles) on sampled tiles, three
    windows."""
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS[name]
    run(cfg, "sketch", steps=3 * cfg.window, tiles=sample_tiles(cfg, 4, 4, seed=cfg.seed + 1),
        numpy_all=False, flush="scan")


# ------------- the closing flush: the step that closes every window, without its read
@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_flush_close_small_batch(name):
    """SKSSM_FLUSH_CLOSE at every closing step of an aligned phase (the
    step's own entry taken from the step inputs, no read at that step),
    every tile, 2W + 8 steps; against the oracle's read-then-flush."""
    cfg = CONFIGS[name].with_(name=name + "_close", batch=3, steps=2 * CONFIGS[name].window + 8)
    run(cfg, "sketch", flush="close")


def test_flush_close_other_instantiations():
    """The closing flush with the state-dependent map (GDN), with
    dense-fallback heads (Mamba-2, KDA), with a 32-slot ring at the real
    delta-rule head shape (GDN) and with W = 1 (Mamba-2: every step closes
    its window with an empty ring)."""
    run(CONFIGS["gdn_b256"].with_(name="gdn_close_map", batch=3, steps=36), "sketch",
        coef="state", flush="close")
    run(CONFIGS["m2_b320"].with_(name="m2_close_dense", batch=3, steps=36, dense_heads=(0, 77)),
        "sketch", flush="close")
    run(CONFIGS["kda_b256"].with_(name="kda_close_dense", batch=3, steps=36, dense_heads=(5,)),
        "sketch", flush="close")
    run(CONFIGS["gdn_b256"].with_(name="gdn_close_w32", batch=2, window=32, steps=70), "sketch",
        flush="close")
    run(CONFIGS["m2_b320"].with_(name="m2_close_w1", batch=2, window=1, steps=6), "sketch",
        flush="close")


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_flush_close_full_batch(name):
    """The aligned full-batch layers with the closing flush (the benchmark's
    configuration) on sampled tiles, three windows."""
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS[name]
    run(cfg, "sketch", steps=3 * cfg.window, tiles=sample_tiles(cfg, 4, 4, seed=cfg.seed + 3),
        numpy_all=False, flush="close")


# ------------- the delta rule's 32-slot chunked flush at the real head shape
@pytest.mark.parametrize("flush", ["due", "list", "scan"])
@pytest.mark.parametrize("name", ["gdn_b256", "kda_b256"])
def test_delta_rule_w32_real_heads(name, flush):
    """dk = dv = 128 with W = 32: the chunked flush applies 32 entries (two
    16-entry blocks of the triangular system), every tile, ragged phases,
    2W + 3 steps; through the due-flag flush, the caller's list and the
    device-side due list."""
    cfg = CONFIGS[name].with_(name=name + "_w32", batch=3, window=32, ragged=True, steps=67)
    run(cfg, "sketch", flush=flush)


def test_delta_rule_w32_full_batch():
    """The same at the full batch of 256 (aligned), on sampled tiles."""
    from tests.gpu_parity import sample_tiles
    for name in ("gdn_b256", "kda_b256"):
        cfg = CONFIGS[name].with_(name=name + "_w32_full", window=32, steps=70)
        run(cfg, "sketch", tiles=sample_tiles(cfg, 4, 4, seed=cfg.seed), numpy_all=False)


# ---------------------------- the checker itself catches a one-tile mistake
def _planted(plant, **kw):
    cfg = CONFIGS["m2_b320"].with_(name="m2_planted", batch=4, steps=16, **kw)
    return run(cfg, "sketch", plant=plant, log=False)


def test_checker_catches_one_tile_mistakes():
    """A mistake planted on the CPU in the oracle's expected values of one
    tile of 512 (5% in one output vector, 5% in one sketch, 6e-5 in one
    state) stays under the pooled gate but fails the per-tile gate; without
    it the same run passes."""
    base = _planted({})
    assert base.tile_o < 0.01 and base.tile_S < 1e-5 and base.tile_U < 0.01
    with pytest.raises(AssertionError, match="per-tile rel-L2\\(o\\)"):
        _planted({"o": (3, 77, 0.05)})
    with pytest.raises(AssertionError, match="per-tile U"):
        _planted({"U": (0, 300, 0.05)})
    with pytest.raises(AssertionError, match="per-tile S"):
        _planted({"S": (0, 5, 6e-5)})


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
