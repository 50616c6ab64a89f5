"""Dense-fallback heads (rank 0) on the GPU against the oracle (needs a GPU).
Such a head's flush writes a copy of its state in the sketch dtype and its
non-flush reads take S^T q~ from that copy.  Outputs, states, sketches of
the sketched heads and the state copies of the dense heads are compared at
the usual tolerances, in layers that mix both kinds."""
import pytest

from synth import CONFIGS, LayerConfig

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_decode_amd import abi
    abi.load()


def run(cfg, **kw):
    from tests.gpu_parity import run_parity
    print(f"\n[dense fallback] {cfg.name} B={cfg.batch} H={cfg.heads} dense={cfg.dense_heads} "
          f"W={cfg.window} ragged={cfg.ragged}", flush=True)
    return run_parity(cfg, "sketch", **kw)


def _tiny(family, seed, **kw):
    base = dict(name=f"tiny_dense_{family}", family=family, batch=3, heads=4, qk_groups=4, dk=16,
                dv=32, window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=20,
                ragged=True, seed=seed, dense_heads=(1,))
    base.update(kw)
    return LayerConfig(**base)


@pytest.mark.parametrize("family,seed", [("mamba2", 51), ("gdn", 52), ("kda", 53)])
def test_tiny(family, seed):
    run(_tiny(family, seed))


@pytest.mark.parametrize("family,seed", [("mamba2", 54), ("gdn", 55), ("kda", 56)])
def test_tiny_every_head_dense(family, seed):
    """No sketched head at all (R = 0): the sketch, basis and map buffers are
    empty and every read comes from the state copies."""
    run(_tiny(family, seed, dense_heads=(0, 1, 2, 3), name=f"tiny_all_dense_{family}"))


@pytest.mark.parametrize("name,dense", [("m2_b320", (0, 17, 63, 127)), ("gdn_b256", (0, 5)),
                                        ("kda_b256", (31,))])
def test_small_batch_ragged(name, dense):
    run(CONFIGS[name].with_(name=name + "_dense", batch=3, ragged=True, steps=36, dense_heads=dense))


@pytest.mark.parametrize("family", ["mamba2", "gdn"])
def test_head_64x64(family):
    base = CONFIGS["m2_b320" if family == "mamba2" else "gdn_b256"]
    run(base.with_(name=f"{family}_64x64_dense", dk=64, dv=64, batch=2, steps=20, ragged=True,
                   dense_heads=(1, 2)))


@pytest.mark.parametrize("name,dense", [("m2_b320", (0, 17, 63, 127)), ("gdn_b256", (0, 5)),
                                        ("kda_b256", (31,))])
def test_window_32(name, dense):
    """A 32-slot ring: the dense reads take up to 31 buffered entries."""
    run(CONFIGS[name].with_(name=name + "_dense_w32", batch=3, ragged=True, window=32, steps=69,
                            dense_heads=dense))


def test_m2_head_128x128():
    run(CONFIGS["m2_b320"].with_(name="m2_128x128_dense", dk=128, dv=128, batch=2, steps=36, ragged=True,
                                 dense_heads=(3, 64)))


def test_state_map():
    run(CONFIGS["kda_b256"].with_(name="kda_dense_map", batch=2, ragged=True, steps=24,
                                  dense_heads=(3, 4)), coef="state")


def test_full_batch_sampled():
    """m2_b320 at full batch in the benchmark's launch configuration with
    four dense heads, the oracle following sampled tiles (dense ones
    included)."""
    import numpy as np
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS["m2_b320"].with_(name="m2_b320_dense", dense_heads=(0, 17, 63, 127))
    tiles = sample_tiles(cfg, 3, 3, seed=cfg.seed)
    extra = np.array([(b, h) for b in (0, cfg.batch - 1) for h in (17, 63)], dtype=np.int64)
    tiles = np.unique(np.concatenate([tiles, extra]), axis=0)
    run(cfg, steps=2 * cfg.window + 6, tiles=tiles, numpy_all=False)
