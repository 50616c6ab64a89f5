"""The state-dependent coefficient map on the GPU against the oracle (needs a
GPU).  Every flush (and the prime) forms each tile's map from its new state
and stored sketch; the reads use it.  Outputs, states, sketches and the maps
of the flushed tiles are compared with the oracle's state-dependent path at
the usual tolerances (relative L2: 1e-5 fp32, 1e-2 where the activations and
the sketch are bf16); ring counts exactly.
"""
import numpy as np
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
    print(f"\n[state-map parity] {cfg.name} B={cfg.batch} H={cfg.heads} W={cfg.window} "
          f"dk={cfg.dk} dv={cfg.dv} ragged={cfg.ragged}", flush=True)
    return run_parity(cfg, "sketch", coef="state", **kw)


def _tiny(family, seed, **kw):
    base = dict(name=f"tiny_{family}", family=family, batch=2, heads=4, qk_groups=4, dk=16, dv=32,
                window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=32,
                ragged=False, seed=seed)
    base.update(kw)
    return LayerConfig(**base)


def test_tiny_m2():
    run(CONFIGS["tiny_m2"])


@pytest.mark.parametrize("family,seed", [("gdn", 11), ("kda", 12)])
def test_tiny_deltanet(family, seed):
    run(_tiny(family, seed))


@pytest.mark.parametrize("family,seed", [("mamba2", 1), ("gdn", 13), ("kda", 14)])
def test_tiny_ragged(family, seed):
    run(_tiny(family, seed, ragged=True, steps=19, batch=5))


@pytest.mark.parametrize("ridge", [1e-2, 1.0])
def test_tiny_ridge(ridge):
    run(CONFIGS["tiny_m2"].with_(name=f"tiny_m2_ridge{ridge:g}", steps=12), ridge=ridge)


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_small_batch_ragged(name):
    run(CONFIGS[name].with_(name=name + "_small", batch=3, ragged=True, steps=40))


@pytest.mark.parametrize("family", ["mamba2", "gdn"])
def test_head_64x64(family):
    base = CONFIGS["m2_b320" if family == "mamba2" else "gdn_b256"]
    run(base.with_(name=f"{family}_64x64", dk=64, dv=64, batch=3, steps=20, ragged=True))


def test_fp32_real_heads():
    run(CONFIGS["kda_b256"].with_(name="kda_f32", act="f32", sketch="f32", batch=2, heads=4,
                                  qk_groups=4, steps=20))


def test_window_one():
    run(CONFIGS["gdn_b256"].with_(name="gdn_w1", window=1, batch=2, steps=6))


def test_stress_point_w32_g16():
    run(CONFIGS["m2_stress_b1024"].with_(name="stress_w32_g16_small", batch=4, window=32,
                                          mean_rank=16, steps=40))


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_full_batch_sampled(name):
    """The full batch in the benchmark's launch configuration; the oracle
    follows sampled tiles for two windows and a half."""
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS[name]
    tiles = sample_tiles(cfg, 3, 3, seed=cfg.seed)
    run(cfg, steps=2 * cfg.window + 8, tiles=tiles, numpy_all=False)
