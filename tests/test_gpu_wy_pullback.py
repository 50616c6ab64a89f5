"""The parallel (triangular-system) pull-back of the GDN/KDA read on the GPU,
and the same with projected per-slot factors (paper App. C.2), against the
oracle's own forms (needs a GPU).  Outputs, states and
sketches at the usual tolerances, over several windows, in the layouts the
serial form is tested in: small ragged layers, both window capacities,
64x64 heads, tiny gates, the state-dependent map, dense-fallback heads and
the full batch in the benchmark's launch configuration (sampled tiles)."""
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


PB = pytest.mark.parametrize("pb", ["wy", "proj"])


def run(cfg, pb, **kw):
    from tests.gpu_parity import run_parity
    print(f"\n[{pb} pull-back] {cfg.name} B={cfg.batch} H={cfg.heads} W={cfg.window} "
          f"ragged={cfg.ragged} {kw.get('coef', 'fixed')}", flush=True)
    return run_parity(cfg, "sketch", pullback=pb, **kw)


def _tiny(family, seed, **kw):
    base = dict(name=f"tiny_wy_{family}", family=family, batch=3, heads=4, qk_groups=4, dk=16,
                dv=32, window=6, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=26,
                ragged=True, seed=seed)
    base.update(kw)
    return LayerConfig(**base)


@pytest.mark.parametrize("family,seed", [("gdn", 61), ("kda", 62)])
@PB
def test_tiny(family, seed, pb):
    run(_tiny(family, seed), pb)


@pytest.mark.parametrize("family,W", [("gdn", 1), ("kda", 2), ("gdn", 16), ("kda", 32)])
@PB
def test_window_sizes(family, W, pb):
    run(_tiny(family, 63 + W, window=W, steps=2 * W + 5, name=f"tiny_wy_{family}_W{W}"), pb)


@pytest.mark.parametrize("name", ["gdn_b256", "kda_b256"])
@PB
def test_small_batch_ragged(name, pb):
    run(CONFIGS[name].with_(name=name + "_wy", batch=3, ragged=True, steps=36), pb)


@pytest.mark.parametrize("family", ["gdn", "kda"])
@PB
def test_head_64x64(family, pb):
    run(CONFIGS[family + "_b256"].with_(name=f"{family}_64x64_wy", dk=64, dv=64, batch=2, steps=20,
                                         ragged=True), pb)


@PB
def test_state_map_and_dense_heads(pb):
    run(CONFIGS["kda_b256"].with_(name="kda_wy_map_dense", batch=2, ragged=True, steps=24,
                                  dense_heads=(3,)), pb, coef="state")
    run(CONFIGS["gdn_b256"].with_(name="gdn_wy_dense", batch=2, ragged=True, steps=24,
                                  dense_heads=(0, 7)), pb)


@pytest.mark.parametrize("name", ["gdn_b256", "kda_b256"])
@PB
def test_full_batch_sampled(name, pb):
    """Full batch in the benchmark's launch configuration, the oracle
    following sampled tiles."""
    from tests.gpu_parity import sample_tiles
    cfg = CONFIGS[name]
    run(cfg, pb, steps=2 * cfg.window + 6, tiles=sample_tiles(cfg, 3, 3, seed=cfg.seed), numpy_all=False)
