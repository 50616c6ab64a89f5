"""sketchssm_read_noalloc (the read whose workspace is the library's own
device array) against sketchssm_read with a caller workspace: twin layers
with identical buffers take the same calls, one through each entry point,
and every output and buffer must stay bit-identical.  Two runs in a row
share the library's array, the second on a smaller layer, so the second
reads an array that still holds the first run's values."""
import numpy as np
import pytest

from synth import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


def _twins(cfg):
    import synth
    from ssm_decode_amd import feed
    li = synth.make_layer_inputs(cfg)
    a = feed.make_layer(cfg, li)
    feed.fill_state(a, cfg, numpy_all=True)
    assert feed.prime(a, li) == 0
    b = feed.make_layer(cfg, li)
    for name in ("S", "U", "ring_k", "ring_v", "ring_gate", "ring_beta", "count", "Scopy"):
        src, dst = getattr(a, name), getattr(b, name)
        if src is not None:
            dst.copy_(src)
    torch.cuda.synchronize()
    return a, b


def _same(a, b, what):
    for name in ("S", "U", "ring_k", "ring_v", "ring_gate", "ring_beta", "count", "Scopy", "err"):
        x, y = getattr(a, name), getattr(b, name)
        if x is not None:
            assert torch.equal(x, y), f"{what}: {name} differs"


def _run(cfg, steps):
    from ssm_decode_amd import abi, feed
    print(f"\n[no-alloc] {cfg.name} B={cfg.batch} W={cfg.window} steps={steps}", flush=True)
    a, b = _twins(cfg)
    sa, sb = a.new_step(), b.new_step()
    for t in range(steps):
        feed.fill_step(sa, cfg, t, numpy_all=True)
        for f in ("q", "k", "v", "gate", "beta"):
            x = getattr(sa, f)
            if x is not None:
                getattr(sb, f).copy_(x)
        assert a.read(sa) == 0
        assert b.read_noalloc(sb) == 0
        torch.cuda.synchronize()
        assert torch.equal(sa.o, sb.o), f"{cfg.name} step {t}: o differs"
        assert a.flush(sa, abi.SKSSM_FLUSH_DUE) == 0
        assert b.flush(sb, abi.SKSSM_FLUSH_DUE) == 0
        torch.cuda.synchronize()
        assert torch.equal(sa.o, sb.o), f"{cfg.name} step {t}: flush-step o differs"
    _same(a, b, cfg.name)
    assert a.error_word() == 0 and b.error_word() == 0


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_decode_amd import abi
    abi.load()


def test_noalloc_read_matches_read_two_calls_shrinking():
    """Mamba-2 at the real head shape (128 x 64, 128 heads, 8 groups):
    first batch 12, then batch 3 (ragged phases, two windows and more)."""
    base = CONFIGS["m2_b320"]
    _run(base.with_(name="m2_noalloc_b12", batch=12, ragged=True), 2 * base.window + 3)
    _run(base.with_(name="m2_noalloc_b3", batch=3, ragged=True, seed=base.seed + 7), base.window + 5)


def test_noalloc_read_delta_rule_dense_heads():
    """GDN with one dense-fallback head uses the workspace too (the pulled-
    back query and buffered term of the dense tiles): batch 4, then 2."""
    base = CONFIGS["gdn_b256"]
    _run(base.with_(name="gdn_noalloc_b4", batch=4, ragged=True, dense_heads=(5,)), 2 * base.window + 1)
    _run(base.with_(name="gdn_noalloc_b2", batch=2, ragged=True, dense_heads=(0,), seed=base.seed + 3),
         base.window + 2)
