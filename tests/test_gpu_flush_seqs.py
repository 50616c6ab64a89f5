"""The flush of listed sequences (sketchssm_flush_seqs) on the GPU (needs a
GPU).  Under a ragged window phase, the due-flag flush and the listed flush
(the sequences whose window filled at this step) run the same per-tile
work, so their outputs, states, sketches and counts agree bit for bit; the
due-flag flush is itself checked against the oracle by the parity tests.
A listed index outside the batch sets its error bit and leaves every tile
alone; an empty list launches nothing."""
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


def _pair(cfg, coef="fixed"):
    import synth
    from ssm_decode_amd import feed
    li = synth.make_layer_inputs(cfg)
    lays = [feed.make_layer(cfg, li, coef=coef) for _ in range(2)]
    for lay in lays:
        feed.fill_state(lay, cfg)
        assert feed.prime(lay, li) == 0
    return lays


def _due(lay, W):
    return torch.nonzero((lay.count == W).any(dim=1)).flatten().to(torch.int32).contiguous()


def _run(cfg, steps, coef="fixed"):
    from ssm_decode_amd import abi, feed
    print(f"\n[flush_seqs] {cfg.name} B={cfg.batch} H={cfg.heads} W={cfg.window} coef={coef}", flush=True)
    la, lb = _pair(cfg, coef)
    sa, sb = la.new_step(), lb.new_step()
    listed = 0
    for t in range(steps):
        feed.fill_step(sa, cfg, t)
        feed.fill_step(sb, cfg, t)
        assert la.read(sa) == 0 and lb.read(sb) == 0
        assert la.flush(sa, abi.SKSSM_FLUSH_DUE) == 0
        due = _due(lb, cfg.window)
        listed += int(due.numel())
        assert lb.flush_seqs(sb, due) == 0
        torch.cuda.synchronize()
        assert torch.equal(sa.o, sb.o), t
    assert listed > 0
    for name in ("S", "U", "count", "ring_k", "ring_v", "ring_gate"):
        assert torch.equal(getattr(la, name), getattr(lb, name)), name
    if coef == "state":
        assert torch.equal(la.Cstate, lb.Cstate)
    assert la.error_word() == 0 and lb.error_word() == 0


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_listed_flush_equals_due_flush(name):
    cfg = CONFIGS[name].with_(name=name + "_ragged_list", batch=6, ragged=True)
    _run(cfg, 2 * cfg.window + 3)


def test_listed_flush_state_map():
    cfg = CONFIGS["gdn_b256"].with_(name="gdn_ragged_list_map", batch=4, ragged=True)
    _run(cfg, cfg.window + 5, coef="state")


def test_listed_flush_stress_batch():
    """Batch 1024, W = 32, ragged: the workload whose due-flag flush is set by
    its idle tiles."""
    import synth
    cfg = synth.get_config("m2_stress_b1024_w32_g8")
    _run(cfg, 6)


def test_bad_index_sets_error_bit_and_touches_nothing():
    from ssm_decode_amd import abi, feed
    cfg = LayerConfig(name="tiny_list", family="gdn", batch=3, heads=4, qk_groups=4, dk=16, dv=32,
                      window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=8,
                      ragged=False, seed=61)
    la, _ = _pair(cfg)
    st = la.new_step()
    for t in range(cfg.window):                    # every ring full: all tiles due
        feed.fill_step(st, cfg, t)
        assert la.read(st) == 0
    S0, U0, c0 = la.S.clone(), la.U.clone(), la.count.clone()
    bad = torch.tensor([cfg.batch, -1], dtype=torch.int32, device="cuda")
    assert la.flush_seqs(st, bad) == 0
    empty = torch.zeros((0,), dtype=torch.int32, device="cuda")
    assert la.flush_seqs(st, empty) == 0
    torch.cuda.synchronize()
    assert la.error_word() == abi.SKSSM_ERRBIT_SEQ
    assert torch.equal(la.S, S0) and torch.equal(la.U, U0) and torch.equal(la.count, c0)
    # a valid list then flushes exactly its sequences
    la.err.zero_()
    assert la.flush_seqs(st, torch.tensor([1], dtype=torch.int32, device="cuda")) == 0
    torch.cuda.synchronize()
    assert la.error_word() == 0
    assert (la.count[1] == 0).all() and (la.count[0] == cfg.window).all() and (la.count[2] == cfg.window).all()
    assert torch.equal(la.S[0], S0[0]) and not torch.equal(la.S[1], S0[1])


def test_duplicate_index_flushes_once():
    """A sequence listed twice is flushed once (each tile is claimed before
    its flush): the result equals the due-flag flush bit for bit, and the
    failed second claim, when it meets the first flush still running, is
    reported as SKSSM_ERRBIT_SEQ."""
    from ssm_decode_amd import abi, feed
    cfg = CONFIGS["m2_b320"].with_(name="m2_dup_list", batch=4, ragged=True)
    la, lb = _pair(cfg)
    sa, sb = la.new_step(), lb.new_step()
    flushed = 0
    for t in range(cfg.window + 2):
        feed.fill_step(sa, cfg, t)
        feed.fill_step(sb, cfg, t)
        assert la.read(sa) == 0 and lb.read(sb) == 0
        assert la.flush(sa, abi.SKSSM_FLUSH_DUE) == 0
        due = _due(lb, cfg.window)
        flushed += int(due.numel())
        dup = torch.cat([due, due])[:cfg.batch].contiguous()      # (a list holds at most batch entries)
        assert lb.flush_seqs(sb, dup) == 0
        torch.cuda.synchronize()
        assert torch.equal(sa.o, sb.o), t
    assert flushed > 0
    for name in ("S", "U", "count", "ring_k", "ring_v", "ring_gate"):
        assert torch.equal(getattr(la, name), getattr(lb, name)), name
    assert la.error_word() == 0 and lb.error_word() in (0, abi.SKSSM_ERRBIT_SEQ)


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256", "kda_b256"])
def test_scan_flush_equals_due_flush(name):
    """The flush over the device-side list (SKSSM_FLUSH_DUE_SCAN) runs the same
    per-tile work as the due-flag flush: bit-identical results."""
    from ssm_decode_amd import abi, feed
    cfg = CONFIGS[name].with_(name=name + "_scan_eq", batch=6, ragged=True)
    la, lb = _pair(cfg)
    sa, sb = la.new_step(), lb.new_step()
    for t in range(2 * cfg.window + 3):
        feed.fill_step(sa, cfg, t)
        feed.fill_step(sb, cfg, t)
        assert la.read(sa) == 0 and lb.read(sb) == 0
        assert la.flush(sa, abi.SKSSM_FLUSH_DUE) == 0
        assert lb.flush(sb, abi.SKSSM_FLUSH_DUE_SCAN) == 0
        torch.cuda.synchronize()
        assert torch.equal(sa.o, sb.o), t
    for nm in ("S", "U", "count", "ring_k", "ring_v", "ring_gate"):
        assert torch.equal(getattr(la, nm), getattr(lb, nm)), nm
    assert la.error_word() == 0 and lb.error_word() == 0


def test_scan_flush_reports_bad_counts():
    """A count outside [0, W] found by the scan sets SKSSM_ERRBIT_COUNT and
    leaves that tile alone; the due tiles are flushed."""
    from ssm_decode_amd import abi, feed
    cfg = LayerConfig(name="tiny_scan", family="kda", batch=3, heads=4, qk_groups=4, dk=16, dv=32,
                      window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=8,
                      ragged=False, seed=62)
    la, _ = _pair(cfg)
    st = la.new_step()
    for t in range(cfg.window):                    # every ring full: all tiles due
        feed.fill_step(st, cfg, t)
        assert la.read(st) == 0
    la.count[2, 1] = cfg.window + 3
    S21 = la.S[2, 1].clone()
    torch.cuda.synchronize()
    assert la.flush(st, abi.SKSSM_FLUSH_DUE_SCAN) == 0
    torch.cuda.synchronize()
    assert la.error_word() == abi.SKSSM_ERRBIT_COUNT
    cnt = la.count.cpu().numpy()
    assert cnt[2, 1] == cfg.window + 3 and torch.equal(la.S[2, 1], S21)
    assert (cnt[0] == 0).all() and (cnt[1] == 0).all() and cnt[2, 0] == 0
