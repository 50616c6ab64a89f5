"""Edge cases of the HIP path, through the C ABI, against the oracle (needs a
GPU): a window of one step, the remaining head shape, fp32 activations at
real head shapes, a flush of every tile in the middle of a window, and the
device error word for a skipped flush, for a closing flush off phase and for
heads of one Mamba-2 group that disagree on the ring fill (forced from the
host; the kernels' own checks turn them into error bits and leave the tiles
untouched)."""
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


def _tiny(family, seed, **kw):
    base = dict(name=f"tiny_{family}", family=family, batch=2, heads=4, qk_groups=4, dk=16, dv=32,
                window=4, mean_rank=4, fixed_rank=4, act="f32", sketch="f32", steps=32,
                ragged=False, seed=seed)
    base.update(kw)
    return LayerConfig(**base)


def run(cfg, method, **kw):
    from tests.gpu_parity import run_parity
    print(f"\n[edge] {cfg.name} {method} B={cfg.batch} H={cfg.heads} dk={cfg.dk} dv={cfg.dv} "
          f"W={cfg.window} act={cfg.act} ragged={cfg.ragged}", flush=True)
    return run_parity(cfg, method, **kw)


@pytest.mark.parametrize("family,seed", [("mamba2", 21), ("gdn", 22), ("kda", 23)])
def test_window_one(family, seed):
    """W = 1: every read only appends and every step flushes, so each output
    is the exact read of the updated state (the oracle pins this to the
    standard recurrence)."""
    run(_tiny(family, seed, name=f"w1_{family}", window=1, steps=10), "sketch")


@pytest.mark.parametrize("family,seed", [("mamba2", 24), ("gdn", 25), ("kda", 26)])
def test_head_shape_64x64(family, seed):
    if family == "mamba2":
        cfg = CONFIGS["m2_b320"].with_(heads=16, qk_groups=2)
    else:
        cfg = CONFIGS[f"{family}_b256"].with_(heads=4, qk_groups=4)
    cfg = cfg.with_(name=f"{family}_64x64", dk=64, dv=64, batch=3, ragged=True, steps=36, seed=seed)
    run(cfg, "sketch")


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256"])
def test_fp32_activations_real_heads(name):
    cfg = CONFIGS[name].with_(name=name + "_f32", act="f32", sketch="f32", batch=2, ragged=True,
                              steps=24)
    run(cfg, "sketch")


@pytest.mark.parametrize("family,seed", [("mamba2", 27), ("gdn", 28), ("kda", 29)])
def test_flush_all_mid_window(family, seed):
    """FLUSH_ALL applies whatever each tile has buffered (fewer than W
    entries), writes S and U and resets the counts, like the oracle's flush
    of every tile."""
    import synth
    import oracle
    from ssm_decode_amd import abi, feed
    from tests.gpu_parity import rel_l2, all_tiles
    cfg = _tiny(family, seed, name=f"flushall_{family}", window=8, batch=3, ragged=True)
    li = synth.make_layer_inputs(cfg)
    tiles = all_tiles(cfg)
    lay = feed.make_layer(cfg, li)
    feed.fill_state(lay, cfg, numpy_all=True)
    assert feed.prime(lay, li) == 0
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets, li.Pt,
                             li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups)
    assert orc.flush(None, all_tiles=True)[0] == 0
    orc.count[:] = li.count0[tiles[:, 0], tiles[:, 1]]
    step = lay.new_step()
    for t in range(5):
        feed.fill_step(step, cfg, t, numpy_all=True)
        si = synth.make_step_inputs(cfg, t)
        assert lay.read(step) == 0 and lay.flush(step, abi.SKSSM_FLUSH_DUE) == 0
        o = np.zeros((len(tiles), cfg.dv))
        assert orc.read(si, o=o)[0] == 0
        if (orc.count == cfg.window).any():
            assert orc.flush(si, o=o)[0] == 0
    assert (orc.count > 0).any() and (orc.count < cfg.window).all()
    assert lay.flush(None, abi.SKSSM_FLUSH_ALL) == 0
    assert orc.flush(None, all_tiles=True)[0] == 0
    torch.cuda.synchronize()
    assert (lay.count.cpu().numpy() == 0).all()
    S_gpu = lay.S.cpu().numpy().reshape(-1, cfg.dk, cfg.dv).astype(np.float64)
    assert rel_l2(S_gpu, orc.S) <= 1e-5
    U_gpu = lay.U.float().cpu().numpy().astype(np.float64)
    Ug = [U_gpu[b, li.offsets[h]:li.offsets[h] + li.ranks[h]] for b, h in tiles]
    Uo = [orc.U[i, :li.ranks[h]] for i, (b, h) in enumerate(tiles)]
    assert rel_l2(np.concatenate(Ug), np.concatenate(Uo)) <= 1e-5
    assert lay.error_word() == 0


def _primed(family, seed, **kw):
    import synth
    from ssm_decode_amd import feed
    cfg = _tiny(family, seed, **kw)
    li = synth.make_layer_inputs(cfg)
    lay = feed.make_layer(cfg, li)
    feed.fill_state(lay, cfg, numpy_all=True)
    assert feed.prime(lay, li) == 0
    step = lay.new_step()
    feed.fill_step(step, cfg, 0, numpy_all=True)
    torch.cuda.synchronize()
    return cfg, lay, step


@pytest.mark.parametrize("family,seed", [("mamba2", 30), ("gdn", 31), ("kda", 32)])
def test_full_ring_read_sets_error(family, seed):
    """A tile whose ring already holds W entries missed its flush: the read
    reports SKSSM_ERRBIT_COUNT and leaves that tile's count and output alone;
    the other sequences advance."""
    from ssm_decode_amd import abi
    cfg, lay, step = _primed(family, seed, name=f"full_{family}")
    W = cfg.window
    lay.count[0, :] = W                      # sequence 0: every head full
    step.o.fill_(7.0)
    torch.cuda.synchronize()
    assert lay.read(step) == 0
    torch.cuda.synchronize()
    assert lay.error_word() & abi.SKSSM_ERRBIT_COUNT
    cnt = lay.count.cpu().numpy()
    assert (cnt[0] == W).all() and (cnt[1] == 1).all()
    assert (step.o[0].float().cpu().numpy() == 7.0).all()
    assert not (step.o[1].float().cpu().numpy() == 7.0).all()


@pytest.mark.parametrize("family,seed", [("mamba2", 40), ("gdn", 41), ("kda", 42)])
def test_closing_flush_off_phase_sets_error(family, seed):
    """SKSSM_FLUSH_CLOSE where a tile's ring does not hold W - 1 entries (the
    caller's phase was not aligned): that sequence reports
    SKSSM_ERRBIT_COUNT and keeps its state, count and output; the sequence
    at W - 1 closes its window (count 0)."""
    from ssm_decode_amd import abi, feed
    cfg, lay, step = _primed(family, seed, name=f"close_{family}")
    W = cfg.window
    lay.count.zero_()
    for t in range(W - 1):                  # W - 1 buffered entries in every ring
        feed.fill_step(step, cfg, t, numpy_all=True)
        assert lay.read(step) == 0
    feed.fill_step(step, cfg, W - 1, numpy_all=True)
    lay.count[1, :] = W - 2                 # sequence 1 off phase
    S_before = lay.S[1].clone()
    step.o.fill_(7.0)
    torch.cuda.synchronize()
    assert lay.error_word() == 0
    assert lay.flush(step, abi.SKSSM_FLUSH_CLOSE) == 0
    torch.cuda.synchronize()
    assert lay.error_word() & abi.SKSSM_ERRBIT_COUNT
    cnt = lay.count.cpu().numpy()
    assert (cnt[0] == 0).all() and (cnt[1] == W - 2).all()
    assert torch.equal(lay.S[1], S_before)
    assert (step.o[1].float().cpu().numpy() == 7.0).all()
    assert not (step.o[0].float().cpu().numpy() == 7.0).all()


@pytest.mark.parametrize("family,seed", [("mamba2", 33), ("gdn", 34), ("kda", 35)])
def test_overfull_ring_flush_sets_error(family, seed):
    from ssm_decode_amd import abi
    cfg, lay, step = _primed(family, seed, name=f"over_{family}")
    lay.count[1, 2] = cfg.window + 1
    S_before = lay.S[1, 2].clone()
    torch.cuda.synchronize()
    assert lay.flush(None, abi.SKSSM_FLUSH_ALL) == 0
    torch.cuda.synchronize()
    assert lay.error_word() & abi.SKSSM_ERRBIT_COUNT
    assert int(lay.count[1, 2]) == cfg.window + 1
    assert torch.equal(lay.S[1, 2], S_before)
    assert (lay.count[0].cpu().numpy() == 0).all()


def test_group_count_mismatch_sets_error():
    """Mamba-2 heads of one B/C group share their keys, so they must agree
    on the ring fill: a disagreeing head is reported (SKSSM_ERRBIT_GROUP) and
    nothing of that group is written."""
    from ssm_decode_amd import abi
    cfg, lay, step = _primed("mamba2", 36, name="grp_m2", heads=4, qk_groups=2, fixed_rank=4)
    lay.count[0, 1] = 1                      # heads 0 and 1 form group 0
    step.o.fill_(3.0)
    torch.cuda.synchronize()
    assert lay.read(step) == 0
    torch.cuda.synchronize()
    assert lay.error_word() & abi.SKSSM_ERRBIT_GROUP
    cnt = lay.count.cpu().numpy()
    assert cnt[0, 0] == 0 and cnt[0, 1] == 1           # group 0 of sequence 0 untouched
    assert (cnt[0, 2:] == 1).all() and (cnt[1] == 1).all()
    assert (step.o[0, :2].float().cpu().numpy() == 3.0).all()


@pytest.mark.parametrize("family,power,seed", [("gdn", 160, 37), ("kda", 60, 38), ("kda", 4, 39)])
def test_small_gates(family, power, seed):
    """Gates raised to a power (the same values on both sides): with tiny
    gates the product of a window's gates underflows on some tiles, which
    then take the serial form of the flush; the others the chunked form.
    Outputs and states against the oracle over three windows."""
    import dataclasses
    import synth
    import oracle
    from ssm_decode_amd import abi, feed
    from ssm_decode_amd.feed import to_device
    from tests.gpu_parity import rel_l2, all_tiles
    cfg = _tiny(family, seed, name=f"gates_{family}_{power}", window=8, batch=3, heads=4,
                qk_groups=4)
    li = synth.make_layer_inputs(cfg)
    tiles = all_tiles(cfg)
    lay = feed.make_layer(cfg, li)
    feed.fill_state(lay, cfg, numpy_all=True)
    assert feed.prime(lay, li) == 0
    S0 = synth.initial_state(cfg).reshape(-1, cfg.dk, cfg.dv)
    orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets, li.Pt,
                             li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups)
    assert orc.flush(None, all_tiles=True)[0] == 0
    step = lay.new_step()
    worst_o = worst_s = 0.0
    for t in range(3 * cfg.window):
        si = synth.make_step_inputs(cfg, t)
        si = dataclasses.replace(si, gate=synth.round_f32(si.gate ** power))
        feed.fill_step(step, cfg, t, numpy_all=True)
        step.gate.copy_(to_device(si.gate, "f32", step.gate.device))
        assert lay.read(step) == 0 and lay.flush(step, abi.SKSSM_FLUSH_DUE) == 0
        o = np.zeros((len(tiles), cfg.dv))
        assert orc.read(si, o=o)[0] == 0
        due = orc.count == cfg.window
        if due.any():
            assert orc.flush(si, o=o)[0] == 0
        torch.cuda.synchronize()
        e = rel_l2(step.o.cpu().numpy().reshape(-1, cfg.dv), o)
        worst_o = max(worst_o, e)
        assert e <= 1e-5, (t, e)
        if due.any():
            S_gpu = lay.S.cpu().numpy().reshape(-1, cfg.dk, cfg.dv).astype(np.float64)
            es = rel_l2(S_gpu, orc.S)
            worst_s = max(worst_s, es)
            assert es <= 1e-5, (t, es)
    assert lay.error_word() == 0
    print(f"  gates^{power}: max rel-L2 o={worst_o:.2e} S={worst_s:.2e}")


@pytest.mark.parametrize("name", ["m2_b320", "gdn_b256"])
def test_graph_replays_match_eager(name):
    """The benchmark times its steps as a captured HIP graph.  A layer that
    runs whole windows as graph replays (eager work and synchronisations in
    between) stays bit-identical to a twin layer run eagerly with the same
    inputs: outputs, states, sketches and counts after every replay."""
    import synth
    from ssm_decode_amd import abi, feed
    cfg = CONFIGS[name].with_(name=name + "_graph", batch=4, ragged=True)
    W = cfg.window
    li = synth.make_layer_inputs(cfg)
    layers = []
    for _ in range(2):
        lay = feed.make_layer(cfg, li)
        feed.fill_state(lay, cfg, numpy_all=True)
        assert feed.prime(lay, li) == 0
        layers.append(lay)
    ge, eg = layers
    steps = [ge.new_step() for _ in range(W)]
    for t, st in enumerate(steps):
        feed.fill_step(st, cfg, t, numpy_all=True)
    outs_g = [ge.new_step().o for _ in range(W)]
    outs_e = [eg.new_step().o for _ in range(W)]
    from ssm_decode_amd.layer import DeviceStep

    def run(lay, outs, handle):
        for t, st in enumerate(steps):
            ds = DeviceStep(st.q, st.k, st.v, st.gate, st.beta, outs[t]).struct()
            assert abi.sketchssm_read(lay.layer_struct, lay.buffers_struct, ds, handle) == 0
            assert abi.sketchssm_flush(lay.layer_struct, lay.buffers_struct, ds, abi.SKSSM_FLUSH_DUE,
                                       handle) == 0

    import ctypes
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(ge, outs_g, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    torch.cuda.synchronize()
    # capture does not execute: both layers are still at the primed state
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        run(eg, outs_e, ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
        torch.cuda.synchronize()
        _ = (ge.S.sum() + eg.S.sum()).item()          # eager work between replays
        for t in range(W):
            assert torch.equal(outs_g[t], outs_e[t]), (rep, t)
        assert torch.equal(ge.S, eg.S), rep
        assert torch.equal(ge.U, eg.U), rep
        assert torch.equal(ge.count, eg.count), rep
        assert torch.equal(ge.ring_v, eg.ring_v), rep
    assert ge.error_word() == 0 and eg.error_word() == 0
