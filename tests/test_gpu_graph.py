"""The benchmark times decode steps captured in a HIP graph (needs a GPU).
A captured sequence of reads and flushes, replayed, must give bit-identical
outputs, states, sketches, maps, state copies, rings, counts and error word
to the same calls made eagerly, on every replay, with the program's own
eager work (restoring the buffers) between the replays.  The flush is the
due-flag flush, the flush of listed sequences with each step's due
sequences (device lists made before the capture), or the flush over the
device-side due list (SKSSM_FLUSH_DUE_SCAN, whose list and count live in
the workspace), or, under an aligned phase, the closing flush
(SKSSM_FLUSH_CLOSE) in place of the closing step's read; the eager listed,
scanned and closing runs are also checked against the eager due-flag run
(the closing run leaves the last ring slot unwritten, so its rings are not
compared with the due-flag run's)."""
import pytest

from synth import CONFIGS

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module", autouse=True)
def _lib():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from ssm_decode_amd import abi
    abi.load()


def _buffers(lay):
    names = ("S", "U", "Cstate", "Scopy", "ring_k", "ring_v", "ring_gate", "ring_beta", "count", "err")
    return {n: getattr(lay, n) for n in names if getattr(lay, n) is not None}


CASES = [
    ("tiny_m2", {}, "fixed", "serial", "due"),
    ("m2_b320", dict(batch=3, ragged=True, dense_heads=(5, 70)), "fixed", "serial", "due"),
    ("gdn_b256", dict(batch=3, ragged=True), "fixed", "serial", "due"),
    ("gdn_b256", dict(batch=2, ragged=True, dense_heads=(1,)), "fixed", "wy", "due"),
    ("kda_b256", dict(batch=2, ragged=True), "state", "serial", "due"),
    ("m2_b320", dict(batch=5, ragged=True), "fixed", "serial", "list"),
    ("kda_b256", dict(batch=3, ragged=True), "state", "serial", "list"),
    ("m2_b320", dict(batch=5, ragged=True), "fixed", "serial", "scan"),
    ("gdn_b256", dict(batch=3, ragged=True, dense_heads=(1,)), "fixed", "serial", "scan"),
    # aligned, 64 sequences due at once: more than the scan flush's grid
    # covers one workgroup each, so its workgroups take several tiles
    ("tiny_m2", dict(batch=64), "fixed", "serial", "scan"),
    # aligned phases, the closing step as one closing flush
    ("m2_b320", dict(batch=3, dense_heads=(5, 70)), "fixed", "serial", "close"),
    ("gdn_b256", dict(batch=2), "fixed", "serial", "close"),
    ("kda_b256", dict(batch=2, dense_heads=(1,)), "state", "serial", "close"),
]


@pytest.mark.parametrize("name,over,coef,pullback,flush", CASES)
def test_graph_replay_matches_eager(name, over, coef, pullback, flush):
    import synth
    from ssm_decode_amd import abi, feed
    cfg = CONFIGS[name].with_(name=name + "_graph", **over)
    print(f"\n[graph] {cfg.name} B={cfg.batch} W={cfg.window} {coef} {pullback} {flush}", flush=True)
    li = synth.make_layer_inputs(cfg)
    lay = feed.make_layer(cfg, li, coef=coef, pullback=pullback)
    feed.fill_state(lay, cfg)
    assert feed.prime(lay, li) == 0
    K = 2 * cfg.window + 3
    steps = [lay.new_step() for _ in range(K)]
    for t, st in enumerate(steps):
        feed.fill_step(st, cfg, t)
    torch.cuda.synchronize()
    start = {n: b.clone() for n, b in _buffers(lay).items()}

    def restore():
        for n, b in _buffers(lay).items():
            b.copy_(start[n])
        for st in steps:
            st.o.zero_()

    # the sequences whose window closes at step t, from the initial fills
    import numpy as np
    c0 = np.asarray(li.count0)
    lists = [torch.from_numpy(np.nonzero((c0[:, 0] + t + 1) % cfg.window == 0)[0].astype(np.int32)).cuda()
             for t in range(K)]

    def run(stream, mode=flush):
        for t, st in enumerate(steps):
            if mode == "close" and (c0[0, 0] + t + 1) % cfg.window == 0:
                assert lay.flush(st, abi.SKSSM_FLUSH_CLOSE, stream=stream) == 0
                continue
            assert lay.read(st, stream=stream) == 0
            if mode == "list":
                assert lay.flush_seqs(st, lists[t], stream=stream) == 0
            elif mode == "scan":
                assert lay.flush(st, abi.SKSSM_FLUSH_DUE_SCAN, stream=stream) == 0
            else:
                assert lay.flush(st, abi.SKSSM_FLUSH_DUE, stream=stream) == 0

    run(None)                                  # eager
    torch.cuda.synchronize()
    eager_o = [st.o.clone() for st in steps]
    eager_b = {n: b.clone() for n, b in _buffers(lay).items()}
    if flush in ("list", "scan", "close"):     # the same results as the due-flag flush
        assert (c0 == c0[:, :1]).all()
        if flush == "close":
            assert (c0 == c0[0, 0]).all()
        restore()
        run(None, "due")
        torch.cuda.synchronize()
        for t, st in enumerate(steps):
            assert torch.equal(st.o, eager_o[t]), ("due vs " + flush, t)
        for n, b in _buffers(lay).items():
            if flush == "close" and n.startswith("ring_"):
                continue
            assert torch.equal(b, eager_b[n]), ("due vs " + flush, n)

    restore()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        run(torch.cuda.current_stream().cuda_stream)
    for rep in range(3):
        restore()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for t, st in enumerate(steps):
            assert torch.equal(st.o, eager_o[t]), (rep, "o", t)
        for n, b in _buffers(lay).items():
            assert torch.equal(b, eager_b[n]), (rep, n)
