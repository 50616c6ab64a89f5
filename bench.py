"""Benchmark of the SketchSSM decode hot path on one MI355X.

One step = one decode step of one layer: the non-flush sketched read, plus
the flush on the step that closes a window.  The workload is the Mamba-2
layer at batch 320 (128 heads, dk 128, dv 64, 8 B/C groups, W = 16, mean
sketch rank 8, bf16 activations and sketch, fp32 state).  L independent
instances of the layer are rotated every step (as consecutive layers of a
model would be), so that the non-flush working set of one instance does not
stay in the 256 MiB last-level cache between its steps.

Printed: one JSON line with the per-layer step time (W-amortised, µs), the
achieved HBM bandwidth of the algorithmic bytes, the roofline of the
dominant kernel (the flush) timed with HIP events on its stream, GPU
baselines (standard full-state step, ReplaySSM step), and the CPU oracle
timed on a bounded sample as a reported baseline.
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=160,
                    help="timed decode steps per layer (rounded up to whole windows)")
    ap.add_argument("--reps", type=int, default=5,
                    help="timed replays of the captured steps (the median is reported)")
    ap.add_argument("--warmup", type=int, default=32)
    ap.add_argument("--workload", default="m2_b320")
    ap.add_argument("--layers", type=int, default=0, help="rotated layer instances (0: auto)")
    ap.add_argument("--pool", type=int, default=16, help="device-resident step inputs cycled")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--no-baselines", action="store_true", help="skip full/replay GPU baselines")
    ap.add_argument("--no-state-map", action="store_true",
                    help="skip the run with the state-dependent coefficient map")
    ap.add_argument("--no-dense", action="store_true",
                    help="skip the run with dense-fallback heads")
    ap.add_argument("--flush-list", action="store_true",
                    help="ragged phase: flush through sketchssm_flush_seqs with each step's due sequences")
    ap.add_argument("--flush-scan", action="store_true",
                    help="flush with SKSSM_FLUSH_DUE_SCAN (the due sequences listed on the device; "
                         "the default under a ragged phase)")
    ap.add_argument("--flush-due", action="store_true",
                    help="flush with SKSSM_FLUSH_DUE after every step's read (a workgroup per tile of "
                         "the batch); under an aligned phase the default is SKSSM_FLUSH_CLOSE at the "
                         "closing step, in place of its read")
    ap.add_argument("--no-wy", action="store_true",
                    help="skip the GDN/KDA run with the triangular-system pull-back")
    ap.add_argument("--cpu-seqs", type=int, default=320, help="sequences in the CPU sample")
    ap.add_argument("--cpu-windows", type=int, default=16, help="windows in the CPU sample")
    return ap.parse_args()


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py runs on one GPU only: this decode path has no multi-GPU mode "
              "(its (sequence, head) tiles are independent; sharding is by sequence or head).",
              file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    import synth
    from synth import torch_gen
    from ssm_decode_amd import abi, feed, traffic
    from ssm_decode_amd.layer import DeviceStep

    abi.load()
    dev = "cuda"
    cfg = synth.get_config(args.workload)
    li = synth.make_layer_inputs(cfg)
    W = cfg.window
    lb = traffic.config_bytes(cfg, int(li.offsets[-1]))

    # ---------------------------------------------------------- layers
    # enough instances that their sketches and rings together span at least
    # twice the 256 MiB last-level cache
    first = feed.make_layer(cfg, li, device=dev)
    nonflush = first.U.nbytes + first.ring_k.nbytes + first.ring_v.nbytes + first.ring_gate.nbytes
    L = args.layers or int(np.clip(np.ceil(2 * 256 * 2 ** 20 / nonflush), 2, 8))
    log(f"[bench] {cfg.name}: B={cfg.batch} H={cfg.heads} dk={cfg.dk} dv={cfg.dv} W={W} "
        f"R={int(li.offsets[-1])} layers={L} (sketch+ring {nonflush / 1e6:.0f} MB each)")
    feed.fill_state(first, cfg, numpy_all=False)
    S_init = first.S.clone()

    def make_layers(coef, cfg_=None, li_=None, pullback="serial"):
        cfg_, li_ = cfg_ or cfg, li_ or li
        out = []
        for _ in range(L):
            lay = feed.make_layer(cfg_, li_, device=dev, coef=coef, pullback=pullback)
            lay.S.copy_(S_init)
            assert feed.prime(lay, li_) == 0
            out.append(lay)
        torch.cuda.synchronize()
        return out

    # -------------------------------------------------- step input pool
    P = max(1, args.pool)
    pool = []
    for t in range(P):
        st = first.new_step()
        q, k, v, gate, beta = torch_gen.step_inputs(cfg, t, dev)
        st.q.copy_(q); st.k.copy_(k); st.v.copy_(v); st.gate.copy_(gate)
        if beta is not None:
            st.beta.copy_(beta)
        pool.append(st)
    # one output buffer per layer
    outs = [first.new_step().o for _ in range(L)]
    del first
    steps_structs = []
    for t in range(P):
        row = []
        for l in range(L):
            s = pool[(t + l) % P]
            row.append(DeviceStep(s.q, s.k, s.v, s.gate, s.beta, outs[l]).struct())
        steps_structs.append(row)
    torch.cuda.synchronize()

    stream = torch.cuda.current_stream()
    sh = ctypes.c_void_p(stream.cuda_stream)
    phase = int(li.phase[0])
    ragged = cfg.ragged
    # the timed steps are whole windows: every window of a layer is one flush
    # and W - 1 reads, so the per-step figure is W-amortised exactly
    K_req = args.steps
    K = timed_steps(K_req, W)
    REPS = max(5, args.reps)
    # listed flush: the sequences whose window closes at step t (t mod W),
    # from each sequence's initial ring fill; device-resident for the graph
    # the flush: the caller's list, the device-side due list or the due
    # flag; by default the due list under a ragged phase (the flush for a
    # caller that does not track phases) and the due flag under an aligned one
    use_scan = args.flush_scan or (ragged and not args.flush_due and not args.flush_list)
    # an aligned phase: the step that closes every window is one closing
    # flush (SKSSM_FLUSH_CLOSE), whose read would only append
    use_close = not ragged and not (args.flush_due or args.flush_list or args.flush_scan)
    reads_per_window = W - 1 if use_close else W
    flush_lists = None
    if args.flush_list and ragged:
        c0 = np.asarray(li.count0)
        assert (c0 == c0[:, :1]).all(), "one window phase per sequence"
        flush_lists = [torch.from_numpy(np.nonzero((c0[:, 0] + r + 1) % W == 0)[0].astype(np.int32)).to(dev)
                       for r in range(W)]

    def measure(layers):
        """Event-timed eager kernels over two windows, then K steps (whole
        windows) captured in one HIP graph, replayed REPS times back to back
        (each replay starts at a window boundary), HIP events around every
        replay; the median replay gives the step time."""

        def one_step(t, ev=None, stream_handle=None):
            sh_ = sh if stream_handle is None else stream_handle
            due = ragged or ((t - phase) % W == 0)
            for l, lay in enumerate(layers):
                st = steps_structs[t % P][l]
                if use_close and due:
                    if ev is not None:
                        ev["flush"].append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                        ev["flush"][-1][0].record(stream)
                    rc = abi.sketchssm_flush(lay.layer_struct, lay.buffers_struct, st, abi.SKSSM_FLUSH_CLOSE, sh_)
                    if ev is not None:
                        ev["flush"][-1][1].record(stream)
                    assert rc == 0
                    continue
                if ev is not None:
                    ev["read"].append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                    ev["read"][-1][0].record(stream)
                rc = abi.sketchssm_read(lay.layer_struct, lay.buffers_struct, st, sh_)
                if ev is not None:
                    ev["read"][-1][1].record(stream)
                assert rc == 0
                if due:
                    if ev is not None:
                        ev["flush"].append((torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)))
                        ev["flush"][-1][0].record(stream)
                    if flush_lists is not None:
                        dl = flush_lists[t % W]
                        rc = abi.sketchssm_flush_seqs(lay.layer_struct, lay.buffers_struct, st,
                                                      ctypes.c_void_p(dl.data_ptr()) if dl.numel() else None,
                                                      int(dl.numel()), sh_)
                    else:
                        rc = abi.sketchssm_flush(lay.layer_struct, lay.buffers_struct, st,
                                                 abi.SKSSM_FLUSH_DUE_SCAN if use_scan
                                                 else abi.SKSSM_FLUSH_DUE, sh_)
                    if ev is not None:
                        ev["flush"][-1][1].record(stream)
                    assert rc == 0

        def realign(t):
            while (t - phase - 1) % W != 0 and not ragged:
                one_step(t)
                t += 1
            return t

        # the timed region starts at a window boundary
        t = 0
        for _ in range(args.warmup):
            one_step(t)
            t += 1
        t = realign(t)
        torch.cuda.synchronize()

        # per-kernel durations: eager launches bracketed by HIP events on
        # the launch stream, over two windows
        ev = {"read": [], "flush": []}
        for i in range(2 * W):
            one_step(t + i, ev)
        torch.cuda.synchronize()
        t += 2 * W
        read_us = [a.elapsed_time(b) * 1000 for a, b in ev["read"]]
        flush_us = [a.elapsed_time(b) * 1000 for a, b in ev["flush"]]

        # the timed steps: K steps, whole windows (every layer's read, and its
        # flush when a window closes) captured in one HIP graph, so that host
        # launch overhead is not timed; the device ring counts advance exactly
        # as in eager execution, and since K is a multiple of W every replay
        # starts at the same window phase
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            capture_handle = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
            for i in range(K):
                one_step(t + i, stream_handle=capture_handle)
        torch.cuda.synchronize()
        graph.replay()                      # warm replay
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(REPS)]
        for a, b in evs:
            a.record(stream)
            graph.replay()
            b.record(stream)
        torch.cuda.synchronize()
        reps_ms = [a.elapsed_time(b) for a, b in evs]
        del graph
        err = max(lay.error_word() for lay in layers)
        assert err == 0, f"device error word {err}"
        med = float(np.median(reps_ms))
        return {"us_per_step": med * 1000.0 / (K * L),
                "reps_us_per_step": [round(x * 1000.0 / (K * L), 3) for x in reps_ms],
                "flush_avg": float(np.mean(flush_us)) if flush_us else float("nan"),
                "flush_n": len(flush_us), "read_avg": float(np.mean(read_us)), "read_n": len(read_us)}

    layers = make_layers("fixed")
    log(f"[bench] layers ready ({torch.cuda.memory_allocated() / 2 ** 30:.1f} GiB)")
    m = measure(layers)
    us_per_step, flush_avg, read_avg = m["us_per_step"], m["flush_avg"], m["read_avg"]
    flush_us, read_us = [0] * m["flush_n"], [0] * m["read_n"]
    log(f"[bench] sketch: {us_per_step:.2f} us/step/layer, median of {REPS} replays "
        f"{m['reps_us_per_step']} (graph of {K} steps = {K // W} windows x {L} layers); "
        f"flush avg {flush_avg:.1f} us ({len(flush_us)} launches); read avg {read_avg:.2f} us")

    achieved_gbs = lb.per_step / (us_per_step * 1e-6) / 1e9
    # a ragged phase flushes about B / W sequences per launch (shared basis once)
    flush_bytes = lb.flush_launch if not ragged else \
        (lb.flush_launch - lb.basis) / W + lb.basis
    flush_gbs = flush_bytes / (flush_avg * 1e-6) / 1e9
    # bytes of one read call: the window's bytes outside the flush over the
    # window's read calls (W - 1 with the closing flush, else W, the read at
    # the closing step appending only)
    read_bytes = lb.read_launch_avg * W / reads_per_window
    read_gbs = read_bytes / (read_avg * 1e-6) / 1e9
    windows_exact = K % W == 0

    # ------------------------------------------------ GPU baselines
    baselines = None
    if not args.no_baselines:
        lay = layers[0]

        def graph_us(call, n):
            """n steps of one call captured in a HIP graph (as the sketch path
            is timed), replayed REPS times; median µs per step."""
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                hc = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
                for i in range(n):
                    assert call(lay.layer_struct, lay.buffers_struct, steps_structs[i % P][0], hc) == 0
            torch.cuda.synchronize()
            g.replay()                          # warm replay
            torch.cuda.synchronize()
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(REPS)]
            for a, b in evs:
                a.record(stream)
                g.replay()
                b.record(stream)
            torch.cuda.synchronize()
            del g
            return float(np.median([a.elapsed_time(b) for a, b in evs])) * 1000 / n

        # standard full-state step
        full_us = graph_us(abi.sketchssm_full_step, W)
        # ReplaySSM over whole windows (its ring restarts from an empty window
        # and is empty again after every replay)
        lay.count.zero_()
        torch.cuda.synchronize()
        replay_us = graph_us(abi.sketchssm_replay_step, W)
        assert lay.error_word() == 0
        baselines = {
            "timing": f"{W} steps (one window) captured in a HIP graph, median of {REPS} replays",
            "full_step_us": round(full_us, 2),
            "full_step_gbs": round(lb.full_step / (full_us * 1e-6) / 1e9, 1),
            "replay_step_us": round(replay_us, 2),
            "replay_step_gbs": round(lb.replay_per_step / (replay_us * 1e-6) / 1e9, 1),
            "speedup_vs_full": round(full_us / us_per_step, 3),
            "speedup_vs_replay": round(replay_us / us_per_step, 3),
        }
        log(f"[bench] baselines: {baselines}")

    # ------------------------- sketch approximation error (information only)
    approx = None
    if not args.no_baselines:
        approx = sketch_error(cfg, li, layers[0], pool, steps=2 * W)
        log(f"[bench] sketched vs exact read: {approx}")

    # --------------- the state-dependent coefficient map (same workload)
    state_map = None
    if not args.no_state_map:
        sm = {}
        if not args.no_baselines:
            sm["sketch_error"] = sketch_error(cfg, li, layers[0], pool, steps=2 * W, coef="state")
            log(f"[bench] state-map sketched vs exact read: {sm['sketch_error']}")
        del layers
        torch.cuda.empty_cache()
        layers = make_layers("state")
        ms = measure(layers)
        lbs = traffic.config_bytes(cfg, int(li.offsets[-1]), "state")
        sflush = lbs.flush_launch if not ragged else (lbs.flush_launch - lbs.basis) / W + lbs.basis
        sgbs = sflush / (ms["flush_avg"] * 1e-6) / 1e9
        sm.update({
            "us_per_step": round(ms["us_per_step"], 3),
            "algorithmic_bytes_per_step": int(round(lbs.per_step)),
            "achieved_gbs": round(lbs.per_step / (ms["us_per_step"] * 1e-6) / 1e9, 1),
            "frac_of_hbm_peak": round(lbs.per_step / (ms["us_per_step"] * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
            "tokens_per_s_per_layer": round(cfg.batch / (ms["us_per_step"] * 1e-6), 1),
            "flush_us": round(ms["flush_avg"], 2), "flush_bytes": int(round(sflush)),
            "flush_gbs": round(sgbs, 1),
            "read_us": round(ms["read_avg"], 2),
            "read_bytes_avg": int(round(lbs.read_launch_avg * W / reads_per_window)),
            "read_gbs": round(lbs.read_launch_avg * W / reads_per_window / (ms["read_avg"] * 1e-6) / 1e9, 1),
        })
        if baselines:
            sm["speedup_vs_full"] = round(baselines["full_step_us"] / ms["us_per_step"], 3)
            sm["speedup_vs_replay"] = round(baselines["replay_step_us"] / ms["us_per_step"], 3)
        state_map = sm
        log(f"[bench] state-dependent map: {sm}")
    del layers

    # ------ dense-fallback heads: the same workload with 1 head in 32 dense
    # (the pages' allocation for one of their models keeps about 3% of the
    # heads dense)
    dense_block = None
    if not args.no_dense:
        torch.cuda.empty_cache()
        dh = tuple(range(0, cfg.heads, 32))
        cfg_d = cfg.with_(dense_heads=dh)
        li_d = synth.make_layer_inputs(cfg_d)
        layers = make_layers("fixed", cfg_d, li_d)
        md = measure(layers)
        lbd = traffic.config_bytes(cfg_d, int(li_d.offsets[-1]))
        dense_block = {
            "dense_heads": list(dh), "us_per_step": round(md["us_per_step"], 3),
            "algorithmic_bytes_per_step": int(round(lbd.per_step)),
            "achieved_gbs": round(lbd.per_step / (md["us_per_step"] * 1e-6) / 1e9, 1),
            "flush_us": round(md["flush_avg"], 2), "read_us": round(md["read_avg"], 2),
        }
        log(f"[bench] dense-fallback heads: {dense_block}")
        del layers

    # ------ GDN/KDA: the same workload with the read's effective query from
    # the triangular system over the buffered slots instead of the serial
    # pull-back (a Mamba-2 effective query is a decay only: no such run)
    wy_block = None
    if not args.no_wy and cfg.family != "mamba2":
        wy_block = {"us_per_step_serial": round(us_per_step, 3), "read_us_serial": round(read_avg, 2)}
        # the triangular-system pull-back, and the same with projected
        # per-slot factors (the algorithmic bytes are those of the serial
        # form; the factors add 64 B per buffered slot and tile)
        for pb in ("wy", "proj"):
            torch.cuda.empty_cache()
            layers = make_layers("fixed", pullback=pb)
            mw = measure(layers)
            wy_block[pb] = {
                "us_per_step": round(mw["us_per_step"], 3),
                "achieved_gbs": round(lb.per_step / (mw["us_per_step"] * 1e-6) / 1e9, 1),
                "flush_us": round(mw["flush_avg"], 2), "read_us": round(mw["read_avg"], 2),
            }
            del layers
        log(f"[bench] triangular-system pull-back (wy) and projected factors (proj): {wy_block}")

    # ------------------------------------------ copy-bandwidth reference
    nbytes = 2 * 2 ** 30
    src = torch.empty(nbytes // 4, dtype=torch.float32, device=dev).fill_(1.0)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(5):
        dst.copy_(src)
    b.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 2 * nbytes * 5 / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    log(f"[bench] copy bandwidth {copy_gbs:.0f} GB/s")

    # ------------------------------------------------ CPU oracle baseline
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(cfg, li, min(args.cpu_seqs, cfg.batch), args.cpu_windows)
        log(f"[bench] cpu oracle: {cpu}")

    result = {
        "metric": "per-layer decode step us (W-amortised) + achieved HBM GB/s vs peak, batch 320",
        "value": round(us_per_step, 3),
        "unit": "us/step",
        "n_gpus": 1,
        "steps": K,
        "steps_requested": K_req,
        "windows": K // W,
        "reps": REPS,
        "reps_us_per_step": m["reps_us_per_step"],
        "warmup": args.warmup,
        "ms_per_step": round(us_per_step / 1000.0, 6),
        "higher_is_better": False,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": cfg.name, "family": cfg.family, "batch": cfg.batch, "heads": cfg.heads,
            "qk_groups": cfg.qk_groups, "dk": cfg.dk, "dv": cfg.dv, "window": W,
            "mean_rank": cfg.mean_rank, "state": "f32", "act": cfg.act, "sketch": cfg.sketch,
            "layers_rotated": L, "windows_exact": windows_exact,
            "flush": ("listed sequences (sketchssm_flush_seqs)" if flush_lists is not None else
                      "due sequences listed on the device (SKSSM_FLUSH_DUE_SCAN)" if use_scan
                      else "closing flush in place of the closing step's read (SKSSM_FLUSH_CLOSE)"
                      if use_close else "due flag"),
        },
        "achieved_gbs": round(achieved_gbs, 1),
        "frac_of_hbm_peak": round(achieved_gbs / HBM_PEAK_GBS, 4),
        "frac_of_copy_bw": round(achieved_gbs / copy_gbs, 4),
        "copy_gbs": round(copy_gbs, 1),
        "tokens_per_s_per_layer": round(cfg.batch / (us_per_step * 1e-6), 1),
        "algorithmic_bytes_per_step": int(round(lb.per_step)),
        "kernels": {
            "flush_us": round(flush_avg, 2), "flush_launches": len(flush_us),
            "flush_bytes": int(round(flush_bytes)), "flush_gbs": round(flush_gbs, 1),
            "read_us": round(read_avg, 2), "read_launches": len(read_us),
            "read_bytes_avg": int(round(read_bytes)), "read_gbs": round(read_gbs, 1),
            "timing": "eager launches bracketed by HIP events on the launch stream",
        },
        "step_timing": f"{K} steps ({K // W} whole windows) x {L} rotated layers captured in one "
                       f"HIP graph, replayed {REPS} times back to back with HIP events around each "
                       "replay; value = the median replay / (steps x layers)",
        "roofline": {
            "bound": "hbm", "kernel": "flush", "achieved": round(flush_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(flush_gbs / HBM_PEAK_GBS, 4),
            "traffic": flush_traffic(cfg.name),
            "traffic_unit": "HBM bytes per flush launch (rocprofv3 FETCH_SIZE x2 + WRITE_SIZE x1, "
                            "copy-calibrated); null when the flush kernel changed since",
        },
        # the non-flush read call (every kernel of sketchssm_read), the
        # other kernel of the step, against the same peak
        "roofline_read": {
            "bound": "hbm", "kernel": "read call", "achieved": round(read_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(read_gbs / HBM_PEAK_GBS, 4),
            "traffic": read_traffic(cfg.name),
            "traffic_unit": "HBM bytes per read call, averaged over the window's calls (rocprofv3 "
                            "FETCH_SIZE x2 + WRITE_SIZE x1 of every read kernel); null when a read "
                            "kernel changed since",
        },
        "baselines": baselines,
        "sketch_error": approx,
        "state_map": state_map,
        "dense_fallback": dense_block,
        "wy_pullback": wy_block,
        "cpu_baseline": cpu,
    }
    print(json.dumps(result), flush=True)


# HBM bytes per flush launch from rocprofv3 FETCH_SIZE + WRITE_SIZE, each
# scaled by what the counter reads for a 2 GiB copy (FETCH_SIZE x 2.000,
# WRITE_SIZE x 1.000), with the digest of the flush kernel's sources at the
# time the counters were taken.  A different digest means the kernel has
# changed since, and the figure is reported as null.
TRAFFIC = {
    "m2_b320": {"bytes": 2902282922,
                "src_sha256": "e1ee89e72ae57e1f55a04c5fb16f1cf495d3c16ed23417b55a529ed49b74fecc"},
    "gdn_b256": {"bytes": 1160803639,
                 "src_sha256": "e1ee89e72ae57e1f55a04c5fb16f1cf495d3c16ed23417b55a529ed49b74fecc"},
    "kda_b256": {"bytes": 1222477881,
                 "src_sha256": "e1ee89e72ae57e1f55a04c5fb16f1cf495d3c16ed23417b55a529ed49b74fecc"},
}
FLUSH_SOURCES = ("sk_tile.hpp", "sk_tile_body.inc", "sk_device.hpp", "sk_params.hpp", "sk_dispatch.hpp",
                 "sk_m2.hip", "sk_gdn.hip", "sk_kda.hip")


def timed_steps(k_req: int, window: int) -> int:
    """The steps timed for a request of k_req: rounded up to whole windows,
    at least one window, so that every layer's window (one flush, W - 1
    reads) is timed whole."""
    return max(window, -(-k_req // window) * window)


# HBM bytes per read call (every kernel of sketchssm_read; mean over the
# window's calls) from the same counter runs, with the digest of the read
# kernels' sources at that time.
TRAFFIC_READ = {
    "m2_b320": {"bytes": 113364584, "src_sha256": "94c78e460afb66aa8ab643aad06b5fc8ecc00f6d7ee781b8dd17b24d11f946cc"},
    "gdn_b256": {"bytes": 62938981, "src_sha256": "94c78e460afb66aa8ab643aad06b5fc8ecc00f6d7ee781b8dd17b24d11f946cc"},
    "kda_b256": {"bytes": 99139966, "src_sha256": "94c78e460afb66aa8ab643aad06b5fc8ecc00f6d7ee781b8dd17b24d11f946cc"},
}
READ_SOURCES = ("sk_read.hpp", "sk_device.hpp", "sk_params.hpp", "sk_dispatch.hpp",
                "sk_m2.hip", "sk_gdn.hip", "sk_kda.hip")


def _digest(files):
    import hashlib
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, "ssm_decode_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()


def read_traffic(name):
    e = TRAFFIC_READ.get(name)
    if e is None or e["src_sha256"] != read_src_digest():
        return None
    return e["bytes"]


def flush_src_digest():
    return _digest(FLUSH_SOURCES)


def read_src_digest():
    return _digest(READ_SOURCES)


def flush_traffic(name):
    e = TRAFFIC.get(name)
    if e is None or e["src_sha256"] != flush_src_digest():
        return None
    return e["bytes"]


def sketch_error(cfg, li, src, pool, steps, coef="fixed"):
    """Relative L2 error of the sketched read against the exact read on the
    same state and inputs: one fresh layer runs the sketch path (prime, read,
    flush when due) with the fixed or the state-dependent coefficient map,
    another the ReplaySSM step, whose outputs are exact.
    Synthetic states and queries have no low-rank structure, so this is far
    from the pages' figures on model states; it is reported, not gated."""
    import numpy as np
    import torch
    from ssm_decode_amd import abi, feed
    from ssm_decode_amd.layer import DeviceStep
    ls, lr = feed.make_layer(cfg, li, coef=coef), feed.make_layer(cfg, li)
    ls.S.copy_(src.S)
    lr.S.copy_(src.S)
    assert feed.prime(ls, li) == 0
    lr.count.copy_(torch.from_numpy(li.count0).to(lr.count.device))
    os_, or_ = ls.new_step().o, lr.new_step().o
    errs, flush_errs = [], []
    for t in range(steps):
        p = pool[t % len(pool)]
        ss = DeviceStep(p.q, p.k, p.v, p.gate, p.beta, os_).struct()
        sr = DeviceStep(p.q, p.k, p.v, p.gate, p.beta, or_).struct()
        assert abi.sketchssm_read(ls.layer_struct, ls.buffers_struct, ss, None) == 0
        due = bool((ls.count == cfg.window).any().item())
        if due:
            assert abi.sketchssm_flush(ls.layer_struct, ls.buffers_struct, ss, abi.SKSSM_FLUSH_DUE, None) == 0
        assert abi.sketchssm_replay_step(lr.layer_struct, lr.buffers_struct, sr, None) == 0
        a, b = os_.double(), or_.double()
        e = float(torch.linalg.vector_norm(a - b) / torch.linalg.vector_norm(b))
        (flush_errs if due and not cfg.ragged else errs).append(e)
    del ls, lr
    out = {"rel_l2_mean": float(np.mean(errs)), "rel_l2_max": float(np.max(errs)),
           "steps": steps, "against": "ReplaySSM step (exact read), same state and inputs"}
    if flush_errs:
        out["flush_steps_rel_l2_max"] = float(np.max(flush_errs))
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(cfg, li, n_seq, windows):
    """The oracle, as it stands, on a bounded sample: n_seq sequences x every
    head of the workload, whole windows (prime excluded), on all host cores
    (OpenMP over tiles), then a smaller sample on one core; both scaled to
    the whole batch per layer step."""
    import oracle
    allc = _cpu_run(cfg, li, n_seq, windows)
    threads = oracle.num_threads()
    oracle.set_num_threads(1)
    try:
        n1, w1 = max(1, n_seq // 16), max(1, windows // 4)
        one = _cpu_run(cfg, li, n1, w1)
    finally:
        oracle.set_num_threads(threads)
    return {"value": allc["value"], "unit": "us/step", "cores": threads, "kind": "oracle",
            "sample": allc["sample"], "seconds": allc["seconds"],
            "value_1core": one["value"], "sample_1core": one["sample"], "seconds_1core": one["seconds"],
            "cpu_model": cpu_model(), "nproc": os.cpu_count(),
            "omp_num_threads": os.environ.get("OMP_NUM_THREADS")}


def _cpu_run(cfg, li, n_seq, windows):
    import numpy as np
    import oracle
    import synth
    seqs = np.arange(n_seq)
    tiles = np.array([(b, h) for b in seqs for h in range(cfg.heads)], dtype=np.int64)
    S0 = synth.initial_state(cfg, b_idx=seqs).reshape(-1, cfg.dk, cfg.dv)
    orc = oracle.OracleLayer(cfg.family, cfg.dk, cfg.dv, cfg.window, li.ranks, li.offsets, li.Pt,
                             li.C, li.A, tiles, S0, cfg.heads, cfg.qk_groups, state_store="f32",
                             sketch_store=cfg.sketch, out_store=cfg.act)
    orc.flush(None, all_tiles=True)
    orc.count[:] = li.count0[tiles[:, 0], tiles[:, 1]]
    nsteps = windows * cfg.window
    dt = 0.0
    for t in range(nsteps):
        st = synth.make_step_inputs(cfg, t, b_idx=seqs)      # generation is not timed
        o = np.zeros((len(tiles), cfg.dv))
        t0 = time.perf_counter()
        orc.read(st, o=o)
        if (orc.count == cfg.window).any():
            orc.flush(st, o=o)
        dt += time.perf_counter() - t0
    frac = cfg.batch / n_seq
    us = dt / nsteps * frac * 1e6
    return {"value": round(us, 1),
            "sample": f"{n_seq} of {cfg.batch} sequences x {cfg.heads} heads, {windows} windows of "
                      f"{cfg.window} steps ({dt:.1f} s), scaled to the batch",
            "seconds": round(dt, 2)}


if __name__ == "__main__":
    main()
