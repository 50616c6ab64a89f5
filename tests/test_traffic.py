"""Byte accounting: the App. D state-traffic model against the ratios the
pages print (tests/golden/app_d_traffic.txt), and invariants of the
algorithmic byte model the benchmark reports."""
import os

import pytest

from ssm_decode_amd import traffic

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "app_d_traffic.txt")


def _golden_rows():
    rows = []
    for line in open(GOLDEN):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        m, K, V, G, W, printed = line.split()
        rows.append((m, int(K), int(V), int(G), int(W), printed))
    return rows


@pytest.mark.parametrize("row", _golden_rows())
def test_app_d_ratio_matches_printed(row):
    method, K, V, G, W, printed = row
    ratio = traffic.state_traffic_ratio(K, V, G, W, method=method)
    assert f"{ratio:.2f}" == printed


def test_replay_ratio_is_2w_over_w_plus_1():
    for W in (1, 4, 16, 32):
        assert traffic.state_traffic_ratio(128, 64, 8, W, "replay") == pytest.approx(2 * W / (W + 1))


def test_window_one_sketch_reads_the_state_every_step():
    # W = 1: every step is a flush, so the sketch path moves the standard bytes
    assert traffic.state_traffic_ratio(128, 64, 8, 1, "sketch") == pytest.approx(1.0)


def _lb(**kw):
    base = dict(family="mamba2", B=320, H=128, G=8, dk=128, dv=64, W=16, R=1024,
                act="bf16", sketch="bf16")
    base.update(kw)
    return traffic.layer_bytes(**base)


def test_window_is_flush_plus_reads():
    for kw in ({}, dict(family="gdn", G=32, H=32, dv=128, R=256, B=256),
               dict(family="kda", G=32, H=32, dv=128, R=256, B=256), dict(W=8), dict(W=32)):
        lb = _lb(**kw)
        assert lb.per_window == lb.flush_launch + round(lb.read_launch_avg * (kw.get("W", 16)))
        assert lb.per_step * kw.get("W", 16) == lb.per_window


def test_state_dominates_the_flush_and_is_absent_from_reads():
    lb = _lb()
    S = 320 * 128 * 128 * 64 * 4
    assert lb.flush_launch > 2 * S
    assert lb.flush_launch - 2 * S < 0.1 * 2 * S
    # a non-flush read never touches S: doubling dk*dv*4 of the state does
    # not change the read bytes except through the basis rows and keys
    lb2 = _lb(dv=128)
    assert lb2.read_launch_avg < 2.1 * lb.read_launch_avg


def test_bytes_scale_linearly_with_batch():
    a, b = _lb(B=160), _lb(B=320)
    basis = 16 * 1024 * 128 * 4
    assert (b.per_window - basis) == 2 * (a.per_window - basis)
    assert b.full_step == 2 * a.full_step


def test_sketch_beats_replay_beats_standard_per_step():
    lb = _lb()
    assert lb.per_step < lb.replay_per_step < lb.full_step


def test_state_map_bytes():
    """The state-dependent map adds each sequence's R x dk map (sketch dtype)
    written at the flush and read at the other W-1 steps, and drops the
    fixed map's shared rows from the W-1 read launches."""
    B, H, G, dk, dv, W, R = 320, 128, 8, 128, 64, 16, 1024
    fx = traffic.layer_bytes("mamba2", B, H, G, dk, dv, W, R, "bf16", "bf16")
    st = traffic.layer_bytes("mamba2", B, H, G, dk, dv, W, R, "bf16", "bf16", coef="state")
    Cseq = R * dk * 2
    assert st.per_window - fx.per_window == B * W * Cseq - (W - 1) * R * dk * 4
    assert st.flush_launch - fx.flush_launch == B * Cseq
    assert st.full_step == fx.full_step and st.replay_per_step == fx.replay_per_step


def test_dense_head_bytes():
    """A dense-fallback head moves its state copy where a sketched head moves
    its sketch: written at the flush and read at the other W-1 steps."""
    B, H, G, dk, dv, W = 320, 128, 8, 128, 64, 16
    base = traffic.layer_bytes("mamba2", B, H, G, dk, dv, W, 1024, "bf16", "bf16")
    d4 = traffic.layer_bytes("mamba2", B, H, G, dk, dv, W, 1024, "bf16", "bf16", dense=4)
    assert d4.per_window - base.per_window == B * W * 4 * dk * dv * 2
    assert d4.flush_launch - base.flush_launch == B * 4 * dk * dv * 2
