"""The C-ABI library loads, exports every entry point its header declares,
and rejects invalid arguments on the host without launching anything (runs
without a GPU: every call here fails validation or has batch 0)."""
import ctypes as C
import os
import re

import numpy as np
import pytest

from ssm_decode_amd import abi

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "sketchssm.h")


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(abi.LIB_PATH):
        from ssm_decode_amd.build import build
        build()
    return abi.load()


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^(?:int|int64_t)\s+(sketchssm_\w+)\s*\(", text, flags=re.M)))


def test_exports_every_declared_symbol(lib):
    names = declared_functions()
    assert set(names) == set(abi.ENTRY_POINTS)
    for n in names:
        assert hasattr(lib, n), n
    assert abi.sketchssm_version() == 102


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict((k, int(v)) for k, v in re.findall(r"#define\s+(SKSSM_\w+)\s+(-?\d+)", text))
    for k, v in consts.items():
        assert getattr(abi, k) == v, k


FAKE = 0x10000  # aligned, never dereferenced: validation fails before any launch


def _layer(offsets, family=abi.SKSSM_MAMBA2, batch=2, heads=4, groups=4, dk=16, dv=32, W=4,
           act=abi.SKSSM_F32, sk=abi.SKSSM_F32, coef=abi.SKSSM_COEF_FIXED, ridge=0.0):
    off = np.ascontiguousarray(np.asarray(offsets, dtype=np.int32))
    L = abi.sketchssm_layer(family, batch, heads, groups, dk, dv, W, act, sk,
                            off.ctypes.data_as(C.POINTER(C.c_int32)), coef, ridge)
    L._keep = off
    return L


def _bufs(**over):
    f = dict(S=FAKE, U=FAKE, Pt=FAKE, C=FAKE, rank_offsets=FAKE, ring_k=FAKE, ring_v=FAKE,
             ring_gate=FAKE, ring_beta=FAKE, count=FAKE, A=FAKE, err=FAKE, work=FAKE, Cstate=FAKE,
             Scopy=FAKE, ring_pc=FAKE)
    f.update(over)
    return abi.sketchssm_buffers(**f)


def _step(**over):
    f = dict(q=FAKE, k=FAKE, v=FAKE, gate=FAKE, beta=FAKE, o=FAKE)
    f.update(over)
    return abi.sketchssm_step(**f)


OK_OFF = [0, 4, 8, 12, 16]


def _all_calls(L, B, S, flags=abi.SKSSM_FLUSH_DUE):
    return [abi.sketchssm_read(L, B, S), abi.sketchssm_flush(L, B, S, flags),
            abi.sketchssm_full_step(L, B, S), abi.sketchssm_replay_step(L, B, S)]


def test_batch_zero_is_a_no_op(lib):
    assert _all_calls(_layer(OK_OFF, batch=0), _bufs(), _step()) == [0, 0, 0, 0]


@pytest.mark.parametrize("kw,code", [
    (dict(family=3), abi.SKSSM_EDIM),
    (dict(act=abi.SKSSM_BF16), abi.SKSSM_EDTYPE),          # act != sketch dtype
    (dict(act=2, sk=2), abi.SKSSM_EDTYPE),
    (dict(dk=32, dv=32), abi.SKSSM_EDIM),
    (dict(W=0), abi.SKSSM_EDIM),
    (dict(W=33), abi.SKSSM_EDIM),
    (dict(heads=4, groups=3), abi.SKSSM_EDIM),
    (dict(family=abi.SKSSM_GDN, groups=2), abi.SKSSM_EDIM),
    (dict(batch=-1), abi.SKSSM_EDIM),
])
def test_bad_layer(lib, kw, code):
    assert _all_calls(_layer(OK_OFF, **kw), _bufs(), _step()) == [code] * 4


def test_heads_per_group_limit(lib):
    off = list(range(0, 4 * 33, 4))
    L = _layer(off, heads=32, groups=1)
    L2 = _layer(off, heads=32, groups=2)
    assert abi.sketchssm_read(L, _bufs(), _step()) == abi.SKSSM_EDIM
    assert abi.sketchssm_read(_layer(off, heads=32, groups=2, batch=0), _bufs(), _step()) == 0
    del L2


@pytest.mark.parametrize("off", [[1, 4, 8, 12, 16], [0, 4, 8, 12, 29], [0, 4, 3, 8, 12]])
def test_bad_rank_table(lib, off):
    assert _all_calls(_layer(off), _bufs(), _step()) == [abi.SKSSM_EDIM] * 4


def test_rank_limit_is_min_dk_16(lib):
    L = _layer([0, 16, 32, 48, 64], batch=0)          # r = dk = 16 allowed
    assert _all_calls(L, _bufs(), _step()) == [0] * 4
    L = _layer([0, 17, 34, 51, 68], dk=128, dv=64, batch=1)
    assert _all_calls(L, _bufs(), _step()) == [abi.SKSSM_EDIM] * 4


def test_null_and_misaligned_pointers(lib):
    L = _layer(OK_OFF)
    assert abi.sketchssm_read(None, _bufs(), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, None, _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(), None) == abi.SKSSM_EINVAL
    assert abi.sketchssm_full_step(L, _bufs(), None) == abi.SKSSM_EINVAL
    assert abi.sketchssm_replay_step(L, _bufs(), None) == abi.SKSSM_EINVAL
    assert abi.sketchssm_flush(L, _bufs(S=FAKE + 4), None, abi.SKSSM_FLUSH_ALL) == abi.SKSSM_EINVAL
    assert abi.sketchssm_flush(L, _bufs(U=None), None, abi.SKSSM_FLUSH_ALL) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(C=FAKE + 8), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(), _step(o=FAKE + 2)) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(A=None), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_replay_step(L, _bufs(count=None), _step()) == abi.SKSSM_EINVAL
    Lg = _layer(OK_OFF, family=abi.SKSSM_GDN)
    assert abi.sketchssm_read(Lg, _bufs(ring_beta=None), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(Lg, _bufs(), _step(beta=None)) == abi.SKSSM_EINVAL
    # a flush without a step writes no output and needs no step pointers
    assert abi.sketchssm_flush(_layer(OK_OFF, batch=0), _bufs(), None, abi.SKSSM_FLUSH_ALL) == 0


def test_bad_flag(lib):
    assert abi.sketchssm_flush(_layer(OK_OFF), _bufs(), None, 4) == abi.SKSSM_EFLAG
    assert abi.sketchssm_flush(_layer(OK_OFF), _bufs(), None, -1) == abi.SKSSM_EFLAG


def test_scan_flush_needs_the_workspace(lib):
    """SKSSM_FLUSH_DUE_SCAN lists the due tiles in bufs.work: a missing or
    misaligned workspace is EINVAL; batch 0 is a no-op."""
    for fam in (abi.SKSSM_MAMBA2, abi.SKSSM_GDN, abi.SKSSM_KDA):
        L = _layer(OK_OFF, family=fam)
        assert abi.sketchssm_flush(L, _bufs(work=None), None, abi.SKSSM_FLUSH_DUE_SCAN) == abi.SKSSM_EINVAL
        assert abi.sketchssm_flush(L, _bufs(work=FAKE + 8), None, abi.SKSSM_FLUSH_DUE_SCAN) == abi.SKSSM_EINVAL
        L0 = _layer(OK_OFF, family=fam, batch=0)
        assert abi.sketchssm_flush(L0, _bufs(work=None), None, abi.SKSSM_FLUSH_DUE_SCAN) == 0


def test_closing_flush_needs_the_step(lib):
    """SKSSM_FLUSH_CLOSE takes the step's own entry and writes its output: no
    step, or a missing or misaligned key, value, gate (beta for the delta
    rule), query or output is EINVAL; batch 0 is a no-op."""
    for fam in (abi.SKSSM_MAMBA2, abi.SKSSM_GDN, abi.SKSSM_KDA):
        L = _layer(OK_OFF, family=fam)
        assert abi.sketchssm_flush(L, _bufs(), None, abi.SKSSM_FLUSH_CLOSE) == abi.SKSSM_EINVAL
        fields = ("k", "v", "gate", "q", "o") + (("beta",) if fam != abi.SKSSM_MAMBA2 else ())
        for f in fields:
            for bad in (None, FAKE + 4):
                assert abi.sketchssm_flush(L, _bufs(), _step(**{f: bad}),
                                           abi.SKSSM_FLUSH_CLOSE) == abi.SKSSM_EINVAL, (fam, f, bad)
        L0 = _layer(OK_OFF, family=fam, batch=0)
        assert abi.sketchssm_flush(L0, _bufs(), _step(), abi.SKSSM_FLUSH_CLOSE) == 0


def _m2_work_bytes(B, R, G, W):
    # the query in every head's basis [B][R], the key-query dot products
    # [B][G][W] and the checked ring fill [B][G], 4 bytes each, every region
    # rounded up to 256 bytes
    a64 = lambda n: (n + 63) // 64 * 64
    return 4 * (a64(B * R) + a64(B * G * W) + a64(B * G))


def _scan_work_bytes(B):
    # the scan flush's due list: the number of due sequences (in a first
    # block of 64 entries), then the list of up to B sequences rounded up to
    # 64 entries, int32
    return 4 * (64 + (B + 63) // 64 * 64)


def test_workspace_bytes(lib):
    """The workspace is the larger of the read's and the scan flush's needs."""
    assert _m2_work_bytes(2, 16, 4, 4) == 768 and _scan_work_bytes(2) == 512
    assert abi.sketchssm_workspace_bytes(_layer(OK_OFF, batch=2)) == 768
    off = np.concatenate([[0], np.cumsum(np.full(128, 8))]).astype(np.int32)
    L = _layer(off, batch=320, heads=128, groups=8, dk=128, dv=64, W=16)
    assert _m2_work_bytes(320, 1024, 8, 16) > _scan_work_bytes(320)
    assert abi.sketchssm_workspace_bytes(L) == _m2_work_bytes(320, 1024, 8, 16)
    L = _layer(off, batch=1024, heads=128, groups=8, dk=128, dv=64, W=32)
    assert abi.sketchssm_workspace_bytes(L) == max(_m2_work_bytes(1024, 1024, 8, 32),
                                                   _scan_work_bytes(1024))
    for fam in (abi.SKSSM_GDN, abi.SKSSM_KDA):
        assert abi.sketchssm_workspace_bytes(_layer(OK_OFF, family=fam)) == _scan_work_bytes(2)
        assert abi.sketchssm_workspace_bytes(_layer(OK_OFF, family=fam, batch=0)) == 0
    assert abi.sketchssm_workspace_bytes(_layer(OK_OFF, W=0)) == abi.SKSSM_EDIM
    assert abi.sketchssm_workspace_bytes(None) == abi.SKSSM_EINVAL


def _dn_work_bytes(B, D, dk, dv):
    # per (sequence, dense head) the pulled-back query [B][D][dk], the
    # buffered term [B][D][dv] and a flag [B][D], 4 bytes each, every region
    # rounded up to 256 bytes
    a64 = lambda n: (n + 63) // 64 * 64
    return 4 * (a64(B * D * dk) + a64(B * D * dv) + a64(B * D))


def test_workspace_bytes_delta_rule_dense_heads(lib):
    """GDN/KDA layers need a workspace only when they have dense-fallback
    heads, and then the read requires it."""
    for fam in (abi.SKSSM_GDN, abi.SKSSM_KDA):
        L = _layer([0, 4, 4, 8, 8], family=fam, batch=3)          # heads 1 and 3 dense
        assert _dn_work_bytes(3, 2, 16, 32) == 1536
        assert abi.sketchssm_workspace_bytes(L) == max(1536, _scan_work_bytes(3))
        assert abi.sketchssm_read(L, _bufs(work=None), _step()) == abi.SKSSM_EINVAL
        assert abi.sketchssm_read(L, _bufs(work=FAKE + 4), _step()) == abi.SKSSM_EINVAL
        off = np.concatenate([[0], np.cumsum([0] + [8] * 31)]).astype(np.int32)
        L = _layer(off, family=fam, batch=256, heads=32, groups=32, dk=128, dv=128, W=16)
        assert abi.sketchssm_workspace_bytes(L) == max(_dn_work_bytes(256, 1, 128, 128),
                                                       _scan_work_bytes(256))


def test_read_needs_its_workspace(lib):
    L = _layer(OK_OFF)
    assert abi.sketchssm_read(L, _bufs(work=None), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(work=FAKE + 4), _step()) == abi.SKSSM_EINVAL
    # the other calls, and families with no workspace, do not look at it
    assert abi.sketchssm_flush(_layer(OK_OFF, batch=0), _bufs(work=None), None,
                               abi.SKSSM_FLUSH_ALL) == 0
    Lg = _layer(OK_OFF, family=abi.SKSSM_GDN, batch=0)
    assert abi.sketchssm_read(Lg, _bufs(work=None), _step()) == 0
    assert abi.sketchssm_read(_layer(OK_OFF, batch=0), _bufs(work=None), _step()) == 0


def test_coefficient_map_mode(lib):
    """The map mode is a flag (unknown values: EFLAG); the state-dependent map
    needs a finite positive ridge and Cstate for the read and the flush, and
    no fixed table C; the fixed map never looks at Cstate."""
    for bad in (2, -1):
        L = _layer(OK_OFF, coef=bad, ridge=1e-4)
        assert _all_calls(L, _bufs(), _step()) == [abi.SKSSM_EFLAG] * 4
    for ridge in (0.0, -1e-3, float("nan"), float("inf")):
        L = _layer(OK_OFF, coef=abi.SKSSM_COEF_STATE, ridge=ridge)
        assert _all_calls(L, _bufs(), _step()) == [abi.SKSSM_EINVAL] * 4
    L = _layer(OK_OFF, coef=abi.SKSSM_COEF_STATE, ridge=1e-4)
    for cs in (None, FAKE + 8):
        assert abi.sketchssm_read(L, _bufs(Cstate=cs), _step()) == abi.SKSSM_EINVAL
        assert abi.sketchssm_flush(L, _bufs(Cstate=cs), None, abi.SKSSM_FLUSH_ALL) == abi.SKSSM_EINVAL
    L0 = _layer(OK_OFF, coef=abi.SKSSM_COEF_STATE, ridge=1e-4, batch=0)
    assert _all_calls(L0, _bufs(C=None), _step()) == [0] * 4
    assert abi.sketchssm_full_step(L0, _bufs(Cstate=None), _step()) == 0
    assert abi.sketchssm_replay_step(L0, _bufs(Cstate=None), _step()) == 0
    Lf = _layer(OK_OFF, batch=0)
    assert _all_calls(Lf, _bufs(Cstate=None), _step()) == [0] * 4
    assert abi.sketchssm_read(_layer(OK_OFF), _bufs(C=None), _step()) == abi.SKSSM_EINVAL


def test_pullback_mode(lib):
    """The pull-back mode is a flag: serial, the triangular-system form or
    that form with projected factors; unknown values are EFLAG on every
    call.  The projected form's GDN/KDA read needs the factor ring."""
    for bad in (3, -1):
        L = _layer(OK_OFF, family=abi.SKSSM_GDN)
        L.pullback = bad
        assert _all_calls(L, _bufs(), _step()) == [abi.SKSSM_EFLAG] * 4
    for fam in (abi.SKSSM_MAMBA2, abi.SKSSM_GDN, abi.SKSSM_KDA):
        for pb in (abi.SKSSM_PULLBACK_WY, abi.SKSSM_PULLBACK_PROJ):
            L = _layer(OK_OFF, family=fam, batch=0)
            L.pullback = pb
            assert _all_calls(L, _bufs(), _step()) == [0] * 4
    for fam in (abi.SKSSM_GDN, abi.SKSSM_KDA):
        L = _layer(OK_OFF, family=fam)
        L.pullback = abi.SKSSM_PULLBACK_PROJ
        for bad in (None, FAKE + 4):
            assert abi.sketchssm_read(L, _bufs(ring_pc=bad), _step()) == abi.SKSSM_EINVAL
            assert abi.sketchssm_read_noalloc(L, _bufs(ring_pc=bad), _step()) == abi.SKSSM_EINVAL
        # the flush and the baselines do not read the factors
        assert abi.sketchssm_flush(_layer(OK_OFF, family=fam, batch=0), _bufs(ring_pc=None), None,
                                   abi.SKSSM_FLUSH_ALL) == 0


def test_dense_fallback_heads(lib):
    """r_h = 0 marks a dense-fallback head: allowed, and then the read and
    the flush need the state copies (Scopy); a layer with no sketched head
    needs no U, basis or map."""
    L = _layer([0, 4, 4, 8, 12])                   # head 1 is dense
    assert abi.sketchssm_read(L, _bufs(Scopy=None), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read(L, _bufs(Scopy=FAKE + 4), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_flush(L, _bufs(Scopy=None), None, abi.SKSSM_FLUSH_ALL) == abi.SKSSM_EINVAL
    L0 = _layer([0, 4, 4, 8, 12], batch=0)
    assert _all_calls(L0, _bufs(), _step()) == [0] * 4
    assert abi.sketchssm_full_step(_layer([0, 4, 4, 8, 12]), _bufs(Scopy=None), None) == abi.SKSSM_EINVAL
    Ld = _layer([0, 0, 0, 0, 0], batch=0)            # every head dense: R = 0
    assert _all_calls(Ld, _bufs(U=None, Pt=None, C=None, Cstate=None), _step()) == [0] * 4
    assert abi.sketchssm_workspace_bytes(_layer([0, 0, 0, 0, 0])) == max(_m2_work_bytes(2, 0, 4, 4),
                                                                      _scan_work_bytes(2))
    # at most 64 dense heads per layer
    off = np.concatenate([[0], np.cumsum([0] * 65 + [4] * 63)]).astype(np.int32)
    assert abi.sketchssm_read(_layer(off, heads=128, groups=128, family=abi.SKSSM_GDN, batch=0),
                              _bufs(), _step()) == abi.SKSSM_EDIM
    off = np.concatenate([[0], np.cumsum([0] * 64 + [4] * 64)]).astype(np.int32)
    assert abi.sketchssm_read(_layer(off, heads=128, groups=128, family=abi.SKSSM_GDN, batch=0),
                              _bufs(), _step()) == 0
    # with sketched heads the sketch is still required
    assert abi.sketchssm_read(_layer([0, 4, 4, 8, 12]), _bufs(U=None), _step()) == abi.SKSSM_EINVAL


def test_flush_seqs_arguments():
    """The listed flush checks its list on the host: count in [0, batch], a
    4-byte aligned device pointer when the list is not empty; an empty list
    launches nothing."""
    import ctypes as C
    L = _layer(OK_OFF, batch=2)
    B = _bufs()
    seqs = C.c_void_p(FAKE)
    assert abi.sketchssm_flush_seqs(L, B, None, seqs, -1) == abi.SKSSM_EDIM
    assert abi.sketchssm_flush_seqs(L, B, None, seqs, 3) == abi.SKSSM_EDIM
    assert abi.sketchssm_flush_seqs(L, B, None, None, 1) == abi.SKSSM_EINVAL
    assert abi.sketchssm_flush_seqs(L, B, None, C.c_void_p(FAKE + 2), 1) == abi.SKSSM_EINVAL
    assert abi.sketchssm_flush_seqs(L, B, None, None, 0) == abi.SKSSM_OK
    assert abi.sketchssm_flush_seqs(L, _bufs(S=FAKE + 4), None, seqs, 1) == abi.SKSSM_EINVAL


def test_flush_seqs_binding_rejects_host_or_wrong_lists():
    """The Python binding refuses a list the kernel could not read: host
    memory, another dtype, or a non-contiguous view (checked before any
    call into the library)."""
    import torch
    from ssm_decode_amd.layer import DecodeLayer

    class _Stub:                    # only the argument checks of flush_seqs run
        flush_seqs = DecodeLayer.flush_seqs
    with pytest.raises(ValueError):
        _Stub().flush_seqs(None, torch.zeros(2, dtype=torch.int32))
    with pytest.raises(ValueError):
        _Stub().flush_seqs(None, torch.zeros(2, dtype=torch.int64))
    with pytest.raises(ValueError):
        _Stub().flush_seqs(None, torch.zeros(4, dtype=torch.int32)[::2])


def test_read_noalloc_validation(lib):
    """The read without a workspace argument validates like the read, ignores
    bufs.work, and refuses (SKSSM_ESCRATCH, nothing launched) a layer whose
    workspace exceeds the library's scratch array; batch 0 is a no-op that
    does not touch the device."""
    L0 = _layer(OK_OFF, batch=0)
    assert abi.sketchssm_read_noalloc(L0, _bufs(work=None), _step()) == 0
    L = _layer(OK_OFF)
    assert abi.sketchssm_read_noalloc(L, _bufs(C=FAKE + 8), _step()) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read_noalloc(L, _bufs(), None) == abi.SKSSM_EINVAL
    assert abi.sketchssm_read_noalloc(_layer(OK_OFF, W=33), _bufs(), _step()) == abi.SKSSM_EDIM
    # the largest Mamba-2 layer that fits, and one sequence more: the query in
    # every head's basis alone is 4 B x R per sequence
    off = np.concatenate([[0], np.cumsum(np.full(128, 16))]).astype(np.int32)   # R = 2048
    cap = abi.SKSSM_NOALLOC_SCRATCH_BYTES
    Bfit = max(b for b in range(1, 4096) if _m2_work_bytes(b, 2048, 8, 32) <= cap)
    Lbig = _layer(off, batch=Bfit + 1, heads=128, groups=8, dk=128, dv=64, W=32)
    assert abi.sketchssm_workspace_bytes(Lbig) > cap
    assert abi.sketchssm_read_noalloc(Lbig, _bufs(), _step()) == abi.SKSSM_ESCRATCH
    assert abi.sketchssm_read_noalloc(Lbig, _bufs(work=None), _step()) == abi.SKSSM_ESCRATCH
    assert Bfit >= 1024                   # the batch-1024 stress layers fit
