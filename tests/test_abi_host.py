"""Host-side checks of the C ABI (no GPU): the library loads and exports every
declared entry point, the schedule generator is bit-exact against the oracle,
and the executor's bookkeeping (validation, slots, live counts, op log,
error codes) matches the oracle on bookkeeping-only handles."""

import ctypes
import os
import re
import subprocess

import pytest

from oracle import schedule as S
from tests.conftest import ROOT

pps = pytest.importorskip("pipeline_schedules_amd.pps")


def _lib_or_skip():
    if not os.path.exists(pps._LIB_PATH):
        pytest.fail("libpps.so is not built; run `python -m pipeline_schedules_amd.build` first")
    return pps.lib()


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "pps.h"), encoding="utf-8").read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pps_[a-z_]+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = _lib_or_skip()
    names = _declared_functions()
    assert len(names) >= 14
    for n in names:
        assert hasattr(lib, n), n
    out = subprocess.run(["nm", "-D", "--defined-only", pps._LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (pps_\w+)", out))
    assert set(names) <= exported
    assert set(pps.EXPORTED) == set(names)


def _oracle_kind(kind):
    return {pps.GPIPE: S.GPIPE, pps.ONE_F_ONE_B: S.ONE_F_ONE_B, pps.ZB1P: S.ZB1P, pps.ZB2P: S.ZB2P}[kind]


@pytest.mark.parametrize("kind", [pps.GPIPE, pps.ONE_F_ONE_B, pps.ZB1P, pps.ZB2P])
def test_make_schedule_bit_exact_v1(kind):
    _lib_or_skip()
    for P in (1, 2, 3, 4, 5, 8, 16):
        for M in sorted({1, 2, P - 1, P, P + 1, 2 * P, 3 * P + 1, 64} - {0}):
            for k in range(P):
                got = pps.make_schedule(P, M, k, 1, kind)
                want = S.stage_ops(P, M, k, 1, _oracle_kind(kind))
                assert got == [tuple(w) for w in want], (P, M, k, kind)


@pytest.mark.parametrize("v", [2, 3, 4])
def test_make_schedule_bit_exact_interleaved(v):
    _lib_or_skip()
    for P in (1, 2, 3, 4, 8):
        for M in (P, 2 * P, 4 * P, 8 * P):
            if M > 64:
                continue
            for k in range(P):
                got = pps.make_schedule(P, M, k, v, pps.ONE_F_ONE_B)
                want = S.stage_ops(P, M, k, v, S.ONE_F_ONE_B)
                assert got == [tuple(w) for w in want], (P, M, k, v)


def test_make_schedule_headline_values():
    _lib_or_skip()
    ops = pps.make_schedule(8, 16, 0, 1, pps.ONE_F_ONE_B)
    assert len(ops) == 32
    assert [("FBW"[o[0]] + str(o[1])) for o in ops][:10] == ["F0", "F1", "F2", "F3", "F4", "F5", "F6", "F7", "B0", "F8"]
    assert max(o[4] for o in ops) == 8
    ops = pps.make_schedule(8, 16, 0, 2, pps.ONE_F_ONE_B)
    assert len(ops) == 64 and max(o[4] for o in ops) == 23
    ops = pps.make_schedule(4, 32, 0, 1, pps.ZB1P)
    assert len(ops) == 96 and max(o[4] for o in ops) == 4
    ops = pps.make_schedule(4, 32, 0, 1, pps.ZB2P)
    assert len(ops) == 96 and max(o[4] for o in ops) == 8
    assert [o[0] for o in ops].index(pps.OP_B) == 7            # 2(P-k)-1 warmup forwards
    assert ops[-1][5] + 1 - ops[0][5] == 96                    # no idle slot in stage 0's span


def test_make_schedule_errors():
    lib = _lib_or_skip()
    import ctypes
    n = ctypes.c_int(-1)
    for args in [(0, 4, 0, 1, 1), (4, 0, 0, 1, 1), (4, 4, 4, 1, 1), (4, 4, -1, 1, 1), (4, 4, 0, 0, 1),
                 (4, 6, 0, 2, 1), (4, 8, 0, 2, pps.GPIPE), (4, 8, 0, 2, pps.ZB1P), (4, 4, 0, 1, 9)]:
        assert lib.pps_make_schedule(*args, None, 0, ctypes.byref(n)) == pps.EINVAL, args
    assert lib.pps_make_schedule(4, 6, 0, 1, 1, None, 0, None) == pps.EINVAL
    arr = (pps.PpsOp * 3)()
    assert lib.pps_make_schedule(4, 6, 0, 1, 1, arr, 3, ctypes.byref(n)) == pps.EFULL
    assert n.value == 12


def _bk_stage(P, M, k, v=1, kind=pps.ONE_F_ONE_B, L=2, d=64, ffn=128, T=16, block=pps.BLOCK_SWIGLU,
              dtype=pps.DTYPE_BF16, flags=0):
    return pps.Stage(P=P, M=M, k=k, v=v, kind=kind, block=block, dtype=dtype, L=L, d=d, ffn=ffn, T=T,
                     flags=pps.FLAG_BOOKKEEPING_ONLY | flags)


def _drive(stage, ops):
    for op, mb, c, *_ in ops:
        if op == pps.OP_F:
            stage.forward(mb, c, None, None)
        elif op == pps.OP_B:
            stage.backward(mb, c, None, None)
        else:
            stage.backward_weight(mb, c)


@pytest.mark.parametrize("kind,v", [(pps.ONE_F_ONE_B, 1), (pps.GPIPE, 1), (pps.ZB1P, 1), (pps.ZB2P, 1),
                                    (pps.ONE_F_ONE_B, 2)])
def test_bookkeeping_oplog_matches_oracle(kind, v):
    _lib_or_skip()
    for P in (1, 2, 4, 8):
        for M in (P, 2 * P, 16):
            if v > 1 and M % P:
                continue
            for k in range(P):
                want = [tuple(w) for w in S.stage_ops(P, M, k, v, _oracle_kind(kind))]
                st = _bk_stage(P, M, k, v, kind)
                for rep in range(2):   # two passes: the second reuses the same slots
                    _drive(st, want)
                    assert st.oplog() == want
                s = st.stats()
                peak = max(w[4] for w in want)
                assert s["n_slots"] == peak
                assert s["peak_live_entries"] == peak
                assert s["live_entries"] == 0 and s["live_bytes"] == 0
                assert s["passes_completed"] == 2
                st.close()


def test_bookkeeping_stash_bytes():
    _lib_or_skip()
    T, d, f, L = 16, 64, 128, 2
    a = lambda b: (b + 255) // 256 * 256
    fwd = L * (a(T * d * 2) + a(T * 4) + 2 * a(T * f * 2))
    extra = L * (a(T * 2 * f * 2) + a(T * d * 2))
    st = _bk_stage(4, 8, 0, T=T, d=d, ffn=f, L=L)
    _drive(st, S.stage_ops(4, 8, 0))
    s = st.stats()
    assert s["slot_bytes"] == fwd and s["pool_bytes"] == 4 * fwd and s["peak_live_bytes"] == 4 * fwd
    st = _bk_stage(4, 8, 0, kind=pps.ZB1P, T=T, d=d, ffn=f, L=L)
    ops = S.stage_ops(4, 8, 0, 1, S.ZB1P)
    _drive(st, ops)
    s = st.stats()
    assert s["slot_bytes"] == fwd + extra
    # peak bytes follows the per-op live composition of the oracle schedule
    live_f, live_b, peak = set(), set(), 0
    for op, mb, *_ in ops:
        if op == 0:
            live_f.add(mb)
        elif op == 1:
            live_b.add(mb)
        else:
            live_f.discard(mb)
            live_b.discard(mb)
        peak = max(peak, len(live_f) * fwd + len(live_b) * extra)
    assert s["peak_live_bytes"] == peak


@pytest.mark.parametrize("dtype,es", [(pps.DTYPE_BF16, 2), (pps.DTYPE_FP32, 4)])
def test_bookkeeping_recompute_stash_bytes(dtype, es):
    """Recompute mode: an entry is the stage input [T, d] alone; the per-block
    tensors of one micro-batch move to library scratch."""
    _lib_or_skip()
    T, d, f, L = 24, 64, 128, 3
    a = lambda b: (b + 255) // 256 * 256
    full = L * (a(T * d * es) + a(T * 4) + 2 * a(T * f * es))
    plain = _bk_stage(4, 8, 1, T=T, d=d, ffn=f, L=L, dtype=dtype)
    ac = _bk_stage(4, 8, 1, T=T, d=d, ffn=f, L=L, dtype=dtype, flags=pps.FLAG_RECOMPUTE)
    ops = S.stage_ops(4, 8, 1)
    for st in (plain, ac):
        _drive(st, ops)
        assert st.oplog() == [tuple(o) for o in ops]
    sp, sa = plain.stats(), ac.stats()
    assert sp["slot_bytes"] == full
    assert sa["slot_bytes"] == a(T * d * es) and sa["pool_bytes"] == 3 * a(T * d * es)
    assert sa["peak_live_bytes"] == 3 * a(T * d * es)          # P - k entries
    assert sa["scratch_bytes"] == sp["scratch_bytes"] + full
    for st in (plain, ac):
        st.close()


def test_recompute_rejected_where_undefined():
    _lib_or_skip()
    for kind in (pps.ZB1P, pps.ZB2P):
        with pytest.raises(pps.PpsError):
            _bk_stage(4, 8, 0, kind=kind, flags=pps.FLAG_RECOMPUTE)
    with pytest.raises(pps.PpsError):
        _bk_stage(4, 8, 0, block=pps.BLOCK_TOY_GELU, dtype=pps.DTYPE_FP32, flags=pps.FLAG_RECOMPUTE)
    for kind, v in ((pps.GPIPE, 1), (pps.ONE_F_ONE_B, 2)):
        _bk_stage(4, 8, 0, v=v, kind=kind, flags=pps.FLAG_RECOMPUTE).close()


def test_bookkeeping_error_codes():
    _lib_or_skip()
    P, M = 4, 8
    st = _bk_stage(P, M, 0)
    # backward before any forward
    assert st.backward_status(0, 0, None, None) == pps.ENOENT
    # forward out of order
    assert st.forward_status(1, 0, None, None) == pps.EORDER
    for i in range(P):
        st.forward(i, 0, None, None)
    # backward of a non-oldest entry
    assert st.backward_status(1, 0, None, None) == pps.EORDER
    # the next forward in order, but the pool (P-k = 4 slots) is full
    assert st.forward_status(P, 0, None, None) == pps.EFULL
    # W on an unsplit schedule
    assert st.backward_weight_status(0) == pps.ESTATE
    st.backward(0, 0, None, None)
    # backward twice
    assert st.backward_status(0, 0, None, None) == pps.ESTATE
    # a rejected call leaves the state unchanged
    assert st.oplog() == [tuple(o) for o in S.stage_ops(P, M, 0)[:P + 1]]
    # bad indices
    assert st.forward_status(M, 0, None, None) == pps.EINVAL
    assert st.forward_status(0, 1, None, None) == pps.EINVAL
    st.close()

    zb = _bk_stage(P, M, 0, kind=pps.ZB1P)
    zb.forward(0, 0, None, None)
    assert zb.backward_weight_status(0) == pps.ESTATE      # W before B
    ops = S.stage_ops(P, M, 0, 1, S.ZB1P)
    zb2 = _bk_stage(P, M, 0, kind=pps.ZB1P)
    _drive(zb2, ops[:6])                                    # F0 F1 F2 F3 B0 W0
    assert zb2.backward_weight_status(0) == pps.ESTATE     # W twice
    zb.close()
    zb2.close()

    # after a completed pass, a backward before the next pass's forward has nothing saved
    st = _bk_stage(P, M, 0)
    _drive(st, S.stage_ops(P, M, 0))
    assert st.backward_status(0, 0, None, None) == pps.ENOENT
    st.forward(0, 0, None, None)                            # starts the next pass
    assert st.oplog() == [tuple(o) for o in S.stage_ops(P, M, 0)[:1]]
    st.close()


def test_create_rejects_bad_descs():
    _lib_or_skip()
    with pytest.raises(pps.PpsError):
        _bk_stage(4, 6, 0, v=2)                 # interleaved needs M % P == 0
    with pytest.raises(pps.PpsError):
        _bk_stage(4, 8, 0, d=60)                # d % 8 != 0
    with pytest.raises(pps.PpsError):
        _bk_stage(4, 8, 0, block=pps.BLOCK_TOY_GELU, dtype=pps.DTYPE_BF16)
    with pytest.raises(pps.PpsError):
        pps.Stage(P=4, M=8, k=0, L=1, d=64, ffn=64, T=8)   # no weights without bookkeeping-only
    # bf16 GEMM operands are addressed with 32-bit byte offsets: dg|du [T, 2 ffn] must stay under 2 GiB
    _bk_stage(8, 16, 0, d=8192, ffn=28672, T=8192)          # the 80-layer slice: 0.94 GB, accepted
    with pytest.raises(pps.PpsError):
        _bk_stage(8, 16, 0, d=8192, ffn=28672, T=32768)     # 3.76 GB
    with pytest.raises(pps.PpsError):
        _bk_stage(8, 16, 0, d=16384, ffn=65536, T=8)        # interleaved gate/up copy 4.3 GB
    _bk_stage(8, 16, 0, d=8192, ffn=28672, T=32768, dtype=pps.DTYPE_FP32)   # the fp32 path has no such limit
    with pytest.raises(pps.PpsError):
        _bk_stage(8, 16, 0, d=16384, ffn=4096, T=100000)    # the [T, d] operands: 3.28 GB


def test_create_rejects_bad_schedule_params_before_allocating():
    # Called through the C ABI with (fake, never dereferenced) weight pointers
    # so the weight-table copy would run if the range checks did not come first.
    L = _lib_or_skip()
    fake = (ctypes.c_void_p * 64)(*([0x1000] * 64))
    base = dict(P=4, M=8, k=0, v=1, kind=pps.ONE_F_ONE_B, block_type=pps.BLOCK_SWIGLU, dtype=pps.DTYPE_BF16,
                L=2, d=64, ffn=128, T=16)
    bad = [dict(v=-1), dict(v=0), dict(P=0), dict(M=0), dict(L=0), dict(L=-3), dict(k=-1), dict(k=4),
           dict(kind=7), dict(kind=-1), dict(P=1 << 12, M=1 << 13), dict(v=1 << 11, L=1 << 10, P=1, M=1)]
    for over in bad:
        desc = pps.PpsStageDesc()
        for key, val in {**base, **over}.items():
            setattr(desc, key, val)
        desc.eps = 1e-6
        desc.weights = ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p))
        h = ctypes.c_void_p()
        assert L.pps_stage_create(ctypes.byref(desc), ctypes.byref(h)) == pps.EINVAL, over
        assert not h.value


def test_simulate_pipeline_matches_oracle():
    import random
    from oracle import schedule as S
    rng = random.Random(5)
    cases = [(2, 4, 1, pps.GPIPE), (4, 6, 1, pps.ONE_F_ONE_B), (8, 16, 1, pps.ONE_F_ONE_B), (8, 16, 2, pps.ONE_F_ONE_B),
             (4, 12, 3, pps.ONE_F_ONE_B), (4, 8, 1, pps.ZB1P), (4, 32, 1, pps.ZB2P), (5, 7, 1, pps.ZB1P)]
    for P, M, v, kind in cases:
        for _ in range(3):
            tf, tb, tw = rng.uniform(0.1, 3), rng.uniform(0.1, 3), rng.uniform(0.1, 3)
            mk, bubble = pps.simulate_pipeline(P, M, v, kind, tf, tb, tw)
            ok, obub = S.simulate_timed(S.all_stage_lists(P, M, v, kind), {S.F: tf, S.B: tb, S.W: tw}, v)
            assert mk == pytest.approx(ok, rel=1e-12), (P, M, v, kind)
            assert bubble == pytest.approx(obub, rel=1e-9, abs=1e-12), (P, M, v, kind)


def test_simulate_pipeline_errors():
    mk = ctypes.c_double(0)
    bu = ctypes.c_double(0)
    L = pps.lib()
    for args in [(4, 6, 1, pps.ONE_F_ONE_B, -1.0, 1.0, 0.0), (4, 6, 1, pps.ONE_F_ONE_B, float("nan"), 1.0, 0.0),
                 (4, 6, 2, pps.ONE_F_ONE_B, 1.0, 1.0, 0.0), (0, 6, 1, pps.ONE_F_ONE_B, 1.0, 1.0, 0.0),
                 (4, 6, 1, 9, 1.0, 1.0, 0.0), (4, 6, 1, pps.ONE_F_ONE_B, 1.0, float("inf"), 0.0)]:
        assert L.pps_simulate_pipeline(*args, ctypes.byref(mk), ctypes.byref(bu)) == pps.EINVAL, args
    assert L.pps_simulate_pipeline(4, 6, 1, pps.ONE_F_ONE_B, 1.0, 1.0, 0.0, None, ctypes.byref(bu)) == pps.EINVAL


def test_noalloc_create_rejects_before_touching_the_device():
    # The size check and the flag check come before any HIP call, so they run
    # without a GPU: a stage larger than the fixed array is PPS_ETOOBIG, and
    # PPS_FLAG_PROFILE (which creates HIP events) is PPS_EINVAL.
    L = _lib_or_skip()
    fake = (ctypes.c_void_p * 64)(*([0x1000] * 64))

    def desc(**over):
        d = pps.PpsStageDesc()
        base = dict(P=4, M=8, k=0, v=1, kind=pps.ONE_F_ONE_B, block_type=pps.BLOCK_SWIGLU, dtype=pps.DTYPE_BF16,
                    L=2, d=1024, ffn=2816, T=2048)
        for key, val in {**base, **over}.items():
            setattr(d, key, val)
        d.eps = 1e-6
        d.weights = ctypes.cast(fake, ctypes.POINTER(ctypes.c_void_p))
        return d

    h = ctypes.c_void_p()
    big = desc()   # 4 stash entries of ~55 MB alone exceed 64 MiB
    assert L.pps_stage_create_noalloc(ctypes.byref(big), ctypes.byref(h)) == pps.ETOOBIG
    assert not h.value
    prof = desc(d=64, ffn=64, T=8, flags=pps.FLAG_PROFILE, profile_capacity=16)
    assert L.pps_stage_create_noalloc(ctypes.byref(prof), ctypes.byref(h)) == pps.EINVAL
    assert not h.value
    assert "no-alloc" in pps.strerror(pps.ETOOBIG)
