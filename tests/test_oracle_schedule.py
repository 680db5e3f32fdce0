"""Pins of the schedule oracle against the pages' worked tables, counts and
closed forms.  CPU only."""

from fractions import Fraction

import pytest

from oracle import schedule as S
from tests.conftest import read_golden


def _parse_rows(lines):
    rows = {}
    for ln in lines:
        if ":" not in ln:
            continue
        key, val = ln.split(":", 1)
        rows[key.strip()] = val.split()
    return rows


def _sim_rows(P, M, kind, v=1):
    lists, starts = S.pipeline_tables(P, M, v, kind)
    tl = S.timeline(lists, starts)
    width = S.total_time(starts)
    return [[r.get(t, ".") for t in range(width)] for r in tl], lists, starts


# --- [Sched §02/§03]: the two-stage, four-micro-batch tables, every cell ----

@pytest.mark.parametrize("fname,kind", [("sched_gpipe_p2_m4.txt", S.GPIPE),
                                        ("sched_1f1b_p2_m4.txt", S.ONE_F_ONE_B)])
def test_p2_m4_tables_every_cell(fname, kind):
    page = _parse_rows(read_golden(fname))
    sim, lists, starts = _sim_rows(2, 4, kind)
    assert sim[0] == page["stage0"]
    assert sim[1] == page["stage1"]
    assert S.total_time(starts) == int(page["window"][0])
    assert S.peak_inflight(lists[0]) == int(page["stage0_peak_inflight"][0])
    if "busy_percent" in page:
        assert Fraction(sum(len(o) for o in lists), 2 * S.total_time(starts)) == Fraction(int(page["busy_percent"][0]), 100)


def test_p2_m4_1f1b_stage1_holds_one():
    lists, _ = S.pipeline_tables(2, 4, 1, S.ONE_F_ONE_B)
    assert S.peak_inflight(lists[1]) == 1


# --- [1F1B §3.1, §4.1, §4.3]: P=4, M=6 --------------------------------------

def test_p4_m6_stage0_row_and_orders():
    page = _parse_rows(read_golden("1f1b_p4_m6_table.txt"))
    sim, lists, starts = _sim_rows(4, 6, S.ONE_F_ONE_B)
    # stage 0 cell for cell on t = 0..11
    assert sim[0][:12] == page["S0"][:12]
    # idle at t = 4..6 (P-1 = 3 slots waiting for B0)
    assert sim[0][4:7] == [".", ".", "."]
    # op order of S0 and S3 (idles dropped)
    for s in ("S0", "S3"):
        k = int(s[1])
        order = [S.KIND_NAME[o[0]] + str(o[1]) for o in lists[k]]
        assert order == [c for c in page[s] if c != "."]
    # dependency-true window is 2(M+P-1) = 18 ([1F1B §4.3])
    assert S.total_time(starts) == 18


def test_p4_m6_stage0_inflight_trace():
    rows = [ln.split() for ln in read_golden("1f1b_stage0_inflight.txt")]
    page_counts = [int(r[2]) for r in rows if r[1] != "wait"]
    page_ops = [r[1] for r in rows if r[1] != "wait"]
    ops = S.one_f_one_b(4, 6, 0)
    assert [S.KIND_NAME[o[0]] + str(o[1]) for o in ops] == page_ops
    assert S.inflight_trace(ops) == page_counts
    assert max(page_counts) == 4  # = P


# --- [1F1B §3.2]: three-phase counts, over a grid ---------------------------

@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 8, 13])
def test_three_phase_counts(P):
    for M in range(1, 3 * P + 3):
        for k in range(P):
            ops = S.one_f_one_b(P, M, k)
            w = min(P - k, M)
            kinds = [o[0] for o in ops]
            assert kinds.count(S.F) == M and kinds.count(S.B) == M
            first_b = kinds.index(S.B)
            assert first_b == w                                  # warmup P-k
            tail = kinds[first_b:]
            steady = tail[: 2 * (M - w)]
            assert steady == [S.B, S.F] * (M - w)                # steady pairs
            assert tail[2 * (M - w):] == [S.B] * w               # cooldown P-k
            assert [o[1] for o in ops if o[0] == S.B] == list(range(M))  # oldest first
            assert S.peak_inflight(ops) == w                     # in-flight bound


# --- [Megatron-PP 三阶段]: P-k-1 warmup convention ---------------------------

def test_megatron_warmup_values_and_equivalence():
    rows = _parse_rows(read_golden("megatron_warmup_pp4.txt"))
    P = int(rows["P"][0])
    want = [int(x) for x in rows["warmup"]]
    got = []
    for k in range(P):
        ops = S.megatron_1f1b(P, 8, k)
        # forwards issued before the first steady forward (one F before the first B)
        got.append([o[0] for o in ops].index(S.B) - 1)
    assert got == want
    for P in range(1, 10):
        for M in range(1, 25):
            for k in range(P):
                assert S.megatron_1f1b(P, M, k) == S.one_f_one_b(P, M, k)


def test_literal_pseudocode_exceeds_bound():
    # The [1F1B §5.2] loop read literally (forward before backward in the
    # steady loop) holds P-k+1 micro-batches: 5 at stage 0 for P=4.
    assert S.peak_inflight(S.pseudocode_literal_1f1b(4, 6, 0)) == 5
    for P in range(2, 9):
        for k in range(P):
            assert S.peak_inflight(S.pseudocode_literal_1f1b(P, 3 * P, k)) == P - k + 1


# --- closed forms: [1F1B §4.3], [Sched §04], [lpnh] -------------------------

@pytest.mark.parametrize("kind", [S.GPIPE, S.ONE_F_ONE_B])
def test_window_busy_bubble_closed_forms(kind):
    for P in range(1, 9):
        for M in range(1, 3 * P + 2):
            lists, starts = S.pipeline_tables(P, M, 1, kind)
            T = S.total_time(starts)
            assert T == 2 * (M + P - 1)
            assert Fraction(sum(len(o) for o in lists), P * T) == Fraction(M, M + P - 1)
            assert Fraction(2 * (P - 1), T) == Fraction(P - 1, M + P - 1)


def test_p8_m16_bubble_percent():
    rows = _parse_rows(read_golden("bubble_values.txt"))
    lists, starts = S.pipeline_tables(8, 16, 1, S.GPIPE)
    bubble = 1 - S.busy_fraction(lists, starts)
    assert round(100 * bubble, 1) == float(rows["P8_M16_bubble_percent"][0])
    lists, starts = S.pipeline_tables(8, 16, 1, S.ONE_F_ONE_B)
    assert abs((1 - S.busy_fraction(lists, starts)) - bubble) < 1e-15  # same as GPipe


def test_stage0_memory_gpipe_vs_1f1b():
    # [1F1B §4.5]: stage 0 holds M (GPipe) vs P (1F1B) micro-batches.
    for P in range(1, 9):
        for M in range(P, 4 * P):
            assert S.peak_inflight(S.gpipe(P, M, 0)) == M
            assert S.peak_inflight(S.one_f_one_b(P, M, 0)) == P


# --- simulator invariants ([Sched §08] checker) ------------------------------

@pytest.mark.parametrize("kind,v", [(S.GPIPE, 1), (S.ONE_F_ONE_B, 1), (S.ONE_F_ONE_B, 2),
                                    (S.ONE_F_ONE_B, 3), (S.ZB1P, 1), (S.ZB2P, 1)])
def test_simulator_invariants(kind, v):
    for P in (1, 2, 3, 4, 6):
        for M in (P, 2 * P, 3 * P):
            lists, starts = S.pipeline_tables(P, M, v, kind)
            end = {}
            for k in range(P):
                st = starts[k]
                assert all(b >= a + 1 for a, b in zip(st, st[1:]))  # no overlap, in order
                for op, t in zip(lists[k], st):
                    end[(op[0], k, op[1], op[2])] = t + 1
            for k in range(P):
                for op, t in zip(lists[k], starts[k]):
                    for dep in S._deps(op, k, P, v):
                        assert end[dep] <= t
                n_f = sum(1 for o in lists[k] if o[0] == S.F)
                n_b = sum(1 for o in lists[k] if o[0] == S.B)
                assert n_f == n_b == M * v


# --- interleaved (v >= 2): [1F1B §6.1], [lpnh] -------------------------------

@pytest.mark.parametrize("v", [2, 3, 4])
def test_interleaved_bubble_closed_form(v):
    for P in (2, 3, 4, 8):
        for M in (P, 2 * P, 3 * P):
            lists, starts = S.pipeline_tables(P, M, v, S.ONE_F_ONE_B)
            T = S.total_time(starts)
            assert T == 2 * (v * M + P - 1)
            assert Fraction(2 * (P - 1), T) == Fraction(P - 1, v * M + P - 1)


def test_interleaved_p8_m16_values():
    lists, starts = S.pipeline_tables(8, 16, 2, S.ONE_F_ONE_B)
    assert S.total_time(starts) == 78
    assert Fraction(14, 78) == Fraction(7, 39)
    # device 0 keeps the warmup's forwards alive: 23 chunk entries
    assert S.peak_inflight(lists[0]) == 23
    assert S.peak_inflight(S.one_f_one_b(8, 16, 0)) == 8


def test_interleaved_warmup_tightness():
    # Under unit costs the last device's warmup is tight (one fewer forward
    # deadlocks) and three fewer forwards deadlock on every device; on the
    # other devices one fewer forward keeps the window (Megatron's count
    # carries one forward of slack there), two fewer lengthen it.
    for P, M, v in [(2, 4, 2), (4, 8, 2), (4, 8, 3), (8, 16, 2)]:
        base = S.total_time(S.simulate([S.interleaved(P, M, s, v) for s in range(P)], v))
        for k in range(P):
            nw = S.interleaved_warmup(P, M, k, v)
            outcome = []
            for cut in (1, 2, 3):
                lists = [S.interleaved(P, M, s, v) for s in range(P)]
                lists[k] = S.interleaved(P, M, k, v, warmup=nw - cut)
                try:
                    outcome.append(S.total_time(S.simulate(lists, v)))
                except S.Deadlock:
                    outcome.append(None)
            assert outcome[2] is None
            if k == P - 1:
                assert outcome[0] is None
            else:
                assert outcome[0] == base and outcome[1] > base


def test_interleaved_layout_matches_80_layer_example():
    # [lpnh]: 80 layers, 8 stages, 5 layers per virtual chunk: GPU0 holds
    # layers 1-5 and 41-45.  Virtual stage of chunk c on device k is c*P + k.
    P, v, L = 8, 2, 5
    k = 0
    layers = [list(range((c * P + k) * L + 1, (c * P + k) * L + L + 1)) for c in range(v)]
    assert layers == [[1, 2, 3, 4, 5], [41, 42, 43, 44, 45]]


def test_interleaved_needs_divisible_m():
    with pytest.raises(S.ScheduleError):
        S.interleaved(4, 6, 0, 2)


# --- ZB1P / ZB2P: [GPipe->ZB ZB1P 与 ZB2P] -----------------------------------

def _zb_idle(lists, starts):
    return [S.idle_in_span(o, t) for o, t in zip(lists, starts)]


@pytest.mark.parametrize("scale", [1, 2])
def test_zb_invariants(scale):
    for P in (1, 2, 3, 4, 8):
        for M in (1, P, 2 * P, 8 * P):
            lists, starts = S.simulate_zb(P, M, scale)
            for k in range(P):
                ops = lists[k]
                kinds = [o[0] for o in ops]
                assert kinds.count(S.F) == kinds.count(S.B) == kinds.count(S.W) == M
                fb = [o for o in ops if o[0] != S.W]
                # F/B in the stage's ZB order; ZB1P keeps the 1F1B order
                assert fb == S.zb_fb_order(P, M, k, scale)
                if scale == 1:
                    assert fb == S.one_f_one_b(P, M, k)
                # backwards oldest first; every W after its own B, oldest first
                assert [o[1] for o in ops if o[0] == S.B] == list(range(M))
                seen_b = []
                for o in ops:
                    if o[0] == S.B:
                        seen_b.append(o[1])
                    elif o[0] == S.W:
                        assert o[1] in seen_b
                assert [o[1] for o in ops if o[0] == S.W] == list(range(M))
                # the page's limit on micro-batches whose backward (W) is not
                # done: p for ZB1P, 2p for ZB2P, counted until W
                assert S.peak_inflight(ops, split=True) <= min(scale * P, M)


def test_zb_limits_four_stage_example():
    # The page's example: a 4-stage pipeline may hold 4 (ZB1P) or 8 (ZB2P)
    # micro-batches with their backward unfinished; with enough micro-batches
    # the greedy placement defers W until it reaches that limit.
    for scale, limit in ((1, 4), (2, 8)):
        lists, _ = S.simulate_zb(4, 32, scale)
        assert [S.peak_inflight(o, split=True) for o in lists] == [limit] * 4


def test_zb2p_runs_more_warmup_forwards():
    # ZB2P does more forwards in warmup than the 1F1B order ZB1P keeps.
    for P in (2, 3, 4, 8):
        for M in (2 * P, 4 * P):
            for scale in (1, 2):
                lists, _ = S.simulate_zb(P, M, scale)
                for k in range(P):
                    fb = [o[0] for o in lists[k] if o[0] != S.W]
                    nf = fb.index(S.B)
                    if scale == 1:
                        assert nf == P - k
                    else:
                        assert nf == 2 * (P - k) - 1
                        assert nf > P - k or k == P - 1


def test_zb_window_lower_bound():
    # Unit costs: every stage runs 3M ops and stage P-1 cannot start before
    # t = P-1, so no schedule of the split backward is shorter than 3M+P-1.
    # With M >= P both ZB placements reach the bound; plain 1F1B with the
    # whole backward (2 units) takes 3M + 3(P-1).
    for P in (1, 2, 3, 4, 8):
        for M in (P, 2 * P, 4 * P, 32):
            for scale in (1, 2):
                lists, starts = S.simulate_zb(P, M, scale)
                assert S.total_time(starts) == 3 * M + P - 1
            mk, _ = S.simulate_timed(S.all_stage_lists(P, M, 1, S.ONE_F_ONE_B), {S.F: 1, S.B: 2, S.W: 0})
            assert mk == 3 * M + 3 * (P - 1)


def test_zb2p_removes_the_bubble_zb1p_keeps_some():
    # [GPipe->ZB ZB1P 与 ZB2P]: under equal F/B/W costs and enough
    # micro-batches ZB2P leaves no idle slot between a stage's first and last
    # op; ZB1P's budget limits how far W can move, so some bubble remains.
    for P in (2, 3, 4, 5, 8):
        for M in range(2 * P - 1, 4 * P + 1):
            l2, s2 = S.simulate_zb(P, M, 2)
            assert _zb_idle(l2, s2) == [0] * P, (P, M)
            l1, s1 = S.simulate_zb(P, M, 1)
            idle1 = _zb_idle(l1, s1)
            assert idle1[0] > 0 and sum(idle1) > 0, (P, M)
            # stage k starts at k and runs without a gap: it ends at 3M + k
            for k in range(P):
                assert s2[k][0] == k and s2[k][-1] + 1 == 3 * M + k
    # the headline ZB shapes
    l1, s1 = S.simulate_zb(4, 32, 1)
    l2, s2 = S.simulate_zb(4, 32, 2)
    assert sum(_zb_idle(l2, s2)) == 0 < sum(_zb_idle(l1, s1))


def test_zb2p_warmup_is_tight():
    # 2(P-k)-1 is the only warmup that removes the bubble on stages k >= 1:
    # one forward fewer leaves stage k waiting for its first backward, one
    # more delays that backward for the stages upstream.
    for P in (3, 4, 8):
        for M in (2 * P, 4 * P):
            base = [2 * (P - k) - 1 for k in range(P)]
            for k in range(P - 1):
                w = list(base)
                w[k] -= 1
                lists, starts = S.simulate_zb(P, M, 2, warmups=w)
                assert _zb_idle(lists, starts)[k] > 0
                if k >= 1:
                    w = list(base)
                    w[k] += 1
                    lists, starts = S.simulate_zb(P, M, 2, warmups=w)
                    assert sum(_zb_idle(lists, starts)) > 0


# --- slots ([1F1B §5.2] activations dict; lowest free index) -----------------

def test_slots_1f1b_and_gpipe():
    for P in range(1, 9):
        for M in range(1, 3 * P):
            for k in range(P):
                rec = S.stage_ops(P, M, k, 1, S.ONE_F_ONE_B)
                w = min(P - k, M)
                for kind, i, c, slot, live, t in rec:
                    assert slot == i % w
                rec = S.stage_ops(P, M, k, 1, S.GPIPE)
                for kind, i, c, slot, live, t in rec:
                    assert slot == i


def test_stage_ops_errors():
    with pytest.raises(S.ScheduleError):
        S.stage_ops(0, 4, 0)
    with pytest.raises(S.ScheduleError):
        S.stage_ops(4, 4, 4)
    with pytest.raises(S.ScheduleError):
        S.stage_ops(4, 6, 0, 2)
    with pytest.raises(S.ScheduleError):
        S.stage_ops(4, 8, 0, 2, S.ZB1P)


# ---- timed simulation (measured-cost prediction of the P-stage timeline) ----

@pytest.mark.parametrize("kind", [S.GPIPE, S.ONE_F_ONE_B])
@pytest.mark.parametrize("P,M", [(2, 4), (4, 6), (8, 16), (4, 32)])
@pytest.mark.parametrize("tf,tb", [(1.0, 1.0), (1.0, 2.0), (0.7, 1.9), (2.5, 1.0)])
def test_timed_closed_form(kind, P, M, tf, tb):
    # [1F1B §4.3], [Sched §04]: the bubble is (P-1) of M+P-1 slots of t_f + t_b
    # for both GPipe and 1F1B; [lpnh] quotes t_b ~ 2 t_f.  Transfers take no time.
    mk, bubble = S.simulate_timed(S.all_stage_lists(P, M, 1, kind), {S.F: tf, S.B: tb, S.W: 0.0})
    assert mk == pytest.approx((M + P - 1) * (tf + tb), rel=1e-12)
    assert bubble == pytest.approx((P - 1) / (M + P - 1), rel=1e-9)


@pytest.mark.parametrize("P,M,v,kind", [(4, 6, 1, S.ONE_F_ONE_B), (4, 8, 2, S.ONE_F_ONE_B), (8, 16, 2, S.ONE_F_ONE_B),
                                        (4, 8, 1, S.ZB1P), (4, 32, 1, S.ZB2P), (3, 5, 1, S.GPIPE)])
def test_timed_unit_costs_match_unit_simulator(P, M, v, kind):
    lists = S.all_stage_lists(P, M, v, kind)
    starts = S.simulate(lists, v)
    mk, bubble = S.simulate_timed(lists, {S.F: 1, S.B: 1, S.W: 1}, v)
    assert mk == S.total_time(starts)
    assert bubble == pytest.approx(1.0 - S.busy_fraction(lists, starts), abs=1e-12)


@pytest.mark.parametrize("P,M,v", [(4, 8, 2), (8, 16, 2), (4, 12, 3)])
def test_timed_interleaved_bubble(P, M, v):
    # [1F1B §6.1]: with v chunks per device the bubble is (P-1)/(vM+P-1)
    _, bubble = S.simulate_timed(S.all_stage_lists(P, M, v, S.ONE_F_ONE_B), {S.F: 1, S.B: 1, S.W: 0}, v)
    assert bubble == pytest.approx((P - 1) / (v * M + P - 1), rel=1e-12)


@pytest.mark.parametrize("P,M", [(4, 8), (4, 32), (8, 16)])
def test_timed_zero_bubble_not_longer(P, M):
    # splitting B into dX then W can only fill gaps: never longer than 1F1B
    # running the whole backward (dX + W) as one op ([GPipe->ZB Zero Bubble])
    tf, tbx, tw = 1.0, 1.0, 1.0
    mk_zb, _ = S.simulate_timed(S.all_stage_lists(P, M, 1, S.ZB1P), {S.F: tf, S.B: tbx, S.W: tw})
    mk_1f1b, _ = S.simulate_timed(S.all_stage_lists(P, M, 1, S.ONE_F_ONE_B), {S.F: tf, S.B: tbx + tw, S.W: 0.0})
    assert mk_zb <= mk_1f1b + 1e-12
