"""Schedule oracle: per-stage op lists and a unit-cost dependency simulator.

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py`` for who may import it and
for the page legend used in the citations below).

Everything here is plain integer Python written for readability, not speed.
An *op* is a tuple ``(kind, mb, chunk)`` with kind F=0 (forward), B=1
(backward; input gradient, and also the weight gradient unless the
Zero-Bubble split is on) or W=2 (deferred weight gradient).

Readings of points the pages leave open:
  * warmup length: [1F1B §2.3/§3.2] warms up P-k forwards then alternates
    B,F; [Megatron-PP 三阶段] warms up P-k-1 forwards then alternates F,B.
    Both give the same op order (``megatron_1f1b`` proves it in tests).
  * the literal loop of [1F1B §5.2] (warmup P-k, then F *before* B) holds
    P-k+1 activations and is rejected (``pseudocode_literal_1f1b``).
  * steady-state backward takes the oldest un-backwarded micro-batch
    ([Megatron-PP 三阶段] pop(0); [Sched §03]).
  * M < P-k: the warmup is clamped to M.
  * GPipe runs its backwards in reverse order (D..A), as in [Sched §02].
  * interleaved order (v >= 2): Megatron-style groups of P micro-batches per
    chunk, warmup 2(P-k-1) + (v-1)P + 1 forwards; requires M % P == 0
    ([Sched §06] notes divisibility constraints).
  * ZB1P / ZB2P ([GPipe->ZB ZB1P 与 ZB2P]): the page sets the number of
    micro-batches a stage may hold with their backward unfinished to p (ZB1P)
    or 2p (ZB2P), p = P the number of stages, the same on every stage.  ZB1P
    keeps the 1F1B F/B order; ZB2P warms up with more forwards, as many as a
    stage can run before its first backward can start under equal F/B/W costs
    (2(P-k)-1), then alternates B and F.  A stage that cannot run its next F/B
    (dependency not done, or an F that would exceed the budget, counted until
    W) runs its oldest pending W.
  * stash slot = lowest free index, taken at F, freed at B (or at W when
    the backward is split).
"""

from __future__ import annotations

from collections import deque

F, B, W = 0, 1, 2
KIND_NAME = {F: "F", B: "B", W: "W"}

GPIPE, ONE_F_ONE_B, ZB1P, ZB2P = 0, 1, 2, 3


class ScheduleError(ValueError):
    pass


class Deadlock(RuntimeError):
    pass


def _check(P, M, k, v=1):
    if P < 1 or M < 1 or v < 1 or not (0 <= k < P):
        raise ScheduleError(f"invalid P={P} M={M} k={k} v={v}")


# ---------------------------------------------------------------------------
# O1: per-stage op lists
# ---------------------------------------------------------------------------

def gpipe(P, M, k):
    """All M forwards, then all backwards in reverse order.

    [Sched §02] (two-stage, four-micro-batch table: backward D..A) and
    [1F1B §4.5] (GPipe keeps M micro-batches in flight).
    """
    _check(P, M, k)
    return [(F, i, 0) for i in range(M)] + [(B, i, 0) for i in reversed(range(M))]


def one_f_one_b(P, M, k):
    """Synchronous 1F1B (PipeDream-Flush) op order of stage k.

    [1F1B §2.3]: stage k warms up with P-k forwards.  [1F1B §3.2]: then
    M-(P-k) steady (B, F) pairs, then P-k cooldown backwards, for M F + M B
    in total.  The backward always takes the oldest micro-batch that has not
    been backwarded ([Megatron-PP 三阶段], pop(0)).
    """
    _check(P, M, k)
    w = min(P - k, M)
    ops = [(F, i, 0) for i in range(w)]
    for j in range(M - w):
        ops.append((B, j, 0))
        ops.append((F, w + j, 0))
    ops += [(B, j, 0) for j in range(M - w, M)]
    return ops


def megatron_1f1b(P, M, k):
    """The same schedule written with Megatron's counts.

    [Megatron-PP 三阶段]: num_warmup = P - k - 1 forwards; each steady step
    does one forward then one backward (oldest first); cooldown backwards.
    """
    _check(P, M, k)
    nw = min(P - k - 1, M)
    ops = [(F, i, 0) for i in range(nw)]
    fi, bi = nw, 0
    for _ in range(M - nw):
        ops.append((F, fi, 0))
        fi += 1
        ops.append((B, bi, 0))
        bi += 1
    while bi < M:
        ops.append((B, bi, 0))
        bi += 1
    return ops


def pseudocode_literal_1f1b(P, M, k):
    """[1F1B §5.2] read literally: P-k warmup forwards, then each steady
    iteration does its forward *before* the backward of ``i - n_warmup``.

    Kept only so a test can show it holds P-k+1 activations at stage k, which
    contradicts the page's own bound of P in flight ([1F1B §4.1]); the
    executor never uses it.
    """
    _check(P, M, k)
    nw = min(P - k, M)
    ops = [(F, i, 0) for i in range(nw)]
    for i in range(nw, M):
        ops.append((F, i, 0))
        ops.append((B, i - nw, 0))
    for j in range(M - nw, M):
        ops.append((B, j, 0))
    return ops


def interleaved_sequences(P, M, v):
    """Forward and backward (chunk, mb) sequences of one device with v chunks.

    Micro-batches go in groups of P; within a group every chunk is visited in
    order (ascending for forward, descending for backward).  Virtual stage of
    chunk c on device k is c*P + k ([1F1B §6.1]; [lpnh] layout where GPU0
    holds layers 1-5 and 41-45).
    """
    groups = M // P
    fseq = [(c, i) for g in range(groups) for c in range(v) for i in range(g * P, g * P + P)]
    bseq = [(c, i) for g in range(groups) for c in reversed(range(v)) for i in range(g * P, g * P + P)]
    return fseq, bseq


def interleaved_warmup(P, M, k, v):
    """Forwards before the first backward on device k (reading of [1F1B §6.1])."""
    return min(2 * (P - k - 1) + (v - 1) * P + 1, M * v)


def interleaved(P, M, k, v, warmup=None):
    """Interleaved 1F1B op order of device k (v >= 2 virtual chunks)."""
    _check(P, M, k, v)
    if M % P != 0:
        raise ScheduleError("interleaved schedule needs M % P == 0")
    fseq, bseq = interleaved_sequences(P, M, v)
    nw = interleaved_warmup(P, M, k, v) if warmup is None else warmup
    ops = [(F, i, c) for (c, i) in fseq[:nw]]
    fi, bi = nw, 0
    while fi < len(fseq):
        c, i = bseq[bi]
        ops.append((B, i, c))
        bi += 1
        c, i = fseq[fi]
        ops.append((F, i, c))
        fi += 1
    while bi < len(bseq):
        c, i = bseq[bi]
        ops.append((B, i, c))
        bi += 1
    return ops


# ---------------------------------------------------------------------------
# O2: unit-cost dependency simulation of all P stages
# ---------------------------------------------------------------------------

def _deps(op, k, P, v):
    """Dependencies of ``op`` run on device k, as (kind, device, mb, chunk).

    A forward needs the previous virtual stage's forward of the same
    micro-batch; a backward needs its own forward and the next virtual
    stage's backward; a deferred W needs its own B ([Sched §08]: each task
    waits for the previous task on its device and for the results it needs
    from the neighbouring stages).
    """
    kind, i, c = op
    s = c * P + k
    out = []
    if kind == F:
        if s > 0:
            sp = s - 1
            out.append((F, sp % P, i, sp // P))
    elif kind == B:
        out.append((F, k, i, c))
        if s + 1 < v * P:
            sn = s + 1
            out.append((B, sn % P, i, sn // P))
    else:
        out.append((B, k, i, c))
    return out


def simulate(lists, v=1):
    """ASAP in-order execution of fixed per-device op lists with unit costs.

    Returns, per device, the start time of each op.  Raises ``Deadlock`` if
    no device can make progress while ops remain.
    """
    P = len(lists)
    end = {}
    starts = [[None] * len(ops) for ops in lists]
    ptr = [0] * P
    free_at = [0] * P
    remaining = sum(len(o) for o in lists)
    while remaining:
        progressed = False
        for k in range(P):
            while ptr[k] < len(lists[k]):
                op = lists[k][ptr[k]]
                deps = _deps(op, k, P, v)
                if any(d not in end for d in deps):
                    break
                t = max([free_at[k]] + [end[d] for d in deps])
                starts[k][ptr[k]] = t
                end[(op[0], k, op[1], op[2])] = t + 1
                free_at[k] = t + 1
                ptr[k] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise Deadlock(f"no device can progress; next ops {[lists[k][ptr[k]] if ptr[k] < len(lists[k]) else None for k in range(P)]}")
    return starts


def zb_warmup(P, M, k, budget_scale):
    """Forwards before the first backward of stage k under ZB1P/ZB2P.

    ZB1P keeps the 1F1B warmup, P-k.  ZB2P "does more forwards in warmup" so
    that the later backwards are ready sooner ([GPipe->ZB ZB1P 与 ZB2P]); the
    reading taken: a stage keeps running forwards until its first backward can
    start.  With unit costs stage k's first forward starts at t = k and the
    gradient of micro-batch 0 reaches it at t = 2P-1-k (P-1-k forwards on the
    way down, P-k backwards on the way back), leaving 2(P-k)-1 slots.
    """
    w = P - k if budget_scale == 1 else 2 * (P - k) - 1
    return min(w, M)


def zb_budget(P, budget_scale):
    """Micro-batches a stage may hold with W not yet done: p for ZB1P, 2p for
    ZB2P, the same on every stage ([GPipe->ZB ZB1P 与 ZB2P]: for a 4-stage
    pipeline the two limits are 4 and 8 micro-batches)."""
    return budget_scale * P


def zb_fb_order(P, M, k, budget_scale, warmup=None):
    """The F/B order of a ZB stage: the warmup forwards, then one B (oldest
    first) and one F alternating, then the remaining backwards."""
    w = zb_warmup(P, M, k, budget_scale) if warmup is None else min(warmup, M)
    ops = [(F, i, 0) for i in range(w)]
    for j in range(M - w):
        ops.append((B, j, 0))
        ops.append((F, w + j, 0))
    ops += [(B, j, 0) for j in range(M - w, M)]
    return ops


def simulate_zb(P, M, budget_scale=1, warmups=None):
    """Zero-Bubble greedy placement of deferred W ops ([GPipe->ZB ZB1P 与 ZB2P]).

    Each stage keeps its F/B order (``zb_fb_order``).  At every integer time t
    a free stage (1) runs its next F/B if that op's dependencies ended at or
    before t and, for an F, its live count stays below ``zb_budget``; (2)
    otherwise runs its oldest pending W; (3) otherwise idles.  ``live`` counts
    entries whose F has started and whose W has not yet run.
    ``budget_scale`` 1 is ZB1P, 2 is ZB2P.  ``warmups`` (per stage) replaces
    the warmup counts, for tests that show the ZB2P warmup is tight.

    Returns (lists, starts): the per-stage op lists with W ops placed, and
    their start times.
    """
    base = [zb_fb_order(P, M, k, budget_scale, None if warmups is None else warmups[k]) for k in range(P)]
    budget = zb_budget(P, budget_scale)
    ptr = [0] * P
    pending = [deque() for _ in range(P)]
    live = [0] * P
    free_at = [0] * P
    end = {}
    lists = [[] for _ in range(P)]
    starts = [[] for _ in range(P)]
    done_w = [0] * P
    t = 0
    limit = 4 * (3 * M + 2 * P) + 16
    while any(done_w[k] < M for k in range(P)):
        if t > limit:
            raise Deadlock("zero-bubble simulation did not finish")
        for k in range(P):
            if free_at[k] > t:
                continue
            ran = None
            if ptr[k] < len(base[k]):
                op = base[k][ptr[k]]
                deps = _deps(op, k, P, 1)
                ok = all(d in end and end[d] <= t for d in deps)
                if ok and op[0] == F and live[k] >= budget:
                    ok = False
                if ok:
                    ran = op
                    ptr[k] += 1
                    if op[0] == F:
                        live[k] += 1
                    else:
                        pending[k].append(op[1])
            if ran is None and pending[k]:
                i = pending[k].popleft()
                ran = (W, i, 0)
                live[k] -= 1
                done_w[k] += 1
            if ran is not None:
                lists[k].append(ran)
                starts[k].append(t)
                end[(ran[0], k, ran[1], ran[2])] = t + 1
                free_at[k] = t + 1
        t += 1
    return lists, starts


def idle_in_span(ops, st):
    """Idle unit slots between a stage's first op start and its last op end:
    the compute bubble the Zero-Bubble schedules fill ([GPipe->ZB ZB1P 与
    ZB2P]; the slots before a stage's first op and after its last are the
    pipeline's fill and drain)."""
    if not st:
        return 0
    return st[-1] + 1 - st[0] - len(ops)


# ---------------------------------------------------------------------------
# Stash bookkeeping of one stage
# ---------------------------------------------------------------------------

def assign_slots(ops, split):
    """Slot and live count after each op, in op-list order.

    Slot = lowest free index, taken at F; released at B, or at W when the
    backward is split (the entry's data must survive until W: [GPipe->ZB
    Zero Bubble], X and G stay resident until W).  Live = entries whose F is
    done and that have not been released ([Sched §03]: forward finished,
    backward not yet released).
    """
    used = set()
    where = {}
    slots, live_after = [], []
    for kind, i, c in ops:
        if kind == F:
            s = 0
            while s in used:
                s += 1
            used.add(s)
            where[(i, c)] = s
            slots.append(s)
        else:
            s = where[(i, c)]
            slots.append(s)
            if (kind == B and not split) or kind == W:
                used.discard(s)
        live_after.append(len(used))
    return slots, live_after


def stage_ops(P, M, k, v=1, kind=ONE_F_ONE_B):
    """Full op records of stage k: (kind, mb, chunk, slot, live_after, t_start).

    The same quantities the library's ``pps_make_schedule`` must produce.
    """
    _check(P, M, k, v)
    if kind in (ZB1P, ZB2P):
        if v != 1:
            raise ScheduleError("zero-bubble split is defined for v == 1 only")
        lists, starts = simulate_zb(P, M, 1 if kind == ZB1P else 2)
        split = True
    else:
        if kind == GPIPE:
            if v != 1:
                raise ScheduleError("GPipe order is defined for v == 1 only")
            lists = [gpipe(P, M, s) for s in range(P)]
        elif v == 1:
            lists = [one_f_one_b(P, M, s) for s in range(P)]
        else:
            lists = [interleaved(P, M, s, v) for s in range(P)]
        starts = simulate(lists, v)
        split = False
    ops = lists[k]
    slots, live = assign_slots(ops, split)
    return [(o[0], o[1], o[2], slots[j], live[j], starts[k][j]) for j, o in enumerate(ops)]


def pipeline_tables(P, M, v=1, kind=ONE_F_ONE_B):
    """Per-stage op lists and start times for every stage."""
    if kind in (ZB1P, ZB2P):
        return simulate_zb(P, M, 1 if kind == ZB1P else 2)
    if kind == GPIPE:
        lists = [gpipe(P, M, s) for s in range(P)]
    elif v == 1:
        lists = [one_f_one_b(P, M, s) for s in range(P)]
    else:
        lists = [interleaved(P, M, s, v) for s in range(P)]
    return lists, simulate(lists, v)


def timeline(lists, starts):
    """Render per-stage rows as {t: 'F3'} dicts (for comparing with tables)."""
    rows = []
    for ops, st in zip(lists, starts):
        row = {}
        for (kind, i, c), t in zip(ops, st):
            row[t] = KIND_NAME[kind] + str(i) + (f"c{c}" if c else "")
        rows.append(row)
    return rows


def simulate_timed(lists, durations, v=1):
    """The same in-order ASAP execution with per-op durations: an op starts
    when its device's previous op has ended and its dependencies have ended
    ([Sched §08]).  ``durations`` maps op kind (F, B, W) to its duration.

    Returns (makespan, bubble) with bubble = 1 - busy / (P * makespan), the
    idle share of the P device timelines ([1F1B §4.3], [Sched §04]).
    """
    P = len(lists)
    end = {}
    ptr = [0] * P
    free_at = [0.0] * P
    busy = 0.0
    makespan = 0.0
    remaining = sum(len(o) for o in lists)
    while remaining:
        progressed = False
        for k in range(P):
            while ptr[k] < len(lists[k]):
                op = lists[k][ptr[k]]
                deps = _deps(op, k, P, v)
                if any(d not in end for d in deps):
                    break
                t = max([free_at[k]] + [end[d] for d in deps])
                dur = float(durations[op[0]])
                end[(op[0], k, op[1], op[2])] = t + dur
                free_at[k] = t + dur
                busy += dur
                makespan = max(makespan, t + dur)
                ptr[k] += 1
                remaining -= 1
                progressed = True
        if not progressed:
            raise Deadlock("no device can progress")
    return makespan, (1.0 - busy / (P * makespan) if makespan > 0 else 0.0)


def all_stage_lists(P, M, v=1, kind=ONE_F_ONE_B):
    """Op lists (op, mb, chunk) of all P devices as the schedule runs them
    (ZB kinds: with their unit-cost W placement)."""
    if kind in (ZB1P, ZB2P):
        return simulate_zb(P, M, 1 if kind == ZB1P else 2)[0]
    if kind == GPIPE:
        return [gpipe(P, M, k) for k in range(P)]
    if v > 1:
        return [interleaved(P, M, k, v) for k in range(P)]
    return [one_f_one_b(P, M, k) for k in range(P)]


def total_time(starts):
    return max((t + 1 for st in starts for t in st), default=0)


def busy_fraction(lists, starts):
    """Average fraction of the window each stage spends computing."""
    T = total_time(starts)
    return sum(len(o) for o in lists) / (len(lists) * T)


def inflight_trace(ops, split=False):
    """Live activation count after each op of one stage (idle slots removed)."""
    return assign_slots(ops, split)[1]


def peak_inflight(ops, split=False):
    return max(inflight_trace(ops, split), default=0)


def closed_form_bubble(P, M, v=1):
    """Bubble / total window: (P-1)/(vM+P-1) ([1F1B §4.3], [1F1B §6.1])."""
    return (P - 1) / (v * M + P - 1)
