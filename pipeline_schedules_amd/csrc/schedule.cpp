// Host-only schedule generation for one pipeline stage (pure integer code).
//
// Page legend: [1F1B] "2. 1F1B"; [GPipe->ZB] "流水线并行：从 GPipe 到 1F1B 与
// Zero Bubble"; [Sched] "流水线调度：GPipe、1F1B、交错与计算通信重叠";
// [Megatron-PP] "Megatron-LM 分布式训练（三）：流水线并行 PP 与 1F1B 调度".
//
// Every device's op list is produced by a closed rule (GPipe, 1F1B,
// interleaved 1F1B) or by a greedy unit-cost placement of the deferred W
// ops (ZB1P / ZB2P).  Start times come from executing all P devices' lists
// with unit costs: an op starts when its device is free and its
// dependencies have ended ([Sched §08]: a task waits for the previous task
// on its device and for the upstream/downstream results it needs).

#include "schedule_internal.h"

#include <algorithm>
#include <cmath>
#include <cstring>
#include <deque>

namespace pps {

namespace {

// ---- closed-form op lists --------------------------------------------------

// `warm` forwards, then (B oldest, F next) pairs, then the remaining
// backwards.
void list_warm_alternate(int M, int warm, std::vector<Op3>& out) {
    out.clear();
    warm = std::min(warm, M);
    int next_f = 0, next_b = 0;
    while (next_f < warm) out.push_back({OP_F, next_f++, 0});
    while (next_f < M) {
        out.push_back({OP_B, next_b++, 0});
        out.push_back({OP_F, next_f++, 0});
    }
    while (next_b < M) out.push_back({OP_B, next_b++, 0});
}

// [1F1B §2.3/§3.2]: P-k warmup forwards, then alternate.
void list_1f1b(int P, int M, int k, std::vector<Op3>& out) { list_warm_alternate(M, P - k, out); }

// [Sched §02]: every forward, then the backwards from the last micro-batch down.
void list_gpipe(int M, std::vector<Op3>& out) {
    out.clear();
    for (int i = 0; i < M; ++i) out.push_back({OP_F, i, 0});
    for (int i = M - 1; i >= 0; --i) out.push_back({OP_B, i, 0});
}

// Interleaved (v chunks per device, [1F1B §6.1]).  Micro-batches advance in
// groups of P; inside a group the forward visits chunks 0..v-1 and the
// backward v-1..0.  Forwards before the first backward:
// min(2(P-k-1) + (v-1)P + 1, M v); afterwards one B then one F.
void list_interleaved(int P, int M, int k, int v, std::vector<Op3>& out) {
    out.clear();
    const int total = M * v;
    auto fwd_at = [&](int n, int& mb, int& c) {
        int group = n / (P * v), rem = n % (P * v);
        c = rem / P;
        mb = group * P + rem % P;
    };
    auto bwd_at = [&](int n, int& mb, int& c) {
        int group = n / (P * v), rem = n % (P * v);
        c = v - 1 - rem / P;
        mb = group * P + rem % P;
    };
    const int warm = std::min(2 * (P - k - 1) + (v - 1) * P + 1, total);
    int nf = 0, nb = 0, mb, c;
    while (nf < warm) { fwd_at(nf++, mb, c); out.push_back({OP_F, mb, c}); }
    while (nf < total) {
        bwd_at(nb++, mb, c); out.push_back({OP_B, mb, c});
        fwd_at(nf++, mb, c); out.push_back({OP_F, mb, c});
    }
    while (nb < total) { bwd_at(nb++, mb, c); out.push_back({OP_B, mb, c}); }
}

// ---- unit-cost execution ----------------------------------------------------

// End time of every F and B op, per virtual stage and micro-batch; T is int
// for the unit-cost placement and double for timed simulation.  -1 = not yet
// ended.
template <typename T>
struct EndTimesT {
    int P, M, v;
    std::vector<T> f, b;
    EndTimesT(int P_, int M_, int v_) : P(P_), M(M_), v(v_),
        f((size_t)P_ * v_ * M_, T(-1)), b((size_t)P_ * v_ * M_, T(-1)) {}
    T& F(int vs, int mb) { return f[(size_t)vs * M + mb]; }
    T& B(int vs, int mb) { return b[(size_t)vs * M + mb]; }
};
using EndTimes = EndTimesT<int>;

// Earliest start of `op` on device `dev` given the ended ops, or -1 if a
// dependency has not ended.  Forward needs the previous virtual stage's
// forward; backward needs its own forward and the next virtual stage's
// backward; W needs its own backward.
template <typename T>
T ready_time(EndTimesT<T>& e, const Op3& op, int dev) {
    const int vs = op.chunk * e.P + dev;
    const int last = e.P * e.v - 1;
    if (op.kind == OP_F) return vs > 0 ? e.F(vs - 1, op.mb) : T(0);
    if (op.kind == OP_W) return e.B(vs, op.mb);
    const T own = e.F(vs, op.mb);
    if (own < 0 || vs == last) return own;
    const T down = e.B(vs + 1, op.mb);
    return down < 0 ? T(-1) : std::max(own, down);
}

template <typename T>
void mark_end(EndTimesT<T>& e, const Op3& op, int dev, T end) {
    const int vs = op.chunk * e.P + dev;
    if (op.kind == OP_F) e.F(vs, op.mb) = end;
    else if (op.kind == OP_B) e.B(vs, op.mb) = end;
}

// ASAP in-order execution of fixed lists.  Returns false on deadlock.
bool run_fixed(const std::vector<std::vector<Op3>>& lists, int P, int M, int v,
               std::vector<std::vector<int>>& start) {
    EndTimes e(P, M, v);
    std::vector<size_t> pos(P, 0);
    std::vector<int> free_at(P, 0);
    start.assign(P, {});
    size_t left = 0;
    for (int d = 0; d < P; ++d) { left += lists[d].size(); start[d].reserve(lists[d].size()); }
    while (left) {
        bool moved = false;
        for (int d = 0; d < P; ++d) {
            while (pos[d] < lists[d].size()) {
                const Op3& op = lists[d][pos[d]];
                int r = ready_time(e, op, d);
                if (r < 0) break;
                int t = std::max(r, free_at[d]);
                start[d].push_back(t);
                mark_end(e, op, d, t + 1);
                free_at[d] = t + 1;
                ++pos[d];
                --left;
                moved = true;
            }
        }
        if (!moved) return false;
    }
    return true;
}

// The same in-order ASAP execution with per-op durations (F, B, W).  Returns
// false on deadlock.
bool run_timed(const std::vector<std::vector<Op3>>& lists, int P, int M, int v, const double (&dur)[3],
               double& makespan, double& busy) {
    EndTimesT<double> e(P, M, v);
    std::vector<size_t> pos(P, 0);
    std::vector<double> free_at(P, 0.0);
    size_t left = 0;
    for (int d = 0; d < P; ++d) left += lists[d].size();
    makespan = 0.0;
    busy = 0.0;
    while (left) {
        bool moved = false;
        for (int d = 0; d < P; ++d) {
            while (pos[d] < lists[d].size()) {
                const Op3& op = lists[d][pos[d]];
                const double r = ready_time(e, op, d);
                if (r < 0) break;
                const double t = std::max(r, free_at[d]);
                const double end = t + dur[op.kind];
                mark_end(e, op, d, end);
                free_at[d] = end;
                busy += dur[op.kind];
                makespan = std::max(makespan, end);
                ++pos[d];
                --left;
                moved = true;
            }
        }
        if (!moved) return false;
    }
    return true;
}

// Zero-Bubble placement ([GPipe->ZB ZB1P 与 ZB2P]).  The page limits the
// micro-batches a device holds with their weight gradient not yet done to p
// (ZB1P) or 2p (ZB2P), p = P, on every device.  ZB1P keeps the 1F1B F/B
// order; ZB2P warms up with 2(P-k)-1 forwards, the slots device k has before
// its first backward can start under equal F/B/W costs, then alternates.  At
// each time step a free device runs its next F/B if the dependencies ended by
// now and (for F) its live count is below the budget; otherwise its oldest
// pending W; otherwise it idles.  Live = entries whose F has started and
// whose W has not.
bool run_zb(int P, int M, int budget_scale, std::vector<std::vector<Op3>>& lists,
            std::vector<std::vector<int>>& start) {
    std::vector<std::vector<Op3>> base(P);
    for (int d = 0; d < P; ++d)
        list_warm_alternate(M, budget_scale == 1 ? P - d : 2 * (P - d) - 1, base[d]);
    const int budget = budget_scale * P;
    EndTimes e(P, M, 1);
    std::vector<size_t> pos(P, 0);
    std::vector<std::deque<int>> pend(P);
    std::vector<int> live(P, 0), free_at(P, 0), w_done(P, 0);
    lists.assign(P, {});
    start.assign(P, {});
    const long limit = 4L * (3L * M + 2L * P) + 16;
    for (long t = 0;; ++t) {
        bool all = true;
        for (int d = 0; d < P; ++d) all = all && w_done[d] == M;
        if (all) break;
        if (t > limit) return false;
        for (int d = 0; d < P; ++d) {
            if (free_at[d] > t) continue;
            bool ran = false;
            Op3 op{};
            if (pos[d] < base[d].size()) {
                op = base[d][pos[d]];
                int r = ready_time(e, op, d);
                bool ok = r >= 0 && r <= t;
                if (ok && op.kind == OP_F && live[d] >= budget) ok = false;
                if (ok) {
                    ++pos[d];
                    if (op.kind == OP_F) ++live[d];
                    else pend[d].push_back(op.mb);
                    ran = true;
                }
            }
            if (!ran && !pend[d].empty()) {
                op = Op3{OP_W, pend[d].front(), 0};
                pend[d].pop_front();
                --live[d];
                ++w_done[d];
                ran = true;
            }
            if (ran) {
                lists[d].push_back(op);
                start[d].push_back((int)t);
                mark_end(e, op, d, (int)t + 1);
                free_at[d] = (int)t + 1;
            }
        }
    }
    return true;
}

}  // namespace

namespace {

// Op lists of all P devices for a schedule kind, with their unit-cost start
// times.  Returns a PPS_* status.
int build_lists(int P, int M, int v, int kind, std::vector<std::vector<Op3>>& lists,
                std::vector<std::vector<int>>& start, bool& split) {
    if (P < 1 || M < 1 || v < 1) return PPS_EINVAL;
    if (kind < PPS_GPIPE || kind > PPS_ZB2P) return PPS_EINVAL;
    // P*v first: with it bounded the product with M cannot overflow
    if ((long long)P * v > (1LL << 24) || (long long)P * v * M > (1LL << 24)) return PPS_EINVAL;
    if (v > 1 && (kind != PPS_1F1B || M % P != 0)) return PPS_EINVAL;
    lists.assign(P, {});
    split = false;
    if (kind == PPS_ZB1P || kind == PPS_ZB2P) {
        if (!run_zb(P, M, kind == PPS_ZB1P ? 1 : 2, lists, start)) return PPS_EINVAL;
        split = true;
    } else {
        for (int d = 0; d < P; ++d) {
            if (kind == PPS_GPIPE) list_gpipe(M, lists[d]);
            else if (v == 1) list_1f1b(P, M, d, lists[d]);
            else list_interleaved(P, M, d, v, lists[d]);
        }
        if (!run_fixed(lists, P, M, v, start)) return PPS_EINVAL;
    }
    return PPS_OK;
}

}  // namespace

int build_schedule(int P, int M, int k, int v, int kind, std::vector<pps_op>& out) {
    out.clear();
    if (k < 0 || k >= P) return PPS_EINVAL;
    std::vector<std::vector<Op3>> lists;
    std::vector<std::vector<int>> start;
    bool split = false;
    const int rc = build_lists(P, M, v, kind, lists, start, split);
    if (rc != PPS_OK) return rc;

    // Stash slots of device k: lowest free index, taken at F, released at B
    // (at W when split).
    const std::vector<Op3>& ops = lists[k];
    std::vector<int> slot_of((size_t)M * v, -1);
    std::vector<char> used;
    int live = 0;
    out.reserve(ops.size());
    for (size_t j = 0; j < ops.size(); ++j) {
        const Op3& op = ops[j];
        const size_t key = (size_t)op.chunk * M + op.mb;
        int s;
        if (op.kind == OP_F) {
            s = 0;
            while (s < (int)used.size() && used[s]) ++s;
            if (s == (int)used.size()) used.push_back(0);
            used[s] = 1;
            slot_of[key] = s;
            ++live;
        } else {
            s = slot_of[key];
            if ((op.kind == OP_B && !split) || op.kind == OP_W) { used[s] = 0; --live; }
        }
        pps_op rec;
        rec.op = op.kind;
        rec.mb = op.mb;
        rec.chunk = op.chunk;
        rec.slot = s;
        rec.inflight_after = live;
        rec.t_start = start[k][j];
        out.push_back(rec);
    }
    return PPS_OK;
}

}  // namespace pps

extern "C" int pps_make_schedule(int P, int M, int k, int v, int kind,
                                 pps_op* ops, int cap, int* n_ops) {
    if (!n_ops) return PPS_EINVAL;
    *n_ops = 0;
    if (cap < 0 || (cap > 0 && !ops)) return PPS_EINVAL;
    std::vector<pps_op> list;
    int rc = pps::build_schedule(P, M, k, v, kind, list);
    if (rc != PPS_OK) return rc;
    *n_ops = (int)list.size();
    if (cap < (int)list.size()) return PPS_EFULL;
    std::memcpy(ops, list.data(), list.size() * sizeof(pps_op));
    return PPS_OK;
}

extern "C" int pps_simulate_pipeline(int P, int M, int v, int kind, double t_f, double t_b, double t_w,
                                     double* makespan, double* bubble) {
    if (!makespan || !bubble) return PPS_EINVAL;
    for (double t : {t_f, t_b, t_w})
        if (!(t >= 0.0) || !std::isfinite(t)) return PPS_EINVAL;
    std::vector<std::vector<pps::Op3>> lists;
    std::vector<std::vector<int>> start;
    bool split = false;
    const int rc = pps::build_lists(P, M, v, kind, lists, start, split);
    if (rc != PPS_OK) return rc;
    const double dur[3] = {t_f, t_b, t_w};
    double end = 0.0, busy = 0.0;
    if (!pps::run_timed(lists, P, M, v, dur, end, busy)) return PPS_EINVAL;
    *makespan = end;
    *bubble = end > 0.0 ? 1.0 - busy / ((double)P * end) : 0.0;
    return PPS_OK;
}
