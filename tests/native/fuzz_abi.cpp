// Randomised calls into the C ABI on bookkeeping-only handles, with the
// library's host code (schedule generator and executor) built under the
// address and undefined-behaviour sanitizers; the kernel objects are linked as
// built, and a bookkeeping-only handle launches none of them.  Checks, besides
// the sanitizers' own:
//   - every status is one the header documents for that call;
//   - pps_make_schedule writes nothing past cap and reports the full count;
//   - a descriptor the header's limits accept creates a handle, one they
//     reject does not (and leaves *out untouched);
//   - the sizes a handle reports did not wrap;
//   - the schedule's own op list, replayed once or twice, is accepted call by
//     call, and the op log equals the schedule;
//   - calls that can never be valid at that point (out-of-range or finished
//     micro-batches, a backward before its forward, W without the split ...)
//     are rejected and change neither the statistics nor the op log.
// Usage: fuzz_abi SEED ITERATIONS.  Exit status 0 on success.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <set>
#include <utility>
#include <vector>

#include "pps.h"

namespace {

std::mt19937_64 rng;
long long checks = 0;

#define REQUIRE(cond, ...)                                                   \
    do {                                                                     \
        ++checks;                                                            \
        if (!(cond)) {                                                       \
            std::fprintf(stderr, "FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
            std::fprintf(stderr, __VA_ARGS__);                               \
            std::fprintf(stderr, "\n");                                      \
            std::exit(1);                                                    \
        }                                                                    \
    } while (0)

int64_t pick(int64_t lo, int64_t hi) { return lo + (int64_t)(rng() % (uint64_t)(hi - lo + 1)); }
template <class T, size_t N>
T pick_of(const T (&a)[N]) { return a[rng() % N]; }
bool coin(double p) { return std::uniform_real_distribution<double>(0.0, 1.0)(rng) < p; }

bool is_status(int rc) { return rc <= 0 && rc >= PPS_ETOOBIG; }

// ---- pps_make_schedule / pps_simulate_pipeline ------------------------------

void fuzz_schedule() {
    const int P = (int)pick(-2, 10), M = (int)pick(-2, 24), k = (int)pick(-2, 10), v = (int)pick(-1, 4);
    const int kind = (int)pick(-1, 4);
    int n = -7;
    int rc = pps_make_schedule(P, M, k, v, kind, nullptr, 0, &n);
    REQUIRE(rc == PPS_EFULL || rc == PPS_EINVAL, "make_schedule(%d,%d,%d,%d,%d) cap 0 -> %d", P, M, k, v, kind, rc);
    const bool valid_shape = P >= 1 && M >= 1 && k >= 0 && k < P && v >= 1 && kind >= PPS_GPIPE && kind <= PPS_ZB2P &&
                             (v == 1 || (kind == PPS_1F1B && M % P == 0));
    REQUIRE((rc == PPS_EFULL) == valid_shape, "make_schedule(%d,%d,%d,%d,%d) validity -> %d", P, M, k, v, kind, rc);
    REQUIRE(pps_make_schedule(P, M, k, v, kind, nullptr, 0, nullptr) == PPS_EINVAL, "NULL n_ops accepted");
    if (rc != PPS_EFULL) return;
    const int per = (kind == PPS_ZB1P || kind == PPS_ZB2P) ? 3 : 2;
    REQUIRE(n == per * M * v, "op count %d for M=%d v=%d kind=%d", n, M, v, kind);
    // a short array: EFULL, the count still set, nothing written past cap
    const int cap = (int)pick(0, n);
    std::vector<pps_op> ops((size_t)n + 4);
    std::memset(ops.data(), 0x5a, ops.size() * sizeof(pps_op));
    int n2 = -1;
    rc = pps_make_schedule(P, M, k, v, kind, ops.data(), cap, &n2);
    REQUIRE(rc == (cap < n ? PPS_EFULL : PPS_OK) && n2 == n, "cap %d of %d -> rc %d n %d", cap, n, rc, n2);
    const unsigned char* tail = reinterpret_cast<const unsigned char*>(ops.data() + cap);
    for (size_t i = 0; i < (ops.size() - (size_t)cap) * sizeof(pps_op); ++i)
        REQUIRE(tail[i] == 0x5a, "byte %zu past cap %d written", i, cap);
    rc = pps_make_schedule(P, M, k, v, kind, ops.data(), n, &n2);
    REQUIRE(rc == PPS_OK && n2 == n, "full array -> %d", rc);
    for (int i = 0; i < n; ++i) {
        const pps_op& o = ops[(size_t)i];
        REQUIRE(o.op >= PPS_OP_F && o.op <= PPS_OP_W && o.mb >= 0 && o.mb < M && o.chunk >= 0 && o.chunk < v &&
                    o.inflight_after >= 0 && o.t_start >= 0,
                "op %d fields out of range", i);
    }
    // the simulator on the same shape, with durations that may be invalid
    const double durs[] = {0.0, 1.0, 2.5, -1.0, INFINITY, NAN, 1e300};
    const double tf = pick_of(durs), tb = pick_of(durs), tw = pick_of(durs);
    double makespan = -1, bubble = -1;
    rc = pps_simulate_pipeline(P, M, v, kind, tf, tb, tw, &makespan, &bubble);
    const bool ok_d = std::isfinite(tf) && std::isfinite(tb) && std::isfinite(tw) && tf >= 0 && tb >= 0 && tw >= 0;
    if (P * M * v <= 4096) {
        REQUIRE(rc == (ok_d ? PPS_OK : PPS_EINVAL), "simulate(%g,%g,%g) -> %d", tf, tb, tw, rc);
        if (rc == PPS_OK) REQUIRE(makespan >= 0 && std::isfinite(makespan) && bubble >= 0 && bubble <= 1,
                                  "makespan %g bubble %g", makespan, bubble);
    } else {
        REQUIRE(rc == PPS_OK || rc == PPS_EINVAL, "simulate -> %d", rc);
    }
    REQUIRE(pps_simulate_pipeline(P, M, v, kind, 1, 1, 1, nullptr, &bubble) == PPS_EINVAL, "NULL makespan accepted");
}

// ---- stage handles ----------------------------------------------------------

struct Snap {
    pps_stats s;
    std::vector<pps_op> log;
};

Snap snap(const pps_stage* h) {
    Snap x;
    REQUIRE(pps_stage_get_stats(h, &x.s) == PPS_OK, "get_stats");
    int n = 0;
    const int rc = pps_stage_get_oplog(h, nullptr, 0, &n);
    REQUIRE(rc == PPS_OK || rc == PPS_EFULL, "get_oplog count -> %d", rc);
    x.log.resize((size_t)n);
    int n2 = 0;
    REQUIRE(pps_stage_get_oplog(h, x.log.data(), n, &n2) == PPS_OK && n2 == n, "get_oplog");
    return x;
}

bool same(const Snap& a, const Snap& b) {
    return std::memcmp(&a.s, &b.s, sizeof(pps_stats)) == 0 && a.log.size() == b.log.size() &&
           (a.log.empty() || std::memcmp(a.log.data(), b.log.data(), a.log.size() * sizeof(pps_op)) == 0);
}

// A call that cannot be accepted in the current state: returns (op, mb, chunk).
struct Bad {
    int op, mb, chunk;
};

Bad bad_call(const pps_stage_desc& d, const std::set<std::pair<int, int>>& fdone, const std::set<std::pair<int, int>>& bdone,
             const std::set<std::pair<int, int>>& wdone) {
    const bool split = d.kind == PPS_ZB1P || d.kind == PPS_ZB2P;
    for (int tries = 0; tries < 64; ++tries) {
        const int op = (int)pick(0, 2), mb = (int)pick(-2, d.M + 1), ch = (int)pick(-1, d.v);
        const bool in_range = mb >= 0 && mb < d.M && ch >= 0 && ch < d.v;
        const std::pair<int, int> key{mb, ch};
        if (!in_range) return {op, mb, ch};
        if (op == PPS_OP_W && !split) return {op, mb, ch};
        if (op == PPS_OP_F && fdone.count(key)) return {op, mb, ch};             // forward already ran
        if (op == PPS_OP_B && (!fdone.count(key) || bdone.count(key))) return {op, mb, ch};  // no entry / twice
        if (op == PPS_OP_W && (!bdone.count(key) || wdone.count(key))) return {op, mb, ch};  // before B / twice
    }
    return {PPS_OP_F, -1, 0};
}

int issue(pps_stage* h, int op, int mb, int chunk) {
    if (op == PPS_OP_F) return pps_stage_forward(h, mb, chunk, nullptr, nullptr);
    if (op == PPS_OP_B) return pps_stage_backward(h, mb, chunk, nullptr, nullptr);
    return pps_stage_backward_weight(h, mb, chunk);
}

pps_stage_desc random_desc(bool& expect_ok) {
    pps_stage_desc d;
    std::memset(&d, 0, sizeof d);
    const bool sane = coin(0.7);
    if (sane) {
        d.P = (int)pick(1, 8);
        d.k = (int)pick(0, d.P - 1);
        d.kind = (int)pick(PPS_GPIPE, PPS_ZB2P);
        d.v = d.kind == PPS_1F1B && coin(0.3) ? (int)pick(2, 3) : 1;
        d.M = d.v > 1 ? d.P * (int)pick(1, 3) : (int)pick(1, 12);
        d.block_type = coin(0.8) ? PPS_BLOCK_SWIGLU : PPS_BLOCK_TOY_GELU;
        d.dtype = d.block_type == PPS_BLOCK_TOY_GELU || coin(0.3) ? PPS_DTYPE_FP32 : PPS_DTYPE_BF16;
        d.L = (int)pick(1, 4);
        d.d = 8 * pick(1, 64);
        d.ffn = 8 * pick(1, 96);
        d.T = pick(0, 600);
        d.eps = 1e-6f;
        d.flags = PPS_FLAG_BOOKKEEPING_ONLY;
        if (d.block_type == PPS_BLOCK_SWIGLU && d.kind != PPS_ZB1P && d.kind != PPS_ZB2P && coin(0.3))
            d.flags |= PPS_FLAG_RECOMPUTE;
        expect_ok = true;
        return d;
    }
    // anything: limits, just past them, and far out
    const int32_t i32s[] = {-2147483647 - 1, -5, -1, 0, 1, 2, 3, 4, 7, 8, 9, 16, 4096, 1 << 20, (1 << 20) + 1,
                            1 << 24, 2147483647};
    const int64_t sizes[] = {INT64_MIN, -8, -1, 0, 1, 7, 8, 9, 64, 264, 16384, 16392, 1 << 20, (int64_t)1 << 24,
                             ((int64_t)1 << 24) + 8, (int64_t)1 << 31, (int64_t)1 << 40, (int64_t)1 << 62, INT64_MAX};
    d.P = pick_of(i32s); d.M = pick_of(i32s); d.k = pick_of(i32s); d.v = pick_of(i32s);
    d.kind = (int)pick(-1, 4); d.block_type = (int)pick(-1, 2); d.dtype = (int)pick(-1, 2);
    d.L = pick_of(i32s);
    d.d = pick_of(sizes); d.ffn = pick_of(sizes); d.T = pick_of(sizes);
    const float epss[] = {1e-6f, 0.0f, -1.0f, NAN, INFINITY};
    d.eps = pick_of(epss);
    d.flags = PPS_FLAG_BOOKKEEPING_ONLY | (coin(0.3) ? PPS_FLAG_RECOMPUTE : 0u) | (coin(0.2) ? 8u : 0u);
    d.profile_capacity = (int)pick(-1, 4);
    expect_ok = false;   // not known: either status is fine, the handle must then work
    return d;
}

void fuzz_stage() {
    bool expect_ok = false;
    pps_stage_desc d = random_desc(expect_ok);
    pps_stage* h = reinterpret_cast<pps_stage*>(uintptr_t(0x1234));
    int rc = coin(0.1) ? pps_stage_create_noalloc(&d, &h) : pps_stage_create(&d, &h);
    REQUIRE(rc == PPS_OK || rc == PPS_EINVAL || rc == PPS_ETOOBIG,
            "create P=%d M=%d k=%d v=%d kind=%d L=%d d=%lld ffn=%lld T=%lld -> %d", d.P, d.M, d.k, d.v, d.kind, d.L,
            (long long)d.d, (long long)d.ffn, (long long)d.T, rc);
    if (rc != PPS_OK) {
        REQUIRE(!expect_ok || rc == PPS_ETOOBIG, "a descriptor within the limits was rejected: %d", rc);
        REQUIRE(h == reinterpret_cast<pps_stage*>(uintptr_t(0x1234)), "*out written on failure");
        return;
    }
    REQUIRE(h != nullptr, "NULL handle on success");
    {
        // the sizes the handle reports did not wrap: each holds at least the
        // tensors it must (one [T, d] input per slot; dx ping-pong [T, d]
        // twice in scratch; a [d] gradient per block)
        pps_stats s;
        REQUIRE(pps_stage_get_stats(h, &s) == PPS_OK, "get_stats");
        const double es = d.dtype == PPS_DTYPE_BF16 ? 2.0 : 4.0, td = (double)d.T * (double)d.d * es;
        REQUIRE((double)s.pool_bytes == (double)s.n_slots * (double)s.slot_bytes && (double)s.slot_bytes >= td &&
                    (double)s.scratch_bytes >= 2.0 * td && (double)s.grad_bytes >= (double)d.v * d.L * d.d * 4.0,
                "sizes: slots %lld x %lld, scratch %lld, grads %lld for T=%lld d=%lld", (long long)s.n_slots,
                (long long)s.slot_bytes, (long long)s.scratch_bytes, (long long)s.grad_bytes, (long long)d.T,
                (long long)d.d);
    }
    int n = 0;
    rc = pps_make_schedule(d.P, d.M, d.k, d.v, d.kind, nullptr, 0, &n);
    REQUIRE(rc == PPS_EFULL, "schedule of an accepted desc -> %d", rc);
    std::vector<pps_op> sched((size_t)n);
    REQUIRE(pps_make_schedule(d.P, d.M, d.k, d.v, d.kind, sched.data(), n, &n) == PPS_OK, "schedule");
    const float* g = nullptr;
    REQUIRE(pps_stage_get_grad(h, 0, 0, 0, &g) == PPS_EINVAL, "get_grad on a bookkeeping handle");
    int nk = 0;
    REQUIRE(pps_stage_kernel_times(h, nullptr, 0, &nk) == PPS_EINVAL, "kernel_times without profiling");
    const int passes = (int)pick(1, 2);
    for (int pass = 0; pass < passes; ++pass) {
        rc = pps_stage_zero_grad(h);
        REQUIRE(rc == PPS_OK, "zero_grad -> %d", rc);
        std::set<std::pair<int, int>> fdone, bdone, wdone;
        for (size_t i = 0; i < sched.size(); ++i) {
            while (coin(0.25)) {
                const Snap before = snap(h);
                const Bad b = bad_call(d, fdone, bdone, wdone);
                rc = issue(h, b.op, b.mb, b.chunk);
                REQUIRE(rc != PPS_OK && is_status(rc), "invalid op %d mb %d chunk %d accepted (%d)", b.op, b.mb, b.chunk,
                        rc);
                REQUIRE(same(before, snap(h)), "rejected op %d mb %d chunk %d changed the handle", b.op, b.mb, b.chunk);
            }
            const pps_op& o = sched[i];
            rc = issue(h, o.op, o.mb, o.chunk);
            REQUIRE(rc == PPS_OK, "pass %d op %zu (%d mb %d chunk %d) -> %d", pass, i, o.op, o.mb, o.chunk, rc);
            (o.op == PPS_OP_F ? fdone : o.op == PPS_OP_B ? bdone : wdone).insert({o.mb, o.chunk});
        }
        const Snap end = snap(h);
        REQUIRE(end.log.size() == sched.size(), "op log %zu entries, schedule %zu", end.log.size(), sched.size());
        for (size_t i = 0; i < sched.size(); ++i) {
            const pps_op &a = end.log[i], &b = sched[i];
            REQUIRE(a.op == b.op && a.mb == b.mb && a.chunk == b.chunk && a.slot == b.slot &&
                        a.inflight_after == b.inflight_after && a.t_start == b.t_start,
                    "op log entry %zu differs from the schedule", i);
        }
        REQUIRE(end.s.passes_completed == pass + 1 && end.s.live_entries == 0 &&
                    end.s.peak_live_entries <= end.s.n_slots,
                "after pass %d: passes %lld live %lld peak %lld slots %lld", pass, (long long)end.s.passes_completed,
                (long long)end.s.live_entries, (long long)end.s.peak_live_entries, (long long)end.s.n_slots);
        // right after a completed pass no backward has an entry
        rc = pps_stage_backward(h, 0, 0, nullptr, nullptr);
        REQUIRE(rc == PPS_ENOENT, "backward after a completed pass -> %d", rc);
    }
    REQUIRE(pps_stage_sync(h) == PPS_OK, "sync");
    pps_stage_destroy(h);
}

void null_handles() {
    REQUIRE(pps_stage_forward(nullptr, 0, 0, nullptr, nullptr) == PPS_EINVAL, "forward(NULL)");
    REQUIRE(pps_stage_backward(nullptr, 0, 0, nullptr, nullptr) == PPS_EINVAL, "backward(NULL)");
    REQUIRE(pps_stage_backward_weight(nullptr, 0, 0) == PPS_EINVAL, "backward_weight(NULL)");
    REQUIRE(pps_stage_zero_grad(nullptr) == PPS_EINVAL, "zero_grad(NULL)");
    REQUIRE(pps_stage_sync(nullptr) == PPS_EINVAL, "sync(NULL)");
    pps_stats s;
    REQUIRE(pps_stage_get_stats(nullptr, &s) == PPS_EINVAL, "get_stats(NULL)");
    int n = 0;
    REQUIRE(pps_stage_get_oplog(nullptr, nullptr, 0, &n) == PPS_EINVAL, "get_oplog(NULL)");
    REQUIRE(pps_stage_create(nullptr, nullptr) == PPS_EINVAL, "create(NULL)");
    pps_stage_destroy(nullptr);
    for (int s2 = -10; s2 <= 1; ++s2) REQUIRE(pps_strerror(s2) != nullptr, "strerror(%d)", s2);
    for (int k2 = -1; k2 <= PPS_K_COUNT; ++k2) REQUIRE(pps_kernel_name(k2) != nullptr, "kernel_name(%d)", k2);
}

}  // namespace

int main(int argc, char** argv) {
    if (argc != 3) return 2;
    rng.seed(std::strtoull(argv[1], nullptr, 10));
    const long iters = std::strtol(argv[2], nullptr, 10);
    null_handles();
    for (long i = 0; i < iters; ++i) {
        fuzz_schedule();
        fuzz_stage();
    }
    std::printf("ok %lld checks\n", checks);
    return 0;
}
