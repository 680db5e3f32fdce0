// The stage executor behind the C ABI: call validation against the stage's
// schedule, the preallocated activation stash, and the per-op kernel
// sequences.
//
// Page legend: [1F1B] "2. 1F1B"; [GPipe->ZB] "流水线并行：从 GPipe 到 1F1B 与
// Zero Bubble"; [Sched] "流水线调度：GPipe、1F1B、交错与计算通信重叠";
// [Megatron-PP] "Megatron-LM 分布式训练（三）：流水线并行 PP 与 1F1B 调度".
//
// The stash plays the role of the per-stage activations dict of [1F1B §5.2]:
// a forward stores what its backward needs, the backward takes the entry
// out and releases it, and the number of live entries is the in-flight count
// ([1F1B §4.1]).  Entries live in a pool of S fixed-size slots allocated once
// at create ([1F1B §5.3]: reuse buffers instead of allocating per message);
// S is the schedule's peak live count (P-k for 1F1B, M for GPipe).
//
// SwiGLU block b of an entry keeps x [T,d], r [T] (fp32), g and u [T,ffn].
// With the Zero-Bubble split ([GPipe->ZB Zero Bubble]: B = dX now, W = dW
// later, X and G stay resident until W) the entry also keeps dg|du [T,2ffn]
// (bf16 on full 256-row tiles: T-contiguous, [2ffn,T]) and dy [T,d] per
// block after B, until W.
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "kernels.h"
#include "schedule_internal.h"

namespace {

using pps::GemmArgs;

constexpr int ST_NONE = 0, ST_F = 1, ST_B = 2, ST_W = 3;

inline size_t align256(size_t b) { return (b + 255) & ~size_t(255); }

struct Layout {
    // offsets inside one slot, per block (index b)
    std::vector<size_t> x, r, g, u, dgu, dy, z, dz;
    size_t fwd_bytes = 0;     // bytes an entry uses before B
    size_t split_bytes = 0;   // extra bytes kept from B until W
    size_t slot_bytes = 0;
};

}  // namespace

struct pps_stage {
    pps_stage_desc d{};
    std::vector<const void*> w;
    bool bookkeeping = false, profile = false, split = false, swiglu = true;
    int es = 2;                       // element size of the storage dtype
    int nw = 4;                       // weights per block
    int S = 0;                        // slots
    std::vector<pps_op> sched;
    std::vector<std::pair<int, int>> fseq, bseq, wseq;   // (mb, chunk) per kind, in order
    std::vector<int> tf, tb, tw;                          // t_start per kind entry
    size_t fpos = 0, bpos = 0, wpos = 0;
    std::vector<int> status, slot_of;                     // [chunk*M + mb]
    std::vector<char> slot_used;
    int live = 0;
    int64_t live_bytes = 0;
    std::vector<pps_op> oplog;
    pps_stats st{};
    bool failed = false;

    hipStream_t stream = nullptr;
    Layout lay;
    bool noalloc = false;             // device memory carved from the fixed array, never freed
    char* pool = nullptr;
    char* scratch = nullptr;
    size_t scratch_bytes = 0;
    // recompute mode: slots hold the stage input only; the per-block tensors
    // of the micro-batch being back-propagated live at scratch + s_rc
    bool ac = false;
    size_t s_rc = 0;
    size_t s_n = 0, s_h = 0, s_dgu = 0, s_dn = 0, s_dxa = 0, s_dxb = 0, s_part = 0, s_dz = 0;
    // bf16 weight gradients: T-contiguous h, n, dy and dg|du (copies, or from the dh epilogue)
    // ([features, Tp], Tp = T rounded up to 8, zero-padded)
    size_t s_hT = 0, s_nT = 0, s_dyT = 0, s_dguT = 0;
    int64_t Tp = 0;
    bool tn = false;                  // bf16 path: the forward GEMMs read K-contiguous weight copies
    int ncu = 256;                    // compute units of the handle's device (GEMM tile waves)
    // bf16 path: per-pass copies of the forward weights, [chunk*L + block]:
    // WguT (swiglu_b_rows(ffn) x d, gate/up interleaved per 32) and WdT (d x ffn)
    char* wcopy = nullptr;
    size_t wcopy_bytes = 0;
    std::vector<size_t> wgu_off, wd_off;
    float* grads = nullptr;
    size_t grad_bytes = 0;
    std::vector<size_t> goff;         // [(chunk*L + block)*4 + which] element offsets

    // kernel timing
    std::vector<hipEvent_t> ev;
    std::vector<int> ev_kernel;
    std::vector<double> ev_flops, ev_bytes;
    int ev_used = 0;
    double kt_ms[PPS_K_COUNT] = {};
    double kt_flops[PPS_K_COUNT] = {};
    double kt_bytes[PPS_K_COUNT] = {};
    int64_t kt_n[PPS_K_COUNT] = {};       // timed launches since the last report
    int64_t kt_calls[PPS_K_COUNT] = {};   // all launches since the last report
    int64_t kt_seen[PPS_K_COUNT] = {};    // all launches since create (the stride's phase)
    int stride = 1;
};

namespace {

int64_t T_(const pps_stage* h) { return h->d.T; }

char* slot_base(pps_stage* h, int s) { return h->pool + (size_t)s * h->lay.slot_bytes; }

// Base of the per-block forward tensors (offsets h->lay.x/r/g/u) of the
// micro-batch in `slot`: the slot itself, or the shared recompute area.
char* acts(pps_stage* h, int slot) { return h->ac ? h->scratch + h->s_rc : slot_base(h, slot); }

// Block b's input; in recompute mode block 0's (the stage input) stays in the slot.
char* act_x(pps_stage* h, int slot, int b) {
    return (h->ac && b == 0) ? slot_base(h, slot) : acts(h, slot) + h->lay.x[b];
}

template <typename F>
hipError_t timed(pps_stage* h, int kernel, double flops, double bytes, F&& launch) {
    bool rec = false;
    if (h->profile) {
        rec = h->kt_seen[kernel]++ % h->stride == 0 && h->ev_used < (int)h->ev_kernel.size();
        ++h->kt_calls[kernel];
    }
    if (rec) {
        hipError_t e = hipEventRecord(h->ev[2 * h->ev_used], h->stream);
        if (e != hipSuccess) return e;
    }
    hipError_t e = launch();
    if (e != hipSuccess) return e;
    if (rec) {
        e = hipEventRecord(h->ev[2 * h->ev_used + 1], h->stream);
        if (e != hipSuccess) return e;
        h->ev_kernel[h->ev_used] = kernel;
        h->ev_flops[h->ev_used] = flops;
        h->ev_bytes[h->ev_used] = bytes;
        ++h->ev_used;
    }
    return hipSuccess;
}

#define PPS_TRY(expr)                          \
    do {                                       \
        hipError_t _e = (expr);                \
        if (_e != hipSuccess) {                \
            h->failed = true;                  \
            return PPS_EHIP;                   \
        }                                      \
    } while (0)

// With the split, each block also keeps dg|du [T, 2 ffn] (or, T-contiguous,
// [2 ffn, T]: same bytes, T being a multiple of 256 then) and dy [T, d] for
// the deferred weight-gradient GEMMs.
Layout make_layout(const pps_stage_desc& d, bool swiglu, bool split, int es) {
    Layout L;
    const size_t T = (size_t)d.T, dm = (size_t)d.d, f = (size_t)d.ffn;
    size_t off = 0;
    const int nb = d.L;
    auto take = [&](std::vector<size_t>& v, size_t bytes) { v.push_back(off); off += align256(bytes); };
    for (int b = 0; b < nb; ++b) {
        if (swiglu) {
            take(L.x, T * dm * es);
            take(L.r, T * 4);
            take(L.g, T * f * es);
            take(L.u, T * f * es);
        } else {
            take(L.x, T * dm * 4);
            take(L.z, T * dm * 4);
        }
    }
    L.fwd_bytes = off;
    if (split) {
        for (int b = 0; b < nb; ++b) {
            if (swiglu) {
                take(L.dgu, T * 2 * f * es);
                take(L.dy, T * dm * es);
            } else {
                take(L.dz, T * dm * 4);
            }
        }
    }
    L.split_bytes = off - L.fwd_bytes;
    L.slot_bytes = std::max<size_t>(off, 256);
    return L;
}

int validate_desc(const pps_stage_desc* d) {
    if (!d) return PPS_EINVAL;
    // Schedule parameters first: everything below sizes host arrays from them.
    if (d->P < 1 || d->M < 1 || d->v < 1 || d->L < 1 || d->k < 0 || d->k >= d->P) return PPS_EINVAL;
    if (d->kind < PPS_GPIPE || d->kind > PPS_ZB2P) return PPS_EINVAL;
    if ((long long)d->P * d->v > (1LL << 24) || (long long)d->P * d->v * d->M > (1LL << 24) ||
        (long long)d->v * d->L > (1LL << 20))
        return PPS_EINVAL;
    if (d->block_type != PPS_BLOCK_SWIGLU && d->block_type != PPS_BLOCK_TOY_GELU) return PPS_EINVAL;
    if (d->dtype != PPS_DTYPE_BF16 && d->dtype != PPS_DTYPE_FP32) return PPS_EINVAL;
    if (d->block_type == PPS_BLOCK_TOY_GELU && d->dtype != PPS_DTYPE_FP32) return PPS_EINVAL;
    // T: the RMSNorm forward launches one workgroup of 256 lanes per row
    if (d->L < 1 || d->d < 8 || d->d % 8 != 0 || d->d > 16384 || d->T < 0 || d->T > (1LL << 24)) return PPS_EINVAL;
    if (d->block_type == PPS_BLOCK_SWIGLU && (d->ffn < 8 || d->ffn % 8 != 0)) return PPS_EINVAL;
    if (d->block_type == PPS_BLOCK_SWIGLU && d->ffn > (1LL << 30)) return PPS_EINVAL;
    {
        // Every byte count the layout forms (stash slots, scratch, gradients,
        // weight copies) stays far inside 64 bits: bound the whole footprint
        // from above in double precision, 4-byte elements and generous
        // padding throughout.
        const double T = (double)d->T, dm = (double)d->d, f = d->block_type == PPS_BLOCK_SWIGLU ? (double)d->ffn : dm;
        const double blocks = (double)d->v * d->L, pad = 64.0 * 256.0;
        const double tensors = (T + 8) * (2.0 * dm + 4.0 * f + 2.0) * 4.0 + pad;   // one block's entry (+ split)
        const double pool = (double)d->M * d->v * (d->L * tensors + pad);
        const double scratch = (T + 8) * (8.0 * dm + 8.0 * f + 8.0) * 4.0 + pad;
        const double params = blocks * ((3.0 * dm * f + dm * dm + dm) * 4.0 + (2.0 * (f + 32) * dm + dm * f) * 2.0 + pad);
        if (pool + tensors * d->L + scratch + params > 1e18) return PPS_EINVAL;
    }
    if ((d->flags & PPS_FLAG_RECOMPUTE) &&
        (d->block_type != PPS_BLOCK_SWIGLU || d->kind == PPS_ZB1P || d->kind == PPS_ZB2P))
        return PPS_EINVAL;
    if (!(d->eps >= 0.0f)) return PPS_EINVAL;
    if (d->block_type == PPS_BLOCK_SWIGLU && d->dtype == PPS_DTYPE_BF16) {
        // The MFMA GEMM addresses each operand with 32-bit byte offsets: the
        // largest ones (dg|du [T, 2 ffn] and its T-contiguous copy, rows
        // padded to a multiple of 8; the [T, d] operands and their copies;
        // the interleaved gate/up weight copy) must stay under 2 GiB.
        const double lim = 2147483648.0, Tp = (double)((d->T + 7) / 8 * 8);
        const double f2 = 2.0 * (double)d->ffn, rows = (double)pps::swiglu_b_rows(d->ffn);
        if (Tp * f2 * 2 >= lim || Tp * (double)d->d * 2 >= lim || rows * (double)d->d * 2 >= lim)
            return PPS_EINVAL;
    }
    if ((d->flags & PPS_FLAG_PROFILE) && (d->profile_capacity < 0 || d->profile_stride < 0)) return PPS_EINVAL;
    if (!(d->flags & PPS_FLAG_BOOKKEEPING_ONLY)) {
        if (!d->weights) return PPS_EINVAL;
        const int nw = d->block_type == PPS_BLOCK_SWIGLU ? 4 : 2;
        for (int i = 0; i < d->v * d->L * nw; ++i)
            if (!d->weights[i]) return PPS_EINVAL;
    }
    return PPS_OK;
}

void release(pps_stage* h) {
    if (!h) return;
    for (hipEvent_t e : h->ev)
        if (e) (void)hipEventDestroy(e);
    if (!h->noalloc) {
        if (h->pool) (void)hipFree(h->pool);
        if (h->scratch) (void)hipFree(h->scratch);
        if (h->grads) (void)hipFree(h->grads);
        if (h->wcopy) (void)hipFree(h->wcopy);
    }
    delete h;
}

bool pass_done(const pps_stage* h) {
    return h->fpos == h->fseq.size() && h->bpos == h->bseq.size() && h->wpos == h->wseq.size();
}

void maybe_new_pass(pps_stage* h) {
    if (pass_done(h)) {
        h->fpos = h->bpos = h->wpos = 0;
        std::fill(h->status.begin(), h->status.end(), ST_NONE);
        h->oplog.clear();
    }
}

// After an accepted op: the op that completes the op list completes a pass.
void count_pass(pps_stage* h) {
    if (pass_done(h)) ++h->st.passes_completed;
}

void log_op(pps_stage* h, int op, int mb, int chunk, int slot, int t) {
    pps_op rec;
    rec.op = op;
    rec.mb = mb;
    rec.chunk = chunk;
    rec.slot = slot;
    rec.inflight_after = h->live;
    rec.t_start = t;
    h->oplog.push_back(rec);
    h->st.live_entries = h->live;
    h->st.live_bytes = h->live_bytes;
    h->st.peak_live_entries = std::max<int64_t>(h->st.peak_live_entries, h->live);
    h->st.peak_live_bytes = std::max<int64_t>(h->st.peak_live_bytes, h->live_bytes);
}

double gemm_flops(double M, double N, double K) { return 2.0 * M * N * K; }

// ---- SwiGLU block sequences ------------------------------------------------

// bf16 path: refresh the K-contiguous copies of the forward weights from the
// caller's Wg, Wu ([d, ffn]), gamma ([d]) and Wd ([ffn, d]).  Done once at the
// start of every pass, so weights updated between passes are picked up.  The
// RMSNorm scale gamma is folded into the gate/up copy: g = (x r gamma) Wg =
// r (x (gamma Wg)), with r applied per row in the GEMM's epilogue.
int refresh_weight_copies(pps_stage* h) {
    const pps_stage_desc& D = h->d;
    const int64_t d = D.d, f = D.ffn;
    for (int i = 0; i < D.v * D.L; ++i) {
        const void* const* wb = h->w.data() + (size_t)i * 4;
        const float* gamma = static_cast<const float*>(wb[3]);
        char* wgu = h->wcopy + h->wgu_off[i];
        char* wdt = h->wcopy + h->wd_off[i];
        PPS_TRY(timed(h, PPS_K_COPY, 0.0, 4.0 * d * f * 2 + 2.0 * d * 4, [&] {
            hipError_t e = pps::transpose_bf16(wb[0], d, f, f, wgu, d, 32, 0, h->stream, gamma);
            if (e == hipSuccess) e = pps::transpose_bf16(wb[1], d, f, f, wgu, d, 32, 1, h->stream, gamma);
            return e;
        }));
        PPS_TRY(timed(h, PPS_K_COPY, 0.0, 2.0 * d * f * 2, [&] {
            return pps::transpose_bf16(wb[2], f, d, d, wdt, f, 0, 0, h->stream);
        }));
    }
    return PPS_OK;
}

// Forward of the chunk's blocks for the micro-batch in `slot`.  With
// `recompute` (recompute mode, inside the backward) the input is the one the
// slot already holds and y_out is unused: the last block's down GEMM, whose
// output no backward reads, is skipped.
int swiglu_forward(pps_stage* h, int slot, int chunk, const void* x_in, void* y_out, bool recompute = false) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d, f = D.ffn;
    const int dt = D.dtype, es = h->es;
    char* ab = acts(h, slot);
    char* sn = h->scratch + h->s_n;
    char* sh = h->scratch + h->s_h;
    const int blk0 = chunk * D.L;
    for (int b = 0; b < D.L; ++b) {
        const void* const* wb = h->w.data() + (size_t)(blk0 + b) * 4;
        const float* gamma = static_cast<const float*>(wb[3]);
        char* xb = act_x(h, slot, b);
        float* rb = reinterpret_cast<float*>(ab + h->lay.r[b]);
        char* gb = ab + h->lay.g[b];
        char* ub = ab + h->lay.u[b];
        const bool copy_in = b == 0 && !recompute;
        const void* xin = copy_in ? x_in : xb;
        // RMSNorm: r per row; block 0 also copies x into the stash.  bf16: the
        // gate/up GEMM reads x and applies r in its epilogue (gamma is in the
        // weight copy), so n is not formed; fp32: n = x r gamma ([T,d]).
        const double norm_bytes = h->tn ? (double)T * d * es * (copy_in ? 2 : 1) + T * 4.0
                                        : (double)T * d * es * (copy_in ? 3 : 2) + T * 4.0 + d * 4.0;
        PPS_TRY(timed(h, PPS_K_RMSNORM_FWD, 0.0, norm_bytes, [&] {
            return pps::rmsnorm_fwd(dt, xin, gamma, D.eps, T, d, rb, h->tn ? nullptr : sn, copy_in ? xb : nullptr,
                                    h->stream);
        }));
        // g, u = n [Wg | Wu] (bf16: r x [gamma Wg | gamma Wu]) with
        // h = silu(g) u in the epilogue.
        GemmArgs a;
        a.M = T; a.N = f; a.nseg = 1;
        a.seg[0].A = sn; a.seg[0].lda = d; a.seg[0].K = d;
        a.a_kcontig = true; a.swiglu_map = true;
        if (h->tn) {
            a.seg[0].A = xin;
            a.seg[0].B = h->wcopy + h->wgu_off[blk0 + b]; a.seg[0].ldb = d; a.b_kcontig = true;
            a.e.rowscale = rb;
        } else {
            a.seg[0].B = wb[0]; a.seg[0].B2 = wb[1]; a.seg[0].ldb = f; a.b_kcontig = false;
        }
        a.epi = pps::EPI_SWIGLU;
        a.e.out0 = gb; a.e.out1 = ub; a.e.out2 = sh; a.e.ld0 = f;
        PPS_TRY(timed(h, PPS_K_GATEUP, gemm_flops(T, 2.0 * f, d), 0.0, [&] { return pps::gemm(dt, a, h->stream); }));
        if (recompute && b == D.L - 1) break;
        // y = x + h Wd, written as the next block's x (or the stage output).
        GemmArgs c;
        c.M = T; c.N = d; c.nseg = 1;
        c.seg[0].A = sh; c.seg[0].lda = f; c.seg[0].K = f;
        c.a_kcontig = true;
        if (h->tn) {
            c.seg[0].B = h->wcopy + h->wd_off[blk0 + b]; c.seg[0].ldb = f; c.b_kcontig = true;
        } else {
            c.seg[0].B = wb[2]; c.seg[0].ldb = d; c.b_kcontig = false;
        }
        c.epi = pps::EPI_RESID;
        c.e.out0 = b == D.L - 1 ? y_out : static_cast<void*>(act_x(h, slot, b + 1));
        c.e.ld0 = d; c.e.in0 = xb; c.e.ldi0 = d;
        PPS_TRY(timed(h, PPS_K_DOWN, gemm_flops(T, d, f), 0.0, [&] { return pps::gemm(dt, c, h->stream); }));
    }
    return PPS_OK;
}

// Weight gradient of block b: dWd += h^T dy; dWg += n^T dg; dWu += n^T du.
// The GEMMs reduce over the T rows.  bf16: the operands are first copied
// T-contiguous ([features, T]) for the K-contiguous kernel; fp32 reads them as
// stored.  With `have_nh` the backward just produced n (scratch) and h
// (bf16: h and dg|du already T-contiguous, written so by the dh epilogue;
// fp32: scratch); otherwise n and h are recomputed from the stash.
// bf16 without the split: the dh epilogue writes hT and dguT (T and ffn
// multiples of the 256 x 256 GEMM tile)
bool hT_fused(const pps_stage* h) { return h->tn && h->d.T % 256 == 0 && h->d.ffn % 256 == 0; }

int swiglu_weight(pps_stage* h, int slot, int chunk, int b, const void* dy, const void* dgu, bool have_nh) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d, f = D.ffn;
    const int dt = D.dtype, es = h->es;
    const void* const* wb = h->w.data() + (size_t)(chunk * D.L + b) * 4;
    const float* gamma = static_cast<const float*>(wb[3]);
    const size_t gi = (size_t)(chunk * D.L + b) * 4;
    float* dWg = h->grads + h->goff[gi + 0];
    float* dWu = h->grads + h->goff[gi + 1];
    float* dWd = h->grads + h->goff[gi + 2];
    char* ab = acts(h, slot);
    char* sn = h->scratch + h->s_n;
    char* sh = h->scratch + h->s_h;
    const char* xb = act_x(h, slot, b);
    const float* rb = reinterpret_cast<const float*>(ab + h->lay.r[b]);
    if (!have_nh && !h->tn) {
        PPS_TRY(timed(h, PPS_K_PREP_W, 0.0, (double)T * (2.0 * d + 3.0 * f) * es + T * 4.0 + d * 4.0, [&] {
            return pps::prep_w(dt, xb, rb, gamma, ab + h->lay.g[b], ab + h->lay.u[b], T, d, f, sn, sh, h->stream);
        }));
    }
    GemmArgs a, c;
    a.M = f; a.N = d; a.nseg = 1;
    a.seg[0].A = sh; a.seg[0].lda = f; a.seg[0].B = dy; a.seg[0].ldb = d; a.seg[0].K = T;
    a.a_kcontig = false; a.b_kcontig = false;
    c.M = d; c.N = 2 * f; c.nseg = 1;
    c.seg[0].A = sn; c.seg[0].lda = d; c.seg[0].B = dgu; c.seg[0].ldb = 2 * f; c.seg[0].K = T;
    c.a_kcontig = false; c.b_kcontig = false;
    if (h->tn) {
        const int64_t Tp = h->Tp;
        char* hT = h->scratch + h->s_hT;
        char* nT = h->scratch + h->s_nT;
        char* dyT = h->scratch + h->s_dyT;
        char* dguT = h->scratch + h->s_dguT;
        auto tr = [&](const void* src, int64_t cols, void* dst, const float* rs = nullptr, const float* cs = nullptr,
                      const void* src2 = nullptr) {
            return timed(h, PPS_K_COPY, 0.0, (src2 ? 3.0 : 2.0) * T * cols * 2, [&] {
                return pps::transpose_bf16(src, T, cols, cols, dst, Tp, 0, 0, h->stream, rs, cs, src2);
            });
        };
        // n = (x r) gamma and (unless the dh epilogue wrote them: have_nh)
        // h = silu(g) u come T-contiguous straight from the stash; dg|du
        // likewise from the dh epilogue, from the entry (split, full tiles)
        // or by a copy
        const bool entry_dguT = h->split && hT_fused(h);
        PPS_TRY(tr(xb, d, nT, rb, gamma));
        if (!have_nh) PPS_TRY(tr(ab + h->lay.g[b], f, hT, nullptr, nullptr, ab + h->lay.u[b]));
        PPS_TRY(tr(dy, d, dyT));
        if (!have_nh && !entry_dguT) PPS_TRY(tr(dgu, 2 * f, dguT));
        a.seg[0].A = hT; a.seg[0].lda = Tp; a.seg[0].B = dyT; a.seg[0].ldb = Tp;
        c.seg[0].A = nT; c.seg[0].lda = Tp; c.seg[0].B = entry_dguT ? dgu : dguT; c.seg[0].ldb = Tp;
        a.a_kcontig = a.b_kcontig = c.a_kcontig = c.b_kcontig = true;
    }
    a.epi = pps::EPI_ACC_F32;
    a.e.out0 = dWd; a.e.ld0 = d; a.e.nsplit = d;
    PPS_TRY(timed(h, PPS_K_WGRAD_DOWN, gemm_flops(f, d, T), 0.0, [&] { return pps::gemm(dt, a, h->stream); }));
    c.epi = pps::EPI_ACC_F32;
    c.e.out0 = dWg; c.e.ld0 = f; c.e.out1 = dWu; c.e.ld1 = f; c.e.nsplit = f;
    if (h->tn) {
        // bf16: dW_g and dW_u in one launch over the 2 ffn columns of dg|du
        // (split at ffn) when that saves a partly filled wave of tiles (one
        // tile per CU at a time), else one launch each: with whole waves
        // either way, two launches measured faster.
        const int64_t t1 = pps::gemm_bf16_tiles(d, f), t2 = pps::gemm_bf16_tiles(d, 2 * f);
        auto waves = [&](int64_t t) { return (t + h->ncu - 1) / h->ncu; };
        if (waves(t2) >= 2 * waves(t1)) {
            c.N = f;
            c.e.out1 = nullptr; c.e.ld1 = 0;
            PPS_TRY(timed(h, PPS_K_WGRAD_GATEUP, gemm_flops(d, f, T), 0.0, [&] { return pps::gemm(dt, c, h->stream); }));
            c.seg[0].B = static_cast<const char*>(c.seg[0].B) + (size_t)f * h->Tp * 2;
            c.e.out0 = dWu;
            PPS_TRY(timed(h, PPS_K_WGRAD_GATEUP, gemm_flops(d, f, T), 0.0, [&] { return pps::gemm(dt, c, h->stream); }));
            return PPS_OK;
        }
    }
    PPS_TRY(timed(h, PPS_K_WGRAD_GATEUP, gemm_flops(d, 2.0 * f, T), 0.0, [&] { return pps::gemm(dt, c, h->stream); }));
    return PPS_OK;
}

int swiglu_backward(pps_stage* h, int slot, int chunk, const void* dy_in, void* dx_out) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d, f = D.ffn;
    const int dt = D.dtype, es = h->es;
    char* sb = slot_base(h, slot);
    char* dxbuf[2] = {h->scratch + h->s_dxa, h->scratch + h->s_dxb};
    float* dn = reinterpret_cast<float*>(h->scratch + h->s_dn);
    float* part = reinterpret_cast<float*>(h->scratch + h->s_part);
    if (h->ac) {
        int rc = swiglu_forward(h, slot, chunk, nullptr, nullptr, true);
        if (rc != PPS_OK) return rc;
    }
    char* ab = acts(h, slot);
    if (h->split) {
        // Keep this micro-batch's output gradient for the deferred W.
        char* dst = sb + h->lay.dy[D.L - 1];
        PPS_TRY(timed(h, PPS_K_COPY, 0.0, 2.0 * T * d * es, [&] { return pps::copy_bytes(dst, dy_in, T * d * es, h->stream); }));
    }
    for (int b = D.L - 1; b >= 0; --b) {
        const void* const* wb = h->w.data() + (size_t)(chunk * D.L + b) * 4;
        const float* gamma = static_cast<const float*>(wb[3]);
        const size_t gi = (size_t)(chunk * D.L + b) * 4;
        float* dgam = h->grads + h->goff[gi + 3];
        const void* dy;
        void* dx;
        char* dgu;
        if (h->split) {
            dy = sb + h->lay.dy[b];
            dx = b == 0 ? dx_out : static_cast<void*>(sb + h->lay.dy[b - 1]);
            // full tiles: the entry keeps dg|du T-contiguous (written by the
            // dh epilogue below) and dn reads the row-major copy in scratch
            dgu = hT_fused(h) ? h->scratch + h->s_dgu : sb + h->lay.dgu[b];
        } else {
            dy = b == D.L - 1 ? dy_in : static_cast<const void*>(dxbuf[(b + 1) & 1]);
            dx = b == 0 ? dx_out : static_cast<void*>(dxbuf[b & 1]);
            dgu = h->scratch + h->s_dgu;
        }
        // dh = dy Wd^T, then dg, du from the stashed g, u (and, for this
        // block's weight gradient right after, h = silu(g) u).
        char* sn = h->split ? nullptr : h->scratch + h->s_n;
        char* sh = h->split ? nullptr : h->scratch + h->s_h;
        GemmArgs a;
        a.M = T; a.N = f; a.nseg = 1;
        a.seg[0].A = dy; a.seg[0].lda = d; a.seg[0].K = d;
        a.seg[0].B = wb[2]; a.seg[0].ldb = d;
        a.a_kcontig = true; a.b_kcontig = true;
        a.epi = pps::EPI_SWIGLU_BWD;
        a.e.in0 = ab + h->lay.g[b]; a.e.in1 = ab + h->lay.u[b]; a.e.ldi0 = f;
        a.e.out0 = dgu; a.e.ld0 = 2 * f; a.e.nsplit = f; a.e.out2 = sh;
        if (h->tn && sh) {
            // the weight gradients read h and dg|du T-contiguous: the epilogue
            // writes them so when its tiles are full; otherwise h and n are
            // recomputed at dW and h, dg|du copied
            const bool fused = hT_fused(h);
            a.e.out2 = fused ? h->scratch + h->s_hT : nullptr;
            a.e.out3 = fused ? h->scratch + h->s_dguT : nullptr;
            a.e.ld2 = h->Tp;
        } else if (h->tn && h->split && hT_fused(h)) {
            a.e.out3 = sb + h->lay.dgu[b];
            a.e.ld2 = h->Tp;
        }
        PPS_TRY(timed(h, PPS_K_DH, gemm_flops(T, f, d), 0.0, [&] { return pps::gemm(dt, a, h->stream); }));
        // dn = dg Wg^T + du Wu^T (one accumulator, K = 2 ffn).
        GemmArgs c;
        c.M = T; c.N = d; c.nseg = 2;
        c.seg[0].A = dgu; c.seg[0].lda = 2 * f; c.seg[0].K = f; c.seg[0].B = wb[0]; c.seg[0].ldb = f;
        c.seg[1].A = dgu + f * es; c.seg[1].lda = 2 * f; c.seg[1].K = f; c.seg[1].B = wb[1]; c.seg[1].ldb = f;
        c.a_kcontig = true; c.b_kcontig = true;
        c.epi = pps::EPI_STORE_F32;
        c.e.out0 = dn; c.e.ld0 = d;
        PPS_TRY(timed(h, PPS_K_DN, gemm_flops(T, d, 2.0 * f), 0.0, [&] { return pps::gemm(dt, c, h->stream); }));
        // RMSNorm backward + residual, dgamma partials, then their fixed-order
        // sum; fp32 without the split, also n for this block's weight gradient.
        int nrows = 0;
        // n row-major only for the fp32 weight gradients (bf16 takes nT from x)
        char* n_out = h->tn ? nullptr : sn;
        PPS_TRY(timed(h, PPS_K_RMSNORM_BWD, 0.0,
                      (double)T * d * 4 + (n_out ? 4.0 : 3.0) * T * d * es + T * 4.0 + d * 4.0 +
                          (double)pps::rmsnorm_bwd_partial_rows(T) * d * 4, [&] {
                          return pps::rmsnorm_bwd(dt, dn, act_x(h, slot, b), reinterpret_cast<const float*>(ab + h->lay.r[b]),
                                                  gamma, dy, T, d, dx, part, &nrows, n_out, h->stream);
                      }));
        const int prow = pps::rmsnorm_bwd_partial_rows(T);
        PPS_TRY(timed(h, PPS_K_DGAMMA, 0.0, (double)prow * d * 4 + 8.0 * d, [&] {
            return pps::column_reduce_acc(part, T > 0 ? prow : 0, d, dgam, h->stream);
        }));
        if (!h->split) {
            int rc = swiglu_weight(h, slot, chunk, b, dy, dgu, !h->tn || hT_fused(h));
            if (rc != PPS_OK) return rc;
        }
    }
    return PPS_OK;
}

int swiglu_backward_weight(pps_stage* h, int slot, int chunk) {
    char* sb = slot_base(h, slot);
    for (int b = h->d.L - 1; b >= 0; --b) {
        int rc = swiglu_weight(h, slot, chunk, b, sb + h->lay.dy[b], sb + h->lay.dgu[b], false);
        if (rc != PPS_OK) return rc;
    }
    return PPS_OK;
}

// ---- toy block sequences (fp32) ---------------------------------------------

int toy_forward(pps_stage* h, int slot, int chunk, const void* x_in, void* y_out) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d;
    char* sb = slot_base(h, slot);
    PPS_TRY(timed(h, PPS_K_COPY, 0.0, 2.0 * T * d * 4, [&] { return pps::copy_bytes(sb + h->lay.x[0], x_in, T * d * 4, h->stream); }));
    for (int b = 0; b < D.L; ++b) {
        const void* const* wb = h->w.data() + (size_t)(chunk * D.L + b) * 2;
        GemmArgs a;
        a.M = T; a.N = d; a.nseg = 1;
        a.seg[0].A = sb + h->lay.x[b]; a.seg[0].lda = d; a.seg[0].K = d;
        a.seg[0].B = wb[0]; a.seg[0].ldb = d;
        a.a_kcontig = true; a.b_kcontig = false;
        a.epi = pps::EPI_BIAS_GELU;
        a.e.bias = static_cast<const float*>(wb[1]);
        a.e.out0 = sb + h->lay.z[b]; a.e.ld0 = d;
        a.e.out1 = b == D.L - 1 ? y_out : static_cast<void*>(sb + h->lay.x[b + 1]); a.e.ld1 = d;
        PPS_TRY(timed(h, PPS_K_TOY_FWD, gemm_flops(T, d, d), 0.0, [&] { return pps::gemm(PPS_DTYPE_FP32, a, h->stream); }));
    }
    return PPS_OK;
}

int toy_weight(pps_stage* h, int slot, int chunk, int b, const float* dz) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d;
    char* sb = slot_base(h, slot);
    const size_t gi = (size_t)(chunk * D.L + b) * 4;
    GemmArgs a;
    a.M = d; a.N = d; a.nseg = 1;
    a.seg[0].A = sb + h->lay.x[b]; a.seg[0].lda = d; a.seg[0].K = T;
    a.seg[0].B = dz; a.seg[0].ldb = d;
    a.a_kcontig = false; a.b_kcontig = false;
    a.epi = pps::EPI_ACC_F32;
    a.e.out0 = h->grads + h->goff[gi + 0]; a.e.ld0 = d; a.e.nsplit = d;
    PPS_TRY(timed(h, PPS_K_TOY_DW, gemm_flops(d, d, T), 0.0, [&] { return pps::gemm(PPS_DTYPE_FP32, a, h->stream); }));
    PPS_TRY(timed(h, PPS_K_TOY_DB, 0.0, (double)T * d * 4 + 8.0 * d, [&] {
        return pps::colsum_acc(dz, T, d, h->grads + h->goff[gi + 1], h->stream);
    }));
    return PPS_OK;
}

int toy_backward(pps_stage* h, int slot, int chunk, const void* dy_in, void* dx_out) {
    const pps_stage_desc& D = h->d;
    const int64_t T = D.T, d = D.d;
    char* sb = slot_base(h, slot);
    char* dxbuf[2] = {h->scratch + h->s_dxa, h->scratch + h->s_dxb};
    for (int b = D.L - 1; b >= 0; --b) {
        const void* const* wb = h->w.data() + (size_t)(chunk * D.L + b) * 2;
        const float* dy = static_cast<const float*>(b == D.L - 1 ? dy_in : static_cast<const void*>(dxbuf[(b + 1) & 1]));
        void* dx = b == 0 ? dx_out : static_cast<void*>(dxbuf[b & 1]);
        float* dz = reinterpret_cast<float*>(h->split ? sb + h->lay.dz[b] : h->scratch + h->s_dz);
        PPS_TRY(timed(h, PPS_K_TOY_DZ, 0.0, 3.0 * T * d * 4, [&] {
            return pps::gelu_bwd(dy, reinterpret_cast<const float*>(sb + h->lay.z[b]), T * d, dz, h->stream);
        }));
        GemmArgs a;
        a.M = T; a.N = d; a.nseg = 1;
        a.seg[0].A = dz; a.seg[0].lda = d; a.seg[0].K = d;
        a.seg[0].B = wb[0]; a.seg[0].ldb = d;
        a.a_kcontig = true; a.b_kcontig = true;
        a.epi = pps::EPI_STORE;
        a.e.out0 = dx; a.e.ld0 = d;
        PPS_TRY(timed(h, PPS_K_TOY_DX, gemm_flops(T, d, d), 0.0, [&] { return pps::gemm(PPS_DTYPE_FP32, a, h->stream); }));
        if (!h->split) {
            int rc = toy_weight(h, slot, chunk, b, dz);
            if (rc != PPS_OK) return rc;
        }
    }
    return PPS_OK;
}

int toy_backward_weight(pps_stage* h, int slot, int chunk) {
    char* sb = slot_base(h, slot);
    for (int b = h->d.L - 1; b >= 0; --b) {
        int rc = toy_weight(h, slot, chunk, b, reinterpret_cast<const float*>(sb + h->lay.dz[b]));
        if (rc != PPS_OK) return rc;
    }
    return PPS_OK;
}

}  // namespace

// ---------------------------------------------------------------------------
// C ABI
// ---------------------------------------------------------------------------

namespace {

// pps_stage_create and pps_stage_create_noalloc: the same handle; `noalloc`
// takes the device memory from the library's fixed array instead of hipMalloc.
int create_stage(const pps_stage_desc* desc, pps_stage** out, bool noalloc) {
    if (!out) return PPS_EINVAL;
    int rc = validate_desc(desc);
    if (rc != PPS_OK) return rc;
    if (noalloc && (desc->flags & PPS_FLAG_PROFILE)) return PPS_EINVAL;
    pps_stage* h = new (std::nothrow) pps_stage();
    if (!h) return PPS_ENOMEM;
    h->d = *desc;
    h->bookkeeping = (desc->flags & PPS_FLAG_BOOKKEEPING_ONLY) != 0;
    h->profile = !h->bookkeeping && (desc->flags & PPS_FLAG_PROFILE) != 0;
    h->stride = std::max(1, desc->profile_stride);
    h->swiglu = desc->block_type == PPS_BLOCK_SWIGLU;
    h->nw = h->swiglu ? 4 : 2;
    h->es = desc->dtype == PPS_DTYPE_BF16 ? 2 : 4;
    h->split = desc->kind == PPS_ZB1P || desc->kind == PPS_ZB2P;
    h->ac = (desc->flags & PPS_FLAG_RECOMPUTE) != 0;
    h->stream = static_cast<hipStream_t>(desc->stream);
    h->d.weights = nullptr;
    if (!h->bookkeeping) h->w.assign(desc->weights, desc->weights + (size_t)desc->v * desc->L * h->nw);

    rc = pps::build_schedule(desc->P, desc->M, desc->k, desc->v, desc->kind, h->sched);
    if (rc != PPS_OK) { release(h); return rc; }
    int peak = 0;
    for (const pps_op& o : h->sched) {
        peak = std::max(peak, o.inflight_after);
        if (o.op == PPS_OP_F) { h->fseq.push_back({o.mb, o.chunk}); h->tf.push_back(o.t_start); }
        else if (o.op == PPS_OP_B) { h->bseq.push_back({o.mb, o.chunk}); h->tb.push_back(o.t_start); }
        else { h->wseq.push_back({o.mb, o.chunk}); h->tw.push_back(o.t_start); }
    }
    h->S = peak;
    h->status.assign((size_t)desc->M * desc->v, ST_NONE);
    h->slot_of.assign((size_t)desc->M * desc->v, -1);
    h->slot_used.assign(h->S, 0);

    h->tn = h->swiglu && desc->dtype == PPS_DTYPE_BF16;
    h->lay = make_layout(*desc, h->swiglu, h->split, h->es);
    const size_t T = (size_t)desc->T, dm = (size_t)desc->d, f = (size_t)desc->ffn;
    size_t off = 0;
    auto take = [&](size_t& o, size_t bytes) { o = off; off += align256(bytes); };
    if (h->ac) {
        // the block tensors move to the recompute area; a slot keeps x alone
        take(h->s_rc, h->lay.fwd_bytes);
        h->lay.fwd_bytes = align256(T * dm * h->es);
        h->lay.slot_bytes = std::max<size_t>(h->lay.fwd_bytes, 256);
    }
    if (h->swiglu) {
        take(h->s_n, T * dm * h->es);
        take(h->s_h, T * f * h->es);
        // the split keeps dg|du in the entry; on full tiles the entry holds
        // it T-contiguous and dn reads a row-major copy from here
        take(h->s_dgu, h->split && !hT_fused(h) ? 256 : T * 2 * f * h->es);
        take(h->s_dn, T * dm * 4);
        take(h->s_part, (size_t)pps::rmsnorm_bwd_partial_rows((int64_t)T) * dm * 4);
        if (h->tn) {
            h->Tp = (desc->T + 7) / 8 * 8;
            const size_t Tp = (size_t)h->Tp;
            take(h->s_hT, f * Tp * 2);
            take(h->s_nT, dm * Tp * 2);
            take(h->s_dyT, dm * Tp * 2);
            take(h->s_dguT, 2 * f * Tp * 2);
            size_t w = 0;
            for (int i = 0; i < desc->v * desc->L; ++i) {
                h->wgu_off.push_back(w);
                w += align256((size_t)pps::swiglu_b_rows(desc->ffn) * dm * 2);
                h->wd_off.push_back(w);
                w += align256(dm * f * 2);
            }
            h->wcopy_bytes = w;
        }
    } else {
        take(h->s_dz, T * dm * 4);
    }
    take(h->s_dxa, T * dm * h->es);
    take(h->s_dxb, T * dm * h->es);
    h->scratch_bytes = std::max<size_t>(off, 256);

    const int nblk = desc->v * desc->L;
    size_t goff = 0;
    for (int i = 0; i < nblk; ++i) {
        if (h->swiglu) {
            h->goff.push_back(goff); goff += dm * f;
            h->goff.push_back(goff); goff += dm * f;
            h->goff.push_back(goff); goff += f * dm;
            h->goff.push_back(goff); goff += dm;
        } else {
            h->goff.push_back(goff); goff += dm * dm;
            h->goff.push_back(goff); goff += dm;
            h->goff.push_back(goff);
            h->goff.push_back(goff);
        }
        goff = (goff + 63) & ~size_t(63);
    }
    h->grad_bytes = goff * sizeof(float);

    h->st.n_slots = h->S;
    h->st.slot_bytes = (int64_t)h->lay.slot_bytes;
    h->st.pool_bytes = (int64_t)h->lay.slot_bytes * h->S;
    h->st.scratch_bytes = (int64_t)(h->scratch_bytes + h->wcopy_bytes);
    h->st.grad_bytes = (int64_t)h->grad_bytes;

    const size_t pool_alloc = std::max<size_t>(h->lay.slot_bytes * h->S, 256);
    const size_t grad_alloc = std::max<size_t>(h->grad_bytes, 256);
    if (!h->bookkeeping && noalloc) {
        const size_t need = align256(pool_alloc) + align256(h->scratch_bytes) + align256(grad_alloc) +
                            align256(h->wcopy_bytes);
        if (need > (size_t)PPS_NOALLOC_MAX_BYTES) { release(h); return PPS_ETOOBIG; }
        char* base = nullptr;
        rc = pps::noalloc_scratch(&base);
        if (rc != PPS_OK) { release(h); return rc; }
        h->noalloc = true;
        size_t o = 0;
        h->pool = base + o; o += align256(pool_alloc);
        h->scratch = base + o; o += align256(h->scratch_bytes);
        h->grads = reinterpret_cast<float*>(base + o); o += align256(grad_alloc);
        h->wcopy = h->wcopy_bytes ? base + o : nullptr;
    }
    if (!h->bookkeeping) {
        int dev = 0, ncu = 0;
        if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            ncu < 1) {
            (void)hipGetLastError();
            release(h);
            return PPS_EHIP;
        }
        h->ncu = ncu;
        if (!noalloc &&
            (hipMalloc(reinterpret_cast<void**>(&h->pool), pool_alloc) != hipSuccess ||
             hipMalloc(reinterpret_cast<void**>(&h->scratch), h->scratch_bytes) != hipSuccess ||
             hipMalloc(reinterpret_cast<void**>(&h->grads), grad_alloc) != hipSuccess ||
             (h->wcopy_bytes && hipMalloc(reinterpret_cast<void**>(&h->wcopy), h->wcopy_bytes) != hipSuccess))) {
            (void)hipGetLastError();
            release(h);
            return PPS_ENOMEM;
        }
        if (pps::fill_zero(h->grads, (int64_t)h->grad_bytes, h->stream) != hipSuccess) { release(h); return PPS_EHIP; }
        // hT's padding columns [T, Tp) are read by the K tail of dW_d and never written
        if (h->tn && pps::fill_zero(h->scratch + h->s_hT, (int64_t)desc->ffn * h->Tp * 2, h->stream) != hipSuccess) {
            release(h);
            return PPS_EHIP;
        }
        // the padding rows of the interleaved gate/up copy must read as zero
        if (h->wcopy && pps::fill_zero(h->wcopy, (int64_t)h->wcopy_bytes, h->stream) != hipSuccess) { release(h); return PPS_EHIP; }
        if (h->profile) {
            const int cap = desc->profile_capacity;
            h->ev.assign((size_t)cap * 2, nullptr);
            h->ev_kernel.assign(cap, 0);
            h->ev_flops.assign(cap, 0.0);
            h->ev_bytes.assign(cap, 0.0);
            for (auto& e : h->ev)
                if (hipEventCreate(&e) != hipSuccess) { release(h); return PPS_EHIP; }
        }
        if (noalloc) {
            if (hipGetLastError() != hipSuccess) { release(h); return PPS_EHIP; }
        } else if (hipStreamSynchronize(h->stream) != hipSuccess) {
            release(h);
            return PPS_EHIP;
        }
    }
    *out = h;
    return PPS_OK;
}

}  // namespace

extern "C" int pps_stage_create(const pps_stage_desc* desc, pps_stage** out) {
    return create_stage(desc, out, false);
}

extern "C" int pps_stage_create_noalloc(const pps_stage_desc* desc, pps_stage** out) {
    return create_stage(desc, out, true);
}

// Caller buffers must be 16-byte aligned (the kernels move 16-byte pieces):
// checked before anything is enqueued.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

extern "C" int pps_stage_forward(pps_stage* h, int mb, int chunk, const void* x_in, void* y_out) {
    if (!h) return PPS_EINVAL;
    if (h->failed) return PPS_EHIP;
    if (mb < 0 || mb >= h->d.M || chunk < 0 || chunk >= h->d.v) return PPS_EINVAL;
    if (!h->bookkeeping && (!x_in || !y_out || !aligned16(x_in) || !aligned16(y_out))) return PPS_EINVAL;
    // A call after a completed pass starts the next one.
    const bool next_pass = pass_done(h);
    const size_t fpos = next_pass ? 0 : h->fpos;
    if (fpos >= h->fseq.size() || h->fseq[fpos] != std::make_pair(mb, chunk)) return PPS_EORDER;
    int slot = 0;
    while (slot < h->S && h->slot_used[slot]) ++slot;
    if (slot == h->S) return PPS_EFULL;
    if (next_pass) maybe_new_pass(h);

    if (!h->bookkeeping) {
        if (h->tn && h->fpos == 0) {
            int rc = refresh_weight_copies(h);
            if (rc != PPS_OK) return rc;
        }
        int rc = h->swiglu ? swiglu_forward(h, slot, chunk, x_in, y_out) : toy_forward(h, slot, chunk, x_in, y_out);
        if (rc != PPS_OK) return rc;
    }
    const size_t key = (size_t)chunk * h->d.M + mb;
    h->slot_used[slot] = 1;
    h->slot_of[key] = slot;
    h->status[key] = ST_F;
    ++h->live;
    h->live_bytes += (int64_t)h->lay.fwd_bytes;
    log_op(h, PPS_OP_F, mb, chunk, slot, h->tf[h->fpos]);
    ++h->fpos;
    ++h->st.n_forward;
    count_pass(h);
    return PPS_OK;
}

extern "C" int pps_stage_backward(pps_stage* h, int mb, int chunk, const void* dy_in, void* dx_out) {
    if (!h) return PPS_EINVAL;
    if (h->failed) return PPS_EHIP;
    if (mb < 0 || mb >= h->d.M || chunk < 0 || chunk >= h->d.v) return PPS_EINVAL;
    if (!h->bookkeeping && (!dy_in || !dx_out || !aligned16(dy_in) || !aligned16(dx_out))) return PPS_EINVAL;
    // dy_in is read again after dx_out is written (the weight gradients of the
    // first block read it), so the two [T, d] buffers must not overlap
    if (!h->bookkeeping && h->d.T > 0) {
        const uintptr_t a = reinterpret_cast<uintptr_t>(dy_in), b = reinterpret_cast<uintptr_t>(dx_out);
        const uintptr_t n = (uintptr_t)h->d.T * (uintptr_t)h->d.d * (uintptr_t)h->es;
        if (a < b + n && b < a + n) return PPS_EINVAL;
    }
    const size_t key = (size_t)chunk * h->d.M + mb;
    // after a completed pass nothing of the next one is saved yet
    if (pass_done(h) || h->status[key] == ST_NONE) return PPS_ENOENT;
    if (h->status[key] != ST_F) return PPS_ESTATE;
    if (h->bpos >= h->bseq.size() || h->bseq[h->bpos] != std::make_pair(mb, chunk)) return PPS_EORDER;
    const int slot = h->slot_of[key];

    if (!h->bookkeeping) {
        int rc = h->swiglu ? swiglu_backward(h, slot, chunk, dy_in, dx_out) : toy_backward(h, slot, chunk, dy_in, dx_out);
        if (rc != PPS_OK) return rc;
    }
    if (h->split) {
        h->status[key] = ST_B;
        h->live_bytes += (int64_t)h->lay.split_bytes;
    } else {
        h->status[key] = ST_W;
        h->slot_used[slot] = 0;
        --h->live;
        h->live_bytes -= (int64_t)h->lay.fwd_bytes;
    }
    log_op(h, PPS_OP_B, mb, chunk, slot, h->tb[h->bpos]);
    ++h->bpos;
    ++h->st.n_backward;
    count_pass(h);
    return PPS_OK;
}

extern "C" int pps_stage_backward_weight(pps_stage* h, int mb, int chunk) {
    if (!h) return PPS_EINVAL;
    if (h->failed) return PPS_EHIP;
    if (mb < 0 || mb >= h->d.M || chunk < 0 || chunk >= h->d.v) return PPS_EINVAL;
    if (!h->split) return PPS_ESTATE;
    const size_t key = (size_t)chunk * h->d.M + mb;
    if (h->status[key] != ST_B) return PPS_ESTATE;
    if (h->wpos >= h->wseq.size() || h->wseq[h->wpos] != std::make_pair(mb, chunk)) return PPS_EORDER;
    const int slot = h->slot_of[key];
    if (!h->bookkeeping) {
        int rc = h->swiglu ? swiglu_backward_weight(h, slot, chunk) : toy_backward_weight(h, slot, chunk);
        if (rc != PPS_OK) return rc;
    }
    h->status[key] = ST_W;
    h->slot_used[slot] = 0;
    --h->live;
    h->live_bytes -= (int64_t)(h->lay.fwd_bytes + h->lay.split_bytes);
    log_op(h, PPS_OP_W, mb, chunk, slot, h->tw[h->wpos]);
    ++h->wpos;
    ++h->st.n_backward_weight;
    count_pass(h);
    return PPS_OK;
}

extern "C" int pps_stage_zero_grad(pps_stage* h) {
    if (!h) return PPS_EINVAL;
    if (h->failed) return PPS_EHIP;
    if (h->bookkeeping) return PPS_OK;
    if (pps::fill_zero(h->grads, (int64_t)h->grad_bytes, h->stream) != hipSuccess) { h->failed = true; return PPS_EHIP; }
    return PPS_OK;
}

extern "C" int pps_stage_get_grad(const pps_stage* h, int chunk, int block, int which, const float** dptr) {
    if (!h || !dptr || h->bookkeeping) return PPS_EINVAL;
    if (chunk < 0 || chunk >= h->d.v || block < 0 || block >= h->d.L) return PPS_EINVAL;
    if (which < 0 || which >= (h->swiglu ? 4 : 2)) return PPS_EINVAL;
    *dptr = h->grads + h->goff[(size_t)(chunk * h->d.L + block) * 4 + which];
    return PPS_OK;
}

extern "C" int pps_stage_sync(pps_stage* h) {
    if (!h) return PPS_EINVAL;
    if (h->bookkeeping) return PPS_OK;
    if (hipStreamSynchronize(h->stream) != hipSuccess) { h->failed = true; return PPS_EHIP; }
    if (hipGetLastError() != hipSuccess) { h->failed = true; return PPS_EHIP; }
    return h->failed ? PPS_EHIP : PPS_OK;
}

extern "C" int pps_stage_get_stats(const pps_stage* h, pps_stats* out) {
    if (!h || !out) return PPS_EINVAL;
    *out = h->st;
    out->live_entries = h->live;
    out->live_bytes = h->live_bytes;
    return PPS_OK;
}

extern "C" int pps_stage_get_oplog(const pps_stage* h, pps_op* ops, int cap, int* n) {
    if (!h || !n || cap < 0 || (cap > 0 && !ops)) return PPS_EINVAL;
    *n = (int)h->oplog.size();
    if (cap < *n) return PPS_EFULL;
    if (*n) std::memcpy(ops, h->oplog.data(), h->oplog.size() * sizeof(pps_op));
    return PPS_OK;
}

extern "C" int pps_stage_kernel_times(pps_stage* h, pps_kernel_time* out, int cap, int* n) {
    if (!h || !n || !h->profile || cap < 0 || (cap > 0 && !out)) return PPS_EINVAL;
    if (hipStreamSynchronize(h->stream) != hipSuccess) { h->failed = true; return PPS_EHIP; }
    for (int i = 0; i < h->ev_used; ++i) {
        float ms = 0.0f;
        if (hipEventElapsedTime(&ms, h->ev[2 * i], h->ev[2 * i + 1]) != hipSuccess) { h->failed = true; return PPS_EHIP; }
        const int k = h->ev_kernel[i];
        h->kt_ms[k] += ms;
        h->kt_flops[k] += h->ev_flops[i];
        h->kt_bytes[k] += h->ev_bytes[i];
        ++h->kt_n[k];
    }
    h->ev_used = 0;
    int cnt = 0;
    for (int k = 0; k < PPS_K_COUNT; ++k)
        if (h->kt_calls[k]) ++cnt;
    *n = cnt;
    if (cap < cnt) return PPS_EFULL;
    int j = 0;
    for (int k = 0; k < PPS_K_COUNT; ++k) {
        if (!h->kt_calls[k]) continue;
        out[j].kernel = k;
        out[j].reserved = 0;
        out[j].launches = h->kt_calls[k];
        out[j].timed = h->kt_n[k];
        out[j].total_ms = h->kt_ms[k];
        out[j].flops = h->kt_flops[k];
        out[j].bytes = h->kt_bytes[k];
        ++j;
        h->kt_n[k] = h->kt_calls[k] = 0;
        h->kt_ms[k] = h->kt_flops[k] = h->kt_bytes[k] = 0.0;
    }
    return PPS_OK;
}

extern "C" const char* pps_kernel_name(int k) {
    static const char* names[PPS_K_COUNT] = {
        "rmsnorm_fwd", "gemm_gateup_swiglu", "gemm_down_residual", "gemm_dh_swiglu_bwd", "gemm_dn",
        "rmsnorm_bwd_residual", "dgamma_reduce", "prep_w", "gemm_wgrad_down", "gemm_wgrad_gateup",
        "copy", "toy_fwd", "toy_dz", "toy_dx", "toy_dw", "toy_db"};
    return (k >= 0 && k < PPS_K_COUNT) ? names[k] : "unknown";
}

extern "C" int pps_scale(void* dst, const void* src, int64_t n, float sc, int dtype, void* stream) {
    if (n < 0 || (n > 0 && (!dst || !src))) return PPS_EINVAL;
    if (dtype != PPS_DTYPE_BF16 && dtype != PPS_DTYPE_FP32) return PPS_EINVAL;
    return pps::scale(dtype, dst, src, n, sc, static_cast<hipStream_t>(stream)) == hipSuccess ? PPS_OK : PPS_EHIP;
}

extern "C" void pps_stage_destroy(pps_stage* h) {
    if (!h) return;
    if (!h->bookkeeping) (void)hipStreamSynchronize(h->stream);
    release(h);
}

extern "C" const char* pps_strerror(int s) {
    switch (s) {
        case PPS_OK: return "ok";
        case PPS_EINVAL: return "invalid argument";
        case PPS_EFULL: return "no room (op array too small or no free stash slot)";
        case PPS_EORDER: return "call is not the next one of its kind in the schedule";
        case PPS_ENOENT: return "no saved forward for this micro-batch";
        case PPS_ESTATE: return "wrong state for this call";
        case PPS_ENOMEM: return "device allocation failed";
        case PPS_EHIP: return "HIP runtime error";
        case PPS_ETOOBIG: return "stage needs more device memory than the no-alloc array holds";
        default: return "unknown status";
    }
}
