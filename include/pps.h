/*
 * pps.h -- C ABI of the MI355X (gfx950) 1F1B pipeline-stage executor.
 *
 * One handle = one pipeline stage (stage k of P) on one GPU: L residual
 * SwiGLU-MLP blocks per chunk (or the toy Linear+GELU block), run over M
 * micro-batches in the order of a pipeline schedule.  The calls follow the
 * stage interface the pages describe: a forward per micro-batch that saves
 * its activations, a backward per micro-batch that takes the oldest saved
 * entry, returns the input gradient for the previous stage and accumulates
 * the weight gradient, and (Zero-Bubble split) a deferred weight-gradient
 * call.
 *
 * Page legend used in the citations:
 *   [1F1B]        "2. 1F1B" (sgdbs.github.io AI_Infra notes)
 *   [GPipe->ZB]   "流水线并行：从 GPipe 到 1F1B 与 Zero Bubble" (dlog.com.cn)
 *   [Sched]       "流水线调度：GPipe、1F1B、交错与计算通信重叠" (xuujii.github.io)
 *   [Megatron-PP] "Megatron-LM 分布式训练（三）：流水线并行 PP 与 1F1B 调度"
 *
 * Conventions (all calls):
 *   - Every call returns an int status: PPS_OK (0) or a negative PPS_E*
 *     code.  Nothing is thrown across the ABI.  A call that fails
 *     validation leaves the handle unchanged and enqueues nothing.
 *   - Device pointers are plain addresses in the current HIP device's
 *     memory, 16-byte aligned at least.  bf16 tensors are raw uint16_t
 *     storage (bfloat16 bit patterns); fp32 tensors are float.
 *   - Activations are row-major [T, d] with one token per row; weights are
 *     row-major [in, out], so a layer computes Y = X W.
 *   - Work is enqueued asynchronously on the handle's stream; a handle is
 *     single-threaded and must not be used from two host threads at once.
 *   - pps_stage_zero_grad, pps_stage_forward, pps_stage_backward and
 *     pps_stage_backward_weight (profiling off) only launch kernels on the
 *     handle's stream: no allocation, memset, copy call or synchronisation,
 *     so a pass may be recorded into a HIP graph on that stream and replayed.
 *     The handle's host-side bookkeeping advances once, during recording.
 *   - Constraints: d % 8 == 0 and ffn % 8 == 0 (16-byte rows); d <= 16384;
 *     T >= 0 (T == 0 is accepted and computes nothing).
 */
#ifndef PPS_H
#define PPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ------------------------------------------------------ */
#define PPS_OK       0
#define PPS_EINVAL  (-1)  /* bad argument or unsupported combination          */
#define PPS_EFULL   (-2)  /* op array too small / no free stash slot            */
#define PPS_EORDER  (-3)  /* call is not the next one of its kind in the schedule */
#define PPS_ENOENT  (-4)  /* backward of a micro-batch with no saved forward     */
#define PPS_ESTATE  (-5)  /* wrong state: W without split mode, W before B, twice */
#define PPS_ENOMEM  (-6)  /* device allocation failed at create                 */
#define PPS_EHIP    (-7)  /* a HIP runtime call or kernel launch failed         */
#define PPS_ETOOBIG (-8)  /* pps_stage_create_noalloc: the stage needs more
                             device memory than PPS_NOALLOC_MAX_BYTES          */

/* Size of the library's fixed per-GPU device array used by
   pps_stage_create_noalloc (64 MiB). */
#define PPS_NOALLOC_MAX_BYTES (64ull << 20)

/* ---- ops and schedule kinds ---------------------------------------------- */
#define PPS_OP_F 0  /* forward                                              */
#define PPS_OP_B 1  /* backward (input gradient; also dW unless split)      */
#define PPS_OP_W 2  /* deferred weight gradient (Zero-Bubble split only)    */

#define PPS_GPIPE 0 /* all forwards, then all backwards in reverse order      */
#define PPS_1F1B  1 /* synchronous 1F1B; interleaved 1F1B when v > 1         */
#define PPS_ZB1P  2 /* 1F1B F/B order with the B/W split, budget P            */
#define PPS_ZB2P  3 /* 2(P-k)-1 warmup forwards, B/W split, budget 2P        */

/* One entry of a stage's op list (also the layout of the executor's op log). */
typedef struct pps_op {
    int32_t op;             /* PPS_OP_F / PPS_OP_B / PPS_OP_W                  */
    int32_t mb;             /* micro-batch index, 0-based                      */
    int32_t chunk;          /* virtual chunk (0 unless v > 1)                  */
    int32_t slot;           /* stash slot: lowest free index, taken at F,
                               released at B (at W when split)                 */
    int32_t inflight_after; /* live stash entries after this op                */
    int32_t t_start;        /* start time in the unit-cost simulation of all P
                               stages (every op costs one unit)                */
} pps_op;

/*
 * pps_make_schedule -- op list of stage k of a P-stage pipeline, M micro-batches.
 *
 * Host only, pure and deterministic; touches no device.
 *   kind PPS_1F1B, v == 1: warmup min(P-k, M) forwards, then M-(P-k) steady
 *     (B, F) pairs, then the remaining backwards; backward takes the oldest
 *     micro-batch ([1F1B §2.3, §3.2]; [Megatron-PP 三阶段] pop(0); the
 *     Megatron warmup of P-k-1 plus the first steady forward is this order).
 *   kind PPS_GPIPE: all M forwards, then backwards M-1..0 ([Sched §02]).
 *   kind PPS_1F1B, v > 1 (interleaved, [1F1B §6.1]): chunk c of device k is
 *     virtual stage c*P+k; micro-batches in groups of P per chunk; warmup
 *     min(2(P-k-1) + (v-1)P + 1, M v) forwards, then alternate B and F.
 *     Needs M % P == 0.
 *   kind PPS_ZB1P / PPS_ZB2P ([GPipe->ZB ZB1P 与 ZB2P]): the page limits
 *     the micro-batches a stage holds with their weight gradient not done
 *     to p (ZB1P) or 2p (ZB2P), p = P, on every stage.  F/B order: ZB1P the
 *     1F1B order; ZB2P warms up with min(2(P-k)-1, M) forwards (the slots
 *     before its first backward can start when F, B and W cost the same),
 *     then alternates B and F.  A W op is placed wherever the stage cannot
 *     run its next F/B in the unit-cost simulation (dependency not done, or
 *     an F that would exceed the budget, entries counted until W); leftover
 *     W ops drain oldest-first after the last B.  With M >= 2P-1, ZB2P
 *     leaves no idle slot between a stage's first and last op.  v must be 1.
 * Arguments: ops = caller-owned array of cap entries (may be NULL if cap==0).
 * Returns PPS_OK; PPS_EFULL if cap < *n_ops (nothing written past cap;
 * *n_ops is still set); PPS_EINVAL for P < 1, M < 1, k not in [0,P), v < 1,
 * v > 1 with M % P != 0, v > 1 with GPipe/ZB, n_ops == NULL, or a problem
 * too large to simulate (P*v*M > 2^24).
 */
int pps_make_schedule(int P, int M, int k, int v, int kind,
                      pps_op* ops, int cap, int* n_ops);

/*
 * pps_simulate_pipeline -- predicted timeline of all P stages running one
 * schedule kind with given per-op durations (any time unit).
 *
 * Host only, pure.  Each device runs its op list (as pps_make_schedule builds
 * it for that stage; the ZB kinds keep their unit-cost W placement) in order,
 * each op as soon as the device is free and its dependencies have ended
 * ([Sched §08]: an op waits for its device's previous op and for the results
 * it needs; [1F1B §4.3], [Sched §04]: the idle share of that timeline is the
 * bubble).  Durations: t_f = forward of one micro-batch (per chunk when
 * v > 1); t_b = its backward, including the weight gradient unless the kind
 * is split; t_w = the deferred weight-gradient op (ZB kinds; otherwise
 * unused).  Transfers between stages take no time.
 * Out: *makespan = end of the last op; *bubble = 1 - (busy time summed over
 * the P devices) / (P * makespan).
 * Returns PPS_OK; PPS_EINVAL for the shapes pps_make_schedule rejects, a
 * negative or non-finite duration, or a NULL output.
 */
int pps_simulate_pipeline(int P, int M, int v, int kind, double t_f, double t_b, double t_w,
                          double* makespan, double* bubble);

/* ---- stage handle -------------------------------------------------------- */
#define PPS_BLOCK_SWIGLU   0  /* RMSNorm -> gate/up -> SiLU-gate -> down -> +x   */
#define PPS_BLOCK_TOY_GELU 1  /* Linear(d->d) with bias, then exact GELU (fp32) */

#define PPS_DTYPE_BF16 0      /* bf16 storage, fp32 accumulation (MFMA)       */
#define PPS_DTYPE_FP32 1      /* fp32 storage and arithmetic                  */

#define PPS_FLAG_BOOKKEEPING_ONLY 1u /* validate calls and track the stash and
                                        op log only: no device memory, no
                                        kernels, pointers are not touched     */
#define PPS_FLAG_PROFILE          2u /* record HIP events around kernels (see
                                        profile_stride)                       */
/* Activation recompute ([GPipe→ZB "GPipe 2018年"]: keep only the stage
   boundary and redo each layer's forward when the backward reaches it;
   [1F1B §4.5]: still advised under 1F1B).  A stash entry is then the stage
   input x [T,d] alone, and pps_stage_backward first re-runs the chunk's
   forward from it into one library-owned area (the per-block x, r, g, u of
   a single micro-batch, shared by all backwards; the last block's output is
   not recomputed: no backward reads it).  Kernels and launch shapes are the
   forward's own, so every result is bit-identical to a run without the
   flag.  SwiGLU blocks with kind GPIPE or 1F1B only (a deferred W would
   need the recomputed tensors kept per micro-batch): PPS_EINVAL otherwise. */
#define PPS_FLAG_RECOMPUTE        4u

typedef struct pps_stage_desc {
    int32_t P, M, k, v, kind;   /* pipeline shape and schedule kind          */
    int32_t block_type;         /* PPS_BLOCK_*                               */
    int32_t dtype;              /* PPS_DTYPE_*                               */
    int32_t L;                  /* blocks per chunk                          */
    int64_t d;                  /* model dim                                 */
    int64_t ffn;                /* SwiGLU hidden dim (ignored for toy)       */
    int64_t T;                  /* tokens (rows) per micro-batch             */
    float   eps;                /* RMSNorm epsilon                           */
    uint32_t flags;             /* PPS_FLAG_*                                */
    int32_t profile_capacity;   /* max kernel launches timed (PROFILE only)  */
    int32_t profile_stride;     /* PROFILE only: time launches 0, s, 2s, ... of
                                   each kernel id (0 or 1: every launch); the
                                   events cost GPU time between kernels      */
    void*   stream;             /* hipStream_t; NULL = the null stream        */
    /* Caller-owned device weights, read-only, must outlive the handle and
       stay unchanged during a pass (first forward to last backward or W:
       bf16 forwards use library copies made at the pass's first forward,
       backwards read these buffers); changes between passes are used.
       Index [(chunk*L + block)*nw + w]:
         SwiGLU (nw=4): Wg [d,ffn], Wu [d,ffn], Wd [ffn,d] in the stage dtype;
                        gamma [d] fp32.
         toy    (nw=2): W [d,d] fp32, b [d] fp32.
       May be NULL with PPS_FLAG_BOOKKEEPING_ONLY. */
    const void* const* weights;
} pps_stage_desc;

typedef struct pps_stage pps_stage;

/*
 * pps_stage_create -- build the handle for stage desc->k.
 * Computes the stage's op list with pps_make_schedule, sizes the stash pool
 * to the schedule's peak live count (P-k for 1F1B; M for GPipe; P for
 * ZB1P and up to 2P for ZB2P) and allocates, once, on the current device:
 * the pool, scratch and the fp32 gradient buffers (library-owned, zeroed).
 * Nothing is allocated later.
 * Limits: P, M, v, L >= 1, 0 <= k < P, kind one of the PPS_* kinds,
 * P*v*M <= 2^24, v*L <= 2^20 (checked before anything is allocated);
 * d a multiple of 8 up to 16384, ffn a multiple of 8 up to 2^30, T up to
 * 2^24 rows, and a memory footprint (pool, scratch, gradients, weight
 * copies) that stays under 10^18 bytes; with bf16 SwiGLU
 * blocks every GEMM operand must stay under 2 GiB (T * 2ffn, T * d and
 * 2*ceil(ffn/32)*32 * d elements of 2 bytes, T rounded up to 8), since the
 * MFMA kernel addresses operands with 32-bit offsets.
 * Returns PPS_EINVAL (bad desc), PPS_ENOMEM, PPS_EHIP.  *out is set only
 * on success.
 */
int pps_stage_create(const pps_stage_desc* desc, pps_stage** out);

/*
 * pps_stage_create_noalloc -- pps_stage_create for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same desc, same handle, same calls
 * afterwards; the difference is where the handle's device memory lives: its
 * stash pool, scratch, fp32 gradients and weight copies are carved from one
 * fixed device array of PPS_NOALLOC_MAX_BYTES that the library holds on each
 * GPU until the process ends (looked up once per device; no hipMalloc,
 * hipFree or other allocating call).  The gradients and the padding the
 * kernels read are cleared with fill kernels enqueued on desc->stream; the
 * call does not synchronize.  Host bookkeeping uses ordinary host memory.
 * Every no-alloc handle on a GPU shares that GPU's array: only one may be in
 * use at a time (ops of two such handles that overlap on one GPU race, and a
 * new handle clears what the previous one left).  PPS_FLAG_PROFILE is
 * rejected (it creates HIP events).
 * Returns PPS_ETOOBIG if the stage needs more than PPS_NOALLOC_MAX_BYTES
 * (pool + scratch + gradients + weight copies, each rounded up to 256
 * bytes), otherwise what pps_stage_create returns.
 */
int pps_stage_create_noalloc(const pps_stage_desc* desc, pps_stage** out);

/*
 * pps_stage_forward -- forward of micro-batch mb (chunk) through the stage's
 * blocks ([1F1B §5.2]: forward, then save the activations in the stash).
 * x_in [T,d] and y_out [T,d] are caller device buffers in the stage dtype.
 * What the backward needs is copied into a stash slot, so x_in may be
 * reused once the stream has passed this op; y_out may be x_in itself (every
 * read of x_in precedes the last block's write of y_out on the stream).
 * Errors: PPS_EORDER if (mb, chunk) is not the schedule's next forward;
 * PPS_EFULL if no stash slot is free; PPS_EINVAL on NULL pointers or
 * pointers not 16-byte aligned (nothing is enqueued).
 */
int pps_stage_forward(pps_stage* h, int mb, int chunk, const void* x_in, void* y_out);

/*
 * pps_stage_backward -- backward of micro-batch mb ([1F1B §5.2]: pop the
 * saved activations, receive the output gradient, send the input gradient
 * upstream).  dy_in [T,d] is the gradient of this stage's output, dx_out
 * [T,d] receives the gradient of its input.  Unsplit schedules also
 * accumulate dW into the fp32 gradient buffers and free the slot; ZB
 * schedules compute only dX (and dgamma) and keep the slot for W
 * ([GPipe->ZB Zero Bubble]: B = G W^T now, W = X^T G later).
 * Errors: PPS_ENOENT if mb has no saved forward in the current pass (also
 * right after a completed pass); PPS_ESTATE if mb was already backwarded in
 * this pass; PPS_EORDER if it is not the schedule's next backward
 * (for 1F1B: the oldest saved entry); PPS_EINVAL on NULL pointers,
 * pointers not 16-byte aligned, or dy_in and dx_out overlapping (nothing is
 * enqueued).
 */
int pps_stage_backward(pps_stage* h, int mb, int chunk, const void* dy_in, void* dx_out);

/*
 * pps_stage_backward_weight -- deferred weight gradient of micro-batch mb
 * (ZB schedules only): accumulates dW in fp32, then frees the slot.
 * Errors: PPS_ESTATE if the schedule is not split, if B of mb has not run,
 * or if W of mb already ran; PPS_EORDER if it is not the schedule's next W.
 */
int pps_stage_backward_weight(pps_stage* h, int mb, int chunk);

/* Enqueue zeroing of every gradient buffer ([1F1B §5.2]: zero_grad after the
   step).  Call before the first op of a pass. */
int pps_stage_zero_grad(pps_stage* h);

/* Gradient buffer of (chunk, block): which = 0 dWg [d,ffn], 1 dWu [d,ffn],
   2 dWd [ffn,d], 3 dgamma [d] (SwiGLU); 0 dW [d,d], 1 db [d] (toy).  fp32,
   library-owned, valid until destroy.  Its contents are written by work on
   the handle's stream: read them on that stream, or after pps_stage_sync
   with the read ordered on the reader's own stream.  PPS_EINVAL out of range
   or with PPS_FLAG_BOOKKEEPING_ONLY. */
int pps_stage_get_grad(const pps_stage* h, int chunk, int block, int which, const float** dptr);

/* Wait for the handle's stream; surfaces asynchronous HIP errors as PPS_EHIP. */
int pps_stage_sync(pps_stage* h);

typedef struct pps_stats {
    int64_t n_slots;            /* stash slots in the pool                     */
    int64_t slot_bytes;         /* bytes per slot (largest entry)              */
    int64_t pool_bytes;         /* n_slots * slot_bytes                        */
    int64_t scratch_bytes;      /* library scratch                             */
    int64_t grad_bytes;         /* fp32 gradient buffers                       */
    int64_t live_entries;       /* entries currently held                      */
    int64_t live_bytes;         /* bytes those entries use                     */
    int64_t peak_live_entries;  /* since create                                */
    int64_t peak_live_bytes;    /* since create                                */
    int64_t n_forward, n_backward, n_backward_weight; /* accepted calls       */
    int64_t passes_completed;   /* full op lists executed                      */
} pps_stats;

int pps_stage_get_stats(const pps_stage* h, pps_stats* out);

/* The accepted calls of the current (or just completed) pass, in call order,
   with the slot each took and the live count after it; t_start is copied
   from the schedule entry the call matched.  PPS_EFULL if cap is too small
   (*n is set). */
int pps_stage_get_oplog(const pps_stage* h, pps_op* ops, int cap, int* n);

/* ---- kernel timing (PPS_FLAG_PROFILE) ------------------------------------ */
#define PPS_K_RMSNORM_FWD   0  /* r = rsqrt(mean x^2 + eps); n = x r gamma      */
#define PPS_K_GATEUP        1  /* g,u = n [Wg|Wu]; h = silu(g) u                */
#define PPS_K_DOWN          2  /* y = x + h Wd                                  */
#define PPS_K_DH            3  /* dh = dy Wd^T; dg, du (SwiGLU backward); h (bf16: h^T) */
#define PPS_K_DN            4  /* dn = dg Wg^T + du Wu^T                         */
#define PPS_K_RMSNORM_BWD   5  /* dx = dy + r a - r^3 x (a.x)/d; dgamma partials; n */
#define PPS_K_DGAMMA        6  /* dgamma += sum of partials                      */
#define PPS_K_PREP_W        7  /* n = x r gamma, h = silu(g) u again at W (fp32 split; bf16 makes them T-contiguous in the copies) */
#define PPS_K_WGRAD_DOWN    8  /* dWd += h^T dy                                  */
#define PPS_K_WGRAD_GATEUP  9  /* dWg += n^T dg, dWu += n^T du                   */
#define PPS_K_COPY         10  /* copies: into the stash; per-pass weight copies; T-contiguous n (from x r gamma), dy (and h from g, u, dg|du where the dh epilogue does not write them) for bf16 dW */
#define PPS_K_TOY_FWD      11  /* z = x W + b; y = GELU(z)                       */
#define PPS_K_TOY_DZ       12  /* dz = dy GELU'(z)                               */
#define PPS_K_TOY_DX       13  /* dx = dz W^T                                    */
#define PPS_K_TOY_DW       14  /* dW += x^T dz                                   */
#define PPS_K_TOY_DB       15  /* db += column sums of dz                        */
#define PPS_K_COUNT        16

typedef struct pps_kernel_time {
    int32_t kernel;      /* PPS_K_*                                          */
    int32_t reserved;
    int64_t launches;    /* launches since the previous call                 */
    int64_t timed;       /* of which timed (see profile_stride); may be 0    */
    double  total_ms;    /* sum of the timed launches' HIP-event durations   */
    double  flops;       /* algorithmic FLOPs summed over the timed launches */
    double  bytes;       /* algorithmic HBM bytes summed over the timed ones */
} pps_kernel_time;

/* Synchronizes the stream, folds the recorded event pairs into per-kernel
   totals, writes one entry per kernel id launched since the previous call,
   and resets the totals (the stride's phase carries on).  Average duration
   = total_ms / timed.  Launches past profile_capacity timed pairs since the
   previous call are counted, not timed.  PPS_EINVAL without
   PPS_FLAG_PROFILE. */
int pps_stage_kernel_times(pps_stage* h, pps_kernel_time* out, int cap, int* n);
const char* pps_kernel_name(int kernel);

/*
 * pps_scale -- dst[i] = src[i] * scale for n elements of the given dtype
 * (PPS_DTYPE_BF16: bf16 storage, product rounded to nearest even; FP32),
 * enqueued on `stream` (hipStream_t, NULL = null stream).  The last stage's
 * output gradient is the loss gradient divided by M ([1F1B §5.2]); the P-stage
 * emulation uses this call for that division.  dst may equal src.
 * PPS_EINVAL on NULL pointers with n > 0, n < 0 or an unknown dtype.
 */
int pps_scale(void* dst, const void* src, int64_t n, float scale, int dtype, void* stream);

void pps_stage_destroy(pps_stage* h);
const char* pps_strerror(int status);

#ifdef __cplusplus
}
#endif

#endif /* PPS_H */
