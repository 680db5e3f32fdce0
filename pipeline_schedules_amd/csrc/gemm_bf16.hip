// bf16 GEMM on the CDNA4 matrix cores (gfx950), fp32 accumulation.
//
// Layout: C[m,n] = sum_k A(m,k) B(n,k) with both operands K-contiguous
// ("TN"): A row-major [M, K] (stride lda), B [N, K] (ldb).  The forward reads
// per-pass K-contiguous copies of the weights; the weight-gradient GEMMs
// dW = X^T Y reduce over tokens and read T-contiguous activations and
// gradients (copies, or written so by the SwiGLU-backward epilogue).  The
// kernel tiles 256 x 256 x 64, takes both operands straight from memory into
// LDS (direct-to-LDS buffer loads, no register staging) and reads zeros
// outside an operand's extent, which pads ragged M, N and K tails.
//
// Kernel: 256 threads = 4 wavefronts in a 2 x 2 grid, one per SIMD,
// 128 x 128 per wavefront = 8 x 8 tiles of v_mfma_f32_16x16x32_bf16 (256
// fp32 accumulators per lane, in AGPRs).  LDS holds a ring of five 32 KB
// operand-tile slots, A of K tile t in slot 2t mod 5 and B in slot 2t+1 mod 5.
// Within a K step on tile t every fragment of tile t is read into registers
// by mid-step (the second K half under the first half's MFMAs); a mid-step
// barrier then frees tile t's slots.  Tile t+2's A is requested during the
// first half (into B(t-1)'s slot), its B during the second half (into A(t)'s
// slot), one request per few MFMAs, so each tile has at least a full step to
// arrive.  The step ends with vmcnt(16) (everything but tile t+2) and a
// barrier, after which tile t+1's first-half fragments are read under the
// last 16 MFMAs, in the order a0 b0 b1 .. b7 a1 .. a7 that the MFMAs consume
// them.  The MFMAs of a K half run over the 8 x 8 tiles in serpentine order
// (rows of j ascending, then descending), so every MFMA shares one operand
// with the one before it: at the chip's power limit the fewer operand bits
// that switch, the higher the clock.  LDS rows are 128 bytes; 16-byte
// chunk c of row r sits at position c ^ ((r >> 1) & 7), which keeps the
// direct-to-LDS writes and the fragment reads free of bank conflicts.
//
// Why this shape: the stage GEMMs run at the chip's power limit, so what
// counts is work per cycle and energy per FLOP.  A lone wavefront per SIMD
// reading 128 x 128 per K step needs a third fewer LDS reads than two
// wavefronts of 128 x 64, and the 16x16x32 MFMA moves half the accumulator
// data of the 32x32x16 one per FLOP.  A lone wavefront has no partner to
// cover its non-MFMA instructions, so the K loop is unrolled over the five
// ring phases: every slot offset is an immediate and the load masks for the
// K tail live in a separate tail loop, which leaves one M0 write per load and
// the LDS reads between the MFMAs.
//
// Workgroup -> tile mapping: the dispatcher places workgroup i on XCD i % 8;
// ids are remapped so each XCD gets a contiguous run of logical tiles, and
// logical tiles are ordered in groups of 8 (or 4) tile-rows so the tiles
// running on one XCD share A rows and B columns in that XCD's L2.
#include <algorithm>
#include <type_traits>

#include "epilogue.h"

namespace pps {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __amdgpu_buffer_rsrc_t rsrc_t;
#define LDS_AS __attribute__((address_space(3)))

constexpr int BM = 256, BN = 256, BK = 64;
constexpr int NTHREADS = 256;            // 4 wavefronts
constexpr int NQ = 8;                    // 1 KB load pieces per wavefront per operand tile
constexpr int ROWB = BK * 2;             // TN: 128 bytes per LDS row
constexpr int OPB = 256 * ROWB;          // 32 KB per operand tile
constexpr int NSLOT = 5;                 // operand-tile slots
constexpr int LDS_BYTES = NSLOT * OPB;   // 160 KB
constexpr uint32_t OOB = 0x80000000u;    // an offset past every operand extent

struct Seg {
    const uint16_t* A;
    const uint16_t* B;
    int64_t lda, ldb, K;
    uint32_t a_bytes, b_bytes;
};

struct Params {
    int64_t M, N, NB;      // NB = rows of B
    int tiles_m, tiles_n, nseg, swiglu;
    int group_m;           // tile rows per group of the workgroup order (4 or 8)
    Seg seg[2];
    EpiArgs e;
};

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn) {
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int per = (nwg + 7) >> 3;
    const int tall = (nwg & 7) ? (nwg & 7) : 8;
    const int xcd = bid & 7, local = bid >> 3;
    const int lin = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
    const int width = p.group_m * p.tiles_n;
    const int first_m = (lin / width) * p.group_m;
    const int gsize = min(p.tiles_m - first_m, p.group_m);
    const int in = lin % width;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// ---- epilogue ---------------------------------------------------------------
// A 16x16 MFMA accumulator gives lane l column l%16 and rows 4*(l/16) + 0..3.
// With B's rows permuted at load time (see the loader) the columns of a
// lane's eight tiles j are consecutive output columns (fp32 outputs: two
// groups of four, 64 columns apart), so every global access is a 16-byte
// vector and 16 lanes cover 256 contiguous bytes of a row.

__device__ __forceinline__ uint2 pack4(const float (&w)[4]) {
    return make_uint2(pack2_bf(w[0], w[1]), pack2_bf(w[2], w[3]));
}

__device__ __forceinline__ void unpack4(uint2 q, float (&w)[4]) {
    w[0] = bf2f(q.x & 0xffffu); w[1] = bf2f(q.x >> 16);
    w[2] = bf2f(q.y & 0xffffu); w[3] = bf2f(q.y >> 16);
}

// The epilogue's memory operands for consecutive output columns of one row: i0/i1 the inputs read, o0/o1/o2 the outputs written (which ones a role
// uses is fixed by EPI; unused pointers are ignored).
struct EpiPtr {
    const char* i0;
    const char* i1;
    char* o0;
    char* o1;
    char* o2;
};

// Gate/up pair for hidden columns col..col+3, already scaled by the row's
// RMSNorm factor: stores g, u (bf16, for the backward) and h = silu(g) u
// computed from the fp32 values (the down GEMM's operand).
__device__ __forceinline__ void epi4_swiglu(const EpiPtr& a, const float (&g)[4], const float (&u)[4]) {
    float hh[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) hh[k] = swiglu_f(g[k], u[k]);
    *reinterpret_cast<uint2*>(a.o0) = pack4(g);
    *reinterpret_cast<uint2*>(a.o1) = pack4(u);
    *reinterpret_cast<uint2*>(a.o2) = pack4(hh);
}

// Eight consecutive output columns of one row (the K-contiguous kernel's
// accumulator layout): 16-byte bf16 and 32-byte fp32 accesses.
__device__ __forceinline__ uint4 pack8(const float (&w)[8]) {
    return make_uint4(pack2_bf(w[0], w[1]), pack2_bf(w[2], w[3]), pack2_bf(w[4], w[5]), pack2_bf(w[6], w[7]));
}

__device__ __forceinline__ void unpack8(uint4 q, float (&w)[8]) {
    const uint32_t v[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        w[2 * k] = bf2f(v[k] & 0xffffu);
        w[2 * k + 1] = bf2f(v[k] >> 16);
    }
}

template <int EPI> struct EpiIn8 {};
template <> struct EpiIn8<EPI_RESID> { uint4 x; };
template <> struct EpiIn8<EPI_SWIGLU_BWD> { uint4 g, u; };
template <> struct EpiIn8<EPI_ACC_F32> { float4 c0, c1; };

// fp32 outputs (dn, the weight gradients): the lane's eight columns are two
// groups of four, 64 columns apart (o0/i0 and o1/i1), so each access
// instruction covers 256 contiguous bytes of a row.  CHK: an edge tile, where
// the second group may lie past N (null pointers).
template <int EPI, bool CHK = false>
__device__ __forceinline__ void epi_load8(const EpiPtr& a, EpiIn8<EPI>& in) {
    if constexpr (EPI == EPI_RESID) {
        in.x = *reinterpret_cast<const uint4*>(a.i0);
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        in.g = *reinterpret_cast<const uint4*>(a.i0);
        in.u = *reinterpret_cast<const uint4*>(a.i1);
    } else if constexpr (EPI == EPI_ACC_F32) {
        in.c0 = *reinterpret_cast<const float4*>(a.i0);
        if (!CHK || a.i1) in.c1 = *reinterpret_cast<const float4*>(a.i1);
    }
}

template <int EPI, bool CHK = false>
__device__ __forceinline__ void epi8(const EpiPtr& a, const float (&w)[8], const EpiIn8<EPI>& in) {
    if constexpr (EPI == EPI_STORE_F32) {
        *reinterpret_cast<float4*>(a.o0) = make_float4(w[0], w[1], w[2], w[3]);
        if (!CHK || a.o1) *reinterpret_cast<float4*>(a.o1) = make_float4(w[4], w[5], w[6], w[7]);
    } else if constexpr (EPI == EPI_STORE) {
        *reinterpret_cast<uint4*>(a.o0) = pack8(w);
    } else if constexpr (EPI == EPI_RESID) {
        float x[8], y[8];
        unpack8(in.x, x);
#pragma unroll
        for (int k = 0; k < 8; ++k) y[k] = x[k] + w[k];
        *reinterpret_cast<uint4*>(a.o0) = pack8(y);
    } else if constexpr (EPI == EPI_ACC_F32) {
        const float4 c0 = in.c0, c1 = in.c1;
        *reinterpret_cast<float4*>(a.o0) = make_float4(c0.x + w[0], c0.y + w[1], c0.z + w[2], c0.w + w[3]);
        if (!CHK || a.o1)
            *reinterpret_cast<float4*>(a.o1) = make_float4(c1.x + w[4], c1.y + w[5], c1.z + w[6], c1.w + w[7]);
    }
}

// SwiGLU backward for 8 columns: stores dg, du and returns them with
// h = silu(g) u (from the stored g, u) packed to bf16, for the caller to
// store transposed.
__device__ __forceinline__ void epi8_swiglu_bwd(const EpiPtr& a, const float (&w)[8], const EpiIn8<EPI_SWIGLU_BWD>& in,
                                                uint4& ph, uint4& pdg, uint4& pdu) {
    float g[8], u[8], dg[8], du[8], hh[8];
    unpack8(in.g, g);
    unpack8(in.u, u);
#pragma unroll
    for (int k = 0; k < 8; ++k) swiglu_h_bwd_f(w[k], g[k], u[k], hh[k], dg[k], du[k]);
    ph = pack8(hh);
    pdg = pack8(dg);
    pdu = pack8(du);
    *reinterpret_cast<uint4*>(a.o0) = pdg;
    *reinterpret_cast<uint4*>(a.o1) = pdu;
}

__device__ __forceinline__ uint32_t u4_at(const uint4& v, int c) { return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w; }

// Transposed outputs of the SwiGLU backward (h, dg, du) go through LDS, 24 KB
// per wavefront: per output a [128 columns][32 rows] bf16 block, 64 bytes per
// column.  Column c sits in slot c ^ ((c >> 3) & 1) and its 16-byte row piece
// p at position p ^ ((c >> 4) & 3), so the 8-byte writes (4 rows of one
// column per lane) and the 16-byte reads (8 rows) spread over all banks.
constexpr int TSTAGE = 24576;
__device__ __forceinline__ int tstage_off(int o, int col, int q8) {   // q8: 8-byte chunk 0..7
    const int slot = col ^ ((col >> 3) & 1);
    return o * 8192 + slot * 64 + (((q8 >> 1) ^ ((col >> 4) & 3)) << 4) + ((q8 & 1) << 3);
}

// s_waitcnt vmcnt(N) lgkmcnt(0) (expcnt left at its maximum).
template <int N>
__device__ __forceinline__ void wait_vm_lgkm0() {
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4));
}

// MFMA x (0..63) of a K half in serpentine order over the 8 x 8 tiles: row
// i = x / 8, columns ascending on even rows and descending on odd ones, so
// consecutive MFMAs always share one operand.  With fragments read in the
// order a0 b0 b1 .. b7 a1 .. a7, MFMA x needs only the first
// min(x + 2, 9 + x / 8) of them.
constexpr int ord_i(int x) { return x >> 3; }
constexpr int ord_j(int x) { return ((x >> 3) & 1) ? 7 - (x & 7) : (x & 7); }

// ---- K-contiguous kernel ----------------------------------------------------
template <int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_tn_kernel(const Params p) {
    __shared__ __attribute__((aligned(1024))) char smem[LDS_BYTES];

    int tm, tn;
    tile_coords(p, tm, tn);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * (p.swiglu ? BN / 2 : BN);   // first output column
    const int64_t nb0 = (int64_t)tn * BN;                         // first B row
    const int wave_s = __builtin_amdgcn_readfirstlane(wave);
    // Epilogue rows of this lane: lr + 16 i + 0..3 (see the epilogue below).
    const int lr = wm * 128 + 4 * (lane >> 4);

    // Loader: each wavefront moves NQ pieces of 1 KB per operand tile; piece q
    // holds LDS rows (wave*NQ+q)*8 .. +7, lane l row + l/8 at position l&7,
    // i.e. logical chunk lcq[q] = (l&7) ^ ((row>>1)&7).  Per-lane byte
    // offsets stay fixed within a K segment; the K step rides in soffset.
    int lcq[NQ];
#pragma unroll
    for (int q = 0; q < NQ; ++q) lcq[q] = (lane & 7) ^ ((((wave * NQ + q) * 8 + (lane >> 3)) >> 1) & 7);
    uint32_t aoff[NQ], boff[NQ];
    rsrc_t ar, br;
    int64_t K = 0;
    int nk = 0;
    // B rows go to LDS permuted within each wavefront's 128 rows: LDS row
    // 16j + c (MFMA tile j, column c) holds B row 8c + j, so a lane's eight
    // accumulators of one row are eight consecutive output columns.  SwiGLU
    // (B rows interleaved in groups of 32 gate and 32 up rows): tiles j < 4
    // hold gate row of hidden column 4c + j, tiles j >= 4 the up row of
    // hidden column 4c + j - 4.  fp32 outputs: tiles j < 4 hold B row 4c + j,
    // tiles j >= 4 B row 64 + 4c + j - 4.
    constexpr bool F32OUT = EPI == EPI_STORE_F32 || EPI == EPI_ACC_F32;
    auto brow = [&](int row) __attribute__((always_inline)) -> int {
        const int blk = row & ~127, j = (row >> 4) & 7, c = row & 15;
        if constexpr (F32OUT) return blk + (j >> 2) * 64 + 4 * c + (j & 3);
        if (!p.swiglu) return blk + 8 * c + j;
        const int x = 4 * c + (j & 3);
        return blk + (x >> 5) * 64 + (j >> 2) * 32 + (x & 31);
    };
    auto set_seg = [&](int s) __attribute__((always_inline)) {
        const Seg g = s == 0 ? p.seg[0] : p.seg[1];   // no dynamic index into the arguments
        ar = make_rsrc(g.A, g.a_bytes);
        br = make_rsrc(g.B, g.b_bytes);
        K = g.K;
        nk = (int)((K + BK - 1) / BK);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            const int row = (wave * NQ + q) * 8 + (lane >> 3);
            const int64_t ra = m0 + row, rb = nb0 + brow(row);
            aoff[q] = ra < p.M ? (uint32_t)(ra * g.lda * 2 + lcq[q] * 16) : OOB;
            boff[q] = rb < p.NB ? (uint32_t)(rb * g.ldb * 2 + lcq[q] * 16) : OOB;
        }
    };
    // Piece q of K tile kt holds K chunk lcq[q]: in range if it starts before K.
    auto kin = [&](int kt, int q) __attribute__((always_inline)) {
        return (int64_t)lcq[q] * 8 < K - (int64_t)kt * BK;
    };
    // Load piece q of operand tile kt into `slot` (masked: chunks past K read
    // zeros through the out-of-range offset).
    auto load = [&](auto isa_c, int slot, int kt, int q, bool masked) __attribute__((always_inline)) {
        constexpr bool ISA = decltype(isa_c)::value;
        const uint32_t o = (!masked || kin(kt, q)) ? (ISA ? aoff[q] : boff[q]) : OOB;
        const int lo = slot * OPB + (wave_s * NQ + q) * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(ISA ? ar : br, (LDS_AS void*)(smem + lo), 16, o, (uint32_t)kt * (BK * 2),
                                                 0, 0);
    };
    using TA = std::true_type;
    using TB = std::false_type;

    // Fragments: A fragment i of K half s is rows wm*128 + i*16 + l%16,
    // logical chunk 4s + l/16 at position chunk ^ ((row>>1)&7) = chunk ^ fsw;
    // the per-lane base is fixed, the slot and i*16 rows are immediates.
    const int fsw = ((lane & 15) >> 1) & 7;
    const int pc0 = ((lane >> 4) ^ fsw) << 4, pc1 = ((4 + (lane >> 4)) ^ fsw) << 4;
    const char* fA = smem + (wm * 128 + (lane & 15)) * ROWB;
    const char* fB = smem + (wn * 128 + (lane & 15)) * ROWB;
    bf16x8 fa[2][8], fb[2][8];
    // fragment x (0..15) of K half s of the tile in slots (sa, sb): a0 b0 b1 .. b7 a1 .. a7
    auto fragx = [&](int sa, int sb, int s, int x, bf16x8 (&a)[8], bf16x8 (&b)[8]) __attribute__((always_inline)) {
        const int pc = s ? pc1 : pc0;
        if (x == 0 || x >= 9) {
            const int y = x == 0 ? 0 : x - 8;
            a[y] = *reinterpret_cast<const bf16x8*>(fA + sa * OPB + y * 16 * ROWB + pc);
        } else {
            const int y = x - 1;
            b[y] = *reinterpret_cast<const bf16x8*>(fB + sb * OPB + y * 16 * ROWB + pc);
        }
    };

    f32x4 acc[8][8];
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto mm = [&](const bf16x8 (&a)[8], const bf16x8 (&b)[8], int lo, int hi) __attribute__((always_inline)) {
#pragma unroll
        for (int x = 0; x < 64; ++x)
            if (x >= lo && x < hi) {
                const int i = ord_i(x), j = ord_j(x);
                acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
    };

    // One K step on tile kt.  PH = kt % 5 when known at compile time (slot
    // offsets become immediates); MASK: tile kt+2 may reach past K.
    auto step = [&](auto ph_c, auto mask_c, int kt) __attribute__((always_inline)) {
        constexpr int PH = decltype(ph_c)::value;
        constexpr bool MASK = decltype(mask_c)::value;
        const int ph = PH >= 0 ? PH : kt % 5;
        const int sA = (2 * ph) % 5, sB = (2 * ph + 1) % 5;          // tile kt
        const int sA1 = (2 * ph + 2) % 5, sB1 = (2 * ph + 3) % 5;    // tile kt+1
        const int sA2 = (2 * ph + 4) % 5, sB2 = (2 * ph + 5) % 5;    // tile kt+2
        // first half: MFMAs on half 0; tile kt+2's A; half 1's fragments
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            mm(fa[0], fb[0], 8 * r, 8 * r + 8);
            __builtin_amdgcn_sched_barrier(0);
            load(TA{}, sA2, kt + 2, r, MASK);
            if (r < 4) {
#pragma unroll
                for (int y = 0; y < 4; ++y) fragx(sA, sB, 1, 4 * r + y, fa[1], fb[1]);
            }
            __builtin_amdgcn_sched_barrier(0);
        }
        // this wavefront's reads of tile kt are done; after the barrier no
        // wavefront reads its slots
        __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt open
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
        // second half: MFMAs on half 1; tile kt+2's B into A(kt)'s slot
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            load(TB{}, sB2, kt + 2, r, MASK);
            __builtin_amdgcn_sched_barrier(0);
            mm(fa[1], fb[1], 6 * r, 6 * r + 6);
            __builtin_amdgcn_sched_barrier(0);
        }
        // vmcnt(16): all but tile kt+2's requests, i.e. tile kt+1, have landed
        wait_vm_lgkm0<2 * NQ>();
        __builtin_amdgcn_s_barrier();
#pragma unroll
        for (int r = 0; r < 16; ++r) {
            fragx(sA1, sB1, 0, r, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
            mm(fa[1], fb[1], 48 + r, 49 + r);
            __builtin_amdgcn_sched_barrier(0);
        }
    };
    using P0 = std::integral_constant<int, 0>;
    using P1 = std::integral_constant<int, 1>;
    using P2 = std::integral_constant<int, 2>;
    using P3 = std::integral_constant<int, 3>;
    using P4 = std::integral_constant<int, 4>;
    using PR = std::integral_constant<int, -1>;

    for (int s = 0; s < p.nseg; ++s) {
        set_seg(s);
        if (nk == 0) continue;
#pragma unroll
        for (int q = 0; q < NQ; ++q) { load(TA{}, 0, 0, q, true); load(TB{}, 1, 0, q, true); }
#pragma unroll
        for (int q = 0; q < NQ; ++q) { load(TA{}, 2, 1, q, true); load(TB{}, 3, 1, q, true); }
        wait_vm_lgkm0<2 * NQ>();   // tile 0 in LDS
        __builtin_amdgcn_s_barrier();
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int x = 0; x < 16; ++x) {
            fragx(0, 1, 0, x, fa[0], fb[0]);
            __builtin_amdgcn_sched_barrier(0);
        }
        // unmasked while tile kt+2 lies wholly inside K
        const int nfull = (int)(K / BK);
        int kt = 0;
        for (; kt + 7 <= nfull; kt += 5) {
            step(P0{}, std::false_type{}, kt);
            step(P1{}, std::false_type{}, kt + 1);
            step(P2{}, std::false_type{}, kt + 2);
            step(P3{}, std::false_type{}, kt + 3);
            step(P4{}, std::false_type{}, kt + 4);
        }
        for (; kt < nk; ++kt) step(PR{}, std::true_type{}, kt);
        // the last steps requested all-zero tiles past K: let them land
        // before another segment reuses the slots (and before the epilogue)
        wait_vm_lgkm0<0>();
        __builtin_amdgcn_s_barrier();
    }

    // Epilogue.  With the permuted B rows, accumulator register r of tile
    // (i, j) is output row lr + 16i + r, column lc + j: each lane holds eight
    // consecutive columns of a row (SwiGLU: gate tiles j < 4 and up tiles
    // j >= 4 of the four hidden columns lc .. lc+3; fp32 outputs: columns
    // lc .. lc+3 in tiles j < 4 and lc+64 .. lc+67 in tiles j >= 4).
    const int lc = p.swiglu || F32OUT ? wn * (p.swiglu ? 64 : 128) + 4 * (lane & 15) : wn * 128 + 8 * (lane & 15);
    // SwiGLU: the RMSNorm factor r of this lane's 32 output rows (the GEMM
    // read x; gamma is folded into B), requested first.
    float rsc[8][4];
    if constexpr (EPI == EPI_SWIGLU) {
        const float* rs = p.e.rowscale;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const int64_t row = m0 + lr + 16 * i;
            if (rs && row + 3 < p.M) {
                const float4 v = *reinterpret_cast<const float4*>(rs + row);
                rsc[i][0] = v.x; rsc[i][1] = v.y; rsc[i][2] = v.z; rsc[i][3] = v.w;
            } else {
#pragma unroll
                for (int k = 0; k < 4; ++k) rsc[i][k] = rs && row + k < p.M ? rs[row + k] : 1.0f;
            }
        }
    }
    const EpiArgs e = p.e;
    const int64_t pM = p.M, pN = p.N;
    constexpr int ESO = (EPI == EPI_STORE_F32 || EPI == EPI_ACC_F32) ? 4 : 2;   // output element bytes
    constexpr bool HAS_IN = EPI == EPI_RESID || EPI == EPI_SWIGLU_BWD || EPI == EPI_ACC_F32;

    // Whole tile inside M x N: every operand is a uniform per-tile base plus
    // this lane's fixed 32-bit offset plus a uniform per-(i, r) offset, so the
    // accesses need no bounds checks and no per-element 64-bit index
    // arithmetic.  The fp32 accumulate splits its columns at nsplit (columns
    // n >= nsplit go to out1 at n - nsplit): a tile on one side takes that
    // side's base, a tile across the split goes the edge way.
    const bool hi_side = EPI == EPI_ACC_F32 && n0 >= e.nsplit;
    const bool straddle = EPI == EPI_ACC_F32 && n0 < e.nsplit && n0 + BN > e.nsplit;
    const bool fast = m0 + BM <= pM && n0 + (p.swiglu ? BN / 2 : BN) <= pN && !straddle;
    char* const ob = hi_side ? static_cast<char*>(e.out1) + (m0 * e.ld1 + n0 - e.nsplit) * ESO
                             : static_cast<char*>(e.out0) + (m0 * e.ld0 + n0) * ESO;   // output tile base
    const int64_t old = hi_side ? e.ld1 : e.ld0;                                      // its leading dimension

    const uint32_t lo = (uint32_t)(((int64_t)lr * old + lc) * ESO);
    const uint32_t li = (uint32_t)(((int64_t)lr * e.ldi0 + lc) * 2);
    auto fptr = [&](int i, int r) __attribute__((always_inline)) -> EpiPtr {
        const int64_t uo = (int64_t)(i * 16 + r) * old * ESO;
        EpiPtr a{};
        char* o = ob + uo + lo;
        a.o0 = o;
        if constexpr (EPI == EPI_SWIGLU) {
            a.o1 = static_cast<char*>(e.out1) + (m0 * e.ld0 + n0) * 2 + uo + lo;
            a.o2 = static_cast<char*>(e.out2) + (m0 * e.ld0 + n0) * 2 + uo + lo;
        } else if constexpr (EPI == EPI_SWIGLU_BWD) {
            a.o1 = o + e.nsplit * 2;
            const int64_t ui = ((int64_t)(i * 16 + r) * e.ldi0 + m0 * e.ldi0 + n0) * 2;
            a.i0 = static_cast<const char*>(e.in0) + ui + li;
            a.i1 = static_cast<const char*>(e.in1) + ui + li;
        } else if constexpr (EPI == EPI_RESID) {
            a.i0 = static_cast<const char*>(e.in0) + ((int64_t)(i * 16 + r) * e.ldi0 + m0 * e.ldi0 + n0) * 2 + li;
        }
        if constexpr (F32OUT) a.o1 = o + 64 * ESO;
        if constexpr (EPI == EPI_ACC_F32) {
            a.i0 = a.o0;
            a.i1 = a.o1;
        }
        return a;
    };
    // edge tiles: the same accesses from (row, col); a column group lies
    // wholly inside or outside N (a multiple of 8)
    auto sptr = [&](int64_t row, int64_t col) __attribute__((always_inline)) -> EpiPtr {
        EpiPtr a{};
        a.o0 = static_cast<char*>(e.out0) + (row * e.ld0 + col) * ESO;
        if constexpr (F32OUT) {
            // two groups of four columns, at col and col + 64 (null past N)
            auto at = [&](int64_t c) __attribute__((always_inline)) -> char* {
                if (c >= pN) return nullptr;
                if (EPI == EPI_ACC_F32 && c >= e.nsplit)
                    return static_cast<char*>(e.out1) + (row * e.ld1 + c - e.nsplit) * ESO;
                return static_cast<char*>(e.out0) + (row * e.ld0 + c) * ESO;
            };
            a.o0 = at(col);
            a.o1 = at(col + 64);
            a.i0 = a.o0;
            a.i1 = a.o1;
        } else {
            if constexpr (EPI == EPI_SWIGLU) {
                a.o1 = static_cast<char*>(e.out1) + (row * e.ld0 + col) * 2;
                a.o2 = static_cast<char*>(e.out2) + (row * e.ld0 + col) * 2;
            } else if constexpr (EPI == EPI_SWIGLU_BWD) {
                a.o1 = a.o0 + e.nsplit * 2;
                a.i0 = static_cast<const char*>(e.in0) + (row * e.ldi0 + col) * 2;
                a.i1 = static_cast<const char*>(e.in1) + (row * e.ldi0 + col) * 2;
            } else if constexpr (EPI == EPI_RESID) {
                a.i0 = static_cast<const char*>(e.in0) + (row * e.ldi0 + col) * 2;
            }
        }
        return a;
    };

    auto run = [&](auto fast_c) __attribute__((always_inline)) {
        constexpr bool FAST = decltype(fast_c)::value;
        auto ptr = [&](int i, int r) __attribute__((always_inline)) -> EpiPtr {
            if constexpr (FAST) return fptr(i, r);
            else return sptr(m0 + lr + i * 16 + r, n0 + lc);
        };
        auto ok = [&](int i, int r) __attribute__((always_inline)) -> bool {
            if constexpr (FAST) return true;
            else return m0 + lr + i * 16 + r < pM && n0 + lc < pN;
        };
        // inputs of row groups i+1 .. i+NB-1 load while row group i computes
        // (the K loop's fragment registers are free by now); the fp32
        // accumulate measured faster one row group ahead than two or three
        constexpr int NB = EPI == EPI_SWIGLU_BWD ? 4 : 2;
        EpiIn8<EPI> in[NB][4];
        auto prefetch = [&](int i, EpiIn8<EPI> (&dst)[4]) __attribute__((always_inline)) {
            if constexpr (HAS_IN) {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (ok(i, r)) epi_load8<EPI, !FAST>(ptr(i, r), dst[r]);
            }
        };
#pragma unroll
        for (int i = 0; i < NB - 1; ++i) prefetch(i, in[i]);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i + NB - 1 < 8) prefetch(i + NB - 1, in[(i + NB - 1) % NB]);
            uint4 pk[3][4];   // SwiGLU backward: h, dg, du of this row group, bf16
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                if constexpr (EPI == EPI_SWIGLU_BWD) {
                    float w[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) w[j] = acc[i][j][r];
                    if (ok(i, r)) epi8_swiglu_bwd(ptr(i, r), w, in[i % NB][r], pk[0][r], pk[1][r], pk[2][r]);
                } else if constexpr (EPI == EPI_SWIGLU) {
                    const float sc = rsc[i][r];
                    const float g[4] = {acc[i][0][r] * sc, acc[i][1][r] * sc, acc[i][2][r] * sc, acc[i][3][r] * sc};
                    const float u[4] = {acc[i][4][r] * sc, acc[i][5][r] * sc, acc[i][6][r] * sc, acc[i][7][r] * sc};
                    if (ok(i, r)) epi4_swiglu(ptr(i, r), g, u);
                } else {
                    float w[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) w[j] = acc[i][j][r];
                    if (ok(i, r)) epi8<EPI, !FAST>(ptr(i, r), w, in[i % NB][r]);
                }
            }
            if constexpr (EPI == EPI_SWIGLU_BWD && FAST) {
                // h (out2) and dg, du (out3) for the weight gradients,
                // written transposed (T-contiguous) through LDS: column j's
                // four rows of this row group are one 8-byte chunk of the
                // wavefront's staging block; after two row groups, 32 rows
                // of each column go out as 16-byte pieces.  Only full tiles:
                // the dispatcher requires them with out2.
                if (e.out2 || e.out3) {
                    const int olo = e.out2 ? 0 : 1, ohi = e.out3 ? 3 : 1;   // outputs olo .. ohi-1
                    char* const wst = smem + wave_s * TSTAGE;
                    const int q8 = 4 * (i & 1) + (lane >> 4);
                    const int lcl = 8 * (lane & 15);
#pragma unroll
                    for (int o = 0; o < 3; ++o) {
                        if (o >= olo && o < ohi) {
#pragma unroll
                            for (int j = 0; j < 8; ++j) {
                                const int c = j >> 1, sh = (j & 1) * 16;
                                const uint32_t r0 = (u4_at(pk[o][0], c) >> sh) & 0xffffu, r1 = (u4_at(pk[o][1], c) >> sh) & 0xffffu;
                                const uint32_t r2 = (u4_at(pk[o][2], c) >> sh) & 0xffffu, r3 = (u4_at(pk[o][3], c) >> sh) & 0xffffu;
                                *reinterpret_cast<uint2*>(wst + tstage_off(o, lcl + j, q8)) = make_uint2(r0 | (r1 << 16), r2 | (r3 << 16));
                            }
                        }
                    }
                    if (i & 1) {
                        // the wavefront's own staging writes are visible to its reads
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                        __builtin_amdgcn_wave_barrier();
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                        const int pq = lane & 3;
                        const int64_t trow = m0 + wm * 128 + 32 * (i >> 1) + 8 * pq;   // first of 8 rows
#pragma unroll
                        for (int o = 0; o < 3; ++o) {
                            if (o >= olo && o < ohi) {
                                char* const dst = o == 0 ? static_cast<char*>(e.out2)
                                                : o == 1 ? static_cast<char*>(e.out3)
                                                         : static_cast<char*>(e.out3) + e.nsplit * e.ld2 * 2;
#pragma unroll
                                for (int k = 0; k < 8; ++k) {
                                    const int col = 16 * k + (lane >> 2);
                                    const uint4 v = *reinterpret_cast<const uint4*>(wst + tstage_off(o, col, 2 * pq));
                                    *reinterpret_cast<uint4*>(dst + ((n0 + wn * 128 + col) * e.ld2 + trow) * 2) = v;
                                }
                            }
                        }
                        // reads done before the next pair overwrites the block
                        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
                        __builtin_amdgcn_wave_barrier();
                        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
                    }
                }
            }
        }
    };
    if (fast) run(std::true_type{});
    else run(std::false_type{});
}

// Byte extent of a row-major operand: (rows-1)*ld + cols' elements of bf16,
// cols' = cols rounded up to the 8-element chunk the loader moves (within
// ld).  The buffer range check works on whole dwords, so an extent that ended
// inside the last row's chunk (cols odd: a K = T of odd length) would drop
// that row's last valid element; the elements of [cols, cols') are the
// row's padding, which the K-tail chunks of every other row read as well
// (zero in the T-contiguous operands).
inline bool extent(int64_t rows, int64_t ld, int64_t cols, uint32_t& out) {
    const int64_t cr = std::min<int64_t>((cols + 7) / 8 * 8, std::max<int64_t>(ld, cols));
    const int64_t b = rows <= 0 ? 0 : ((rows - 1) * ld + cr) * 2;
    if (b >= (int64_t)OOB) return false;
    out = (uint32_t)b;
    return true;
}

template <int EPI>
hipError_t launch(const Params& p, hipStream_t s) {
    hipLaunchKernelGGL((gemm_tn_kernel<EPI>), dim3(p.tiles_m * p.tiles_n), dim3(NTHREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

int64_t swiglu_b_rows(int64_t ffn) { return 2 * ((ffn + 31) / 32) * 32; }

int64_t gemm_bf16_tiles(int64_t M, int64_t N) { return ((M + BM - 1) / BM) * ((N + BN - 1) / BN); }

// Requires A and B K-contiguous, every operand extent under 2 GB, N, the
// output and input leading dimensions and the SwiGLU-backward split column
// multiples of 8 and the epilogue pointers 16-byte aligned (the epilogue
// moves 8 consecutive output columns, SwiGLU 4 hidden columns, per 16-byte
// access); the fp32 accumulate's split column nsplit and out1's leading
// dimension are multiples of 8 when nsplit < N.  With the
// SwiGLU map, B is the gate/up weight interleaved per 32 hidden columns (32
// gate rows, then 32 up rows; swiglu_b_rows(N) rows) and N is the number of
// hidden columns.
hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
    if (!a.a_kcontig || !a.b_kcontig) return hipErrorInvalidValue;
    const bool in = a.epi == EPI_RESID || a.epi == EPI_SWIGLU_BWD;
    if (a.N % 8 || a.e.ld0 % 8 || (in && a.e.ldi0 % 8) || (a.epi == EPI_SWIGLU_BWD && a.e.nsplit % 8))
        return hipErrorInvalidValue;
    if (a.epi == EPI_ACC_F32 && a.e.nsplit < a.N && (!a.e.out1 || a.e.nsplit % 8 || a.e.ld1 % 8))
        return hipErrorInvalidValue;
    if (a.epi == EPI_SWIGLU_BWD && (a.e.out2 || a.e.out3) && (a.M % BM || a.N % BN || a.e.ld2 < a.M || a.e.ld2 % 8))
        return hipErrorInvalidValue;   // h, dg, du are written transposed from full tiles only
    if (a.e.out3 && a.epi != EPI_SWIGLU_BWD) return hipErrorInvalidValue;
    const uintptr_t ptrs = reinterpret_cast<uintptr_t>(a.e.out0) | reinterpret_cast<uintptr_t>(a.e.out1) |
                           reinterpret_cast<uintptr_t>(a.e.out2) | reinterpret_cast<uintptr_t>(a.e.in0) |
                           reinterpret_cast<uintptr_t>(a.e.in1) | reinterpret_cast<uintptr_t>(a.e.rowscale) |
                           reinterpret_cast<uintptr_t>(a.e.out3);
    if (ptrs % 16) return hipErrorInvalidValue;
    Params p{};
    p.M = a.M;
    p.N = a.N;
    p.nseg = a.nseg;
    p.swiglu = a.swiglu_map ? 1 : 0;
    const int64_t cols_per_tile = a.swiglu_map ? BN / 2 : BN;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    p.tiles_n = (int)((a.N + cols_per_tile - 1) / cols_per_tile);
    p.NB = a.swiglu_map ? swiglu_b_rows(a.N) : a.N;
    // The 32 tiles an XCD runs at once span group_m tile rows x 32/group_m
    // tile columns: 8 x 4 fetches each B panel slice for 8 tiles and each A
    // slice for 4, 4 x 8 the other way round.  With more than twice as many
    // A rows as B rows (weight gradient of W_d: A = h^T, B = dy^T) A is the
    // operand that does not stay in the on-package cache, so its panels are
    // the ones to share; the SwiGLU-backward role measured faster with 4 too.
    p.group_m = (a.M > 2 * p.NB || a.epi == EPI_SWIGLU_BWD) ? 4 : 8;
    for (int i = 0; i < a.nseg; ++i) {
        const GemmSeg& g = a.seg[i];
        p.seg[i].A = static_cast<const uint16_t*>(g.A);
        p.seg[i].B = static_cast<const uint16_t*>(g.B);
        p.seg[i].lda = g.lda;
        p.seg[i].ldb = g.ldb;
        p.seg[i].K = g.K;
        const bool ok = extent(a.M, g.lda, g.K, p.seg[i].a_bytes) && extent(p.NB, g.ldb, g.K, p.seg[i].b_bytes);
        if (!ok) return hipErrorInvalidValue;
    }
    p.e = a.e;
    if (p.tiles_m == 0 || p.tiles_n == 0) return hipSuccess;
    switch (a.epi) {
        case EPI_SWIGLU: return launch<EPI_SWIGLU>(p, s);
        case EPI_RESID: return launch<EPI_RESID>(p, s);
        case EPI_SWIGLU_BWD: return launch<EPI_SWIGLU_BWD>(p, s);
        case EPI_STORE_F32: return launch<EPI_STORE_F32>(p, s);
        case EPI_ACC_F32: return launch<EPI_ACC_F32>(p, s);
        case EPI_STORE: return launch<EPI_STORE>(p, s);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace pps
