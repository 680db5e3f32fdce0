// bf16 GEMM on the CDNA4 matrix cores (gfx950), fp32 accumulation.
//
// Macro-tile 256 x 256 x 64, 256 threads = 4 wavefronts of 64 lanes laid out
// 2 x 2; each wavefront owns a 128 x 128 sub-tile = 4 x 4 tiles of
// v_mfma_f32_32x32x16_bf16 (256 fp32 accumulators per lane).
//
// Data path: global -> registers -> LDS (double buffered, one barrier per K
// step) -> MFMA operands.  In LDS every operand tile is stored "K-major":
// 256 rows (M or N) x 64 k of bf16 = 128 bytes per row, in 16-byte chunks of
// 8 consecutive k, chunk c of row r at position c ^ (r & 7) (XOR swizzle so
// that the 8 lanes of a ds_read_b128 group hit distinct banks).  Operands
// whose contiguous dimension is M or N (activations used transposed in the
// weight-gradient GEMMs, weights [in,out] in the forward) are loaded as 8 x 8
// bf16 blocks and transposed in registers before the LDS store.
//
// Workgroup -> tile mapping: the dispatcher places workgroup i on XCD i % 8;
// ids are remapped so each XCD gets a contiguous run of logical tiles, and
// logical tiles are ordered in groups of 8 tile-rows so the tiles running on
// one XCD share A rows and B columns in that XCD's L2.
#include "epilogue.h"

namespace pps {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

constexpr int BM = 256, BN = 256, BK = 64, NTHREADS = 256;
constexpr int ROWB = BK * 2;            // bytes per LDS tile row
constexpr int OPB = 256 * ROWB;         // one operand tile: 32 KB
constexpr int STAGEB = 2 * OPB;         // A + B
constexpr int LDS_BYTES = 2 * STAGEB;   // two stages: 128 KB
constexpr int GROUP_M = 8;

struct Params {
    int64_t M, N;
    int tiles_m, tiles_n, nseg, pad;
    const uint16_t* A[2];
    const uint16_t* B[2];
    const uint16_t* B2[2];
    int64_t lda[2], ldb[2], K[2];
    EpiArgs e;
};

__device__ __forceinline__ void tile_coords(const Params& p, int& tm, int& tn) {
    const int nwg = gridDim.x, bid = blockIdx.x;
    const int per = (nwg + 7) >> 3;
    const int tall = (nwg & 7) ? (nwg & 7) : 8;
    const int xcd = bid & 7, local = bid >> 3;
    const int lin = xcd < tall ? xcd * per + local : tall * per + (xcd - tall) * (per - 1) + local;
    const int width = GROUP_M * p.tiles_n;
    const int first_m = (lin / width) * GROUP_M;
    const int gsize = min(p.tiles_m - first_m, GROUP_M);
    const int in = lin % width;
    tm = first_m + in % gsize;
    tn = in / gsize;
}

// K-contiguous operand: 256 rows x 8 chunks; thread t loads chunk (t & 7) of
// rows (t >> 3) + 32 i.
__device__ __forceinline__ void load_kc(uint4 (&v)[8], const uint16_t* base, int64_t ld,
                                        int64_t r0, int64_t nrows, int64_t k0, int64_t K, int t) {
    const int64_t k = k0 + (t & 7) * 8;
    const int rr = t >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = r0 + rr + 32 * i;
        if (k < K && row < nrows) v[i] = *reinterpret_cast<const uint4*>(base + row * ld + k);
        else v[i] = make_uint4(0u, 0u, 0u, 0u);
    }
}

__device__ __forceinline__ void store_kc(const uint4 (&v)[8], char* lds, int t) {
    const int c = t & 7, rr = t >> 3;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = rr + 32 * i;
        *reinterpret_cast<uint4*>(lds + row * ROWB + ((c ^ (rr & 7)) << 4)) = v[i];
    }
}

// M/N-contiguous operand stored [K][R]: thread t loads the 8 x 8 block of
// k rows k0 + (t & 7)*8 + j and the 8 columns starting at `col`.
__device__ __forceinline__ void load_mn(uint4 (&v)[8], const uint16_t* base, int64_t ld,
                                        int64_t col, bool colok, int64_t k0, int64_t K, int t) {
    const int64_t kb = k0 + (t & 7) * 8;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const int64_t k = kb + j;
        if (colok && k < K) v[j] = *reinterpret_cast<const uint4*>(base + k * ld + col);
        else v[j] = make_uint4(0u, 0u, 0u, 0u);
    }
}

// Transpose the 8 (k) x 8 (row) block in registers and store 8 chunks.
__device__ __forceinline__ void store_mn(const uint4 (&v)[8], char* lds, int t) {
    const int kb = t & 7, rb = t >> 3;
    uint32_t w[8][4];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        w[j][0] = v[j].x; w[j][1] = v[j].y; w[j][2] = v[j].z; w[j][3] = v[j].w;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        uint32_t d[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = w[2 * q][i >> 1], b = w[2 * q + 1][i >> 1];
            d[q] = (i & 1) ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
        }
        const int row = rb * 8 + i;
        *reinterpret_cast<uint4*>(lds + row * ROWB + ((kb ^ i) << 4)) = make_uint4(d[0], d[1], d[2], d[3]);
    }
}

template <bool AK, bool BKC, bool SWMAP, int EPI>
__global__ __launch_bounds__(NTHREADS, 1) void gemm_bf16_kernel(const Params p) {
    static_assert(!(SWMAP && BKC), "the SwiGLU column map needs an N-contiguous B");
    __shared__ __attribute__((aligned(16))) char smem[LDS_BYTES];

    int tm, tn;
    tile_coords(p, tm, tn);
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t m0 = (int64_t)tm * BM;
    const int64_t n0 = (int64_t)tn * (SWMAP ? BN / 2 : BN);

    f32x16 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.0f;

    for (int s = 0; s < p.nseg; ++s) {
        const int64_t K = p.K[s];
        const int nk = (int)((K + BK - 1) / BK);
        if (nk == 0) continue;
        const uint16_t* A = p.A[s];
        const int64_t lda = p.lda[s], ldb = p.ldb[s];

        // Per-thread column block for M/N-contiguous operands.
        const int cb = (t >> 3) * 8;
        const int64_t acol = m0 + cb;
        const bool acolok = acol < p.M;
        const uint16_t* bbase = p.B[s];
        int64_t bcol = n0 + cb;
        if constexpr (SWMAP) {
            // tile column c -> group c/128; first 64 from B (gate), next 64 from B2 (up)
            const int grp = cb >> 7, w = cb & 127;
            bbase = (w >= 64) ? p.B2[s] : p.B[s];
            bcol = n0 + grp * 64 + (w & 63);
        }
        const bool bcolok = bcol < p.N;

        uint4 ra[8], rb[8];
        auto gload = [&](int kt) {
            const int64_t k0 = (int64_t)kt * BK;
            if constexpr (AK) load_kc(ra, A, lda, m0, p.M, k0, K, t);
            else load_mn(ra, A, lda, acol, acolok, k0, K, t);
            if constexpr (BKC) load_kc(rb, p.B[s], ldb, n0, p.N, k0, K, t);
            else load_mn(rb, bbase, ldb, bcol, bcolok, k0, K, t);
        };
        auto lstore = [&](int buf) {
            char* la = smem + buf * STAGEB;
            if constexpr (AK) store_kc(ra, la, t); else store_mn(ra, la, t);
            if constexpr (BKC) store_kc(rb, la + OPB, t); else store_mn(rb, la + OPB, t);
        };

        gload(0);
        lstore(0);
        __syncthreads();
        for (int kt = 0; kt < nk; ++kt) {
            const int cur = kt & 1;
            if (kt + 1 < nk) gload(kt + 1);
            const char* la = smem + cur * STAGEB;
            const char* lb = la + OPB;
#pragma unroll
            for (int kk = 0; kk < BK / 16; ++kk) {
                const int ch = kk * 2 + (lane >> 5);
                const int sw = (ch ^ (lane & 7)) << 4;
                bf16x8 a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    a[i] = *reinterpret_cast<const bf16x8*>(la + (wm * 128 + i * 32 + (lane & 31)) * ROWB + sw);
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    b[j] = *reinterpret_cast<const bf16x8*>(lb + (wn * 128 + j * 32 + (lane & 31)) * ROWB + sw);
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
            }
            if (kt + 1 < nk) lstore(cur ^ 1);
            __syncthreads();
        }
    }

    // Accumulator layout of a 32x32 MFMA tile: lane l, element e holds
    // row (e/4)*8 + (l/32)*4 + e%4, column l%32.
#pragma clang loop unroll(full)
    for (int i = 0; i < 4; ++i) {
#pragma clang loop unroll(full)
        for (int e = 0; e < 16; ++e) {
            const int64_t row = m0 + wm * 128 + i * 32 + (e >> 2) * 8 + (lane >> 5) * 4 + (e & 3);
            const bool rok = row < p.M;
            if constexpr (EPI == EPI_SWIGLU) {
#pragma clang loop unroll(full)
                for (int j = 0; j < 2; ++j) {
                    const int64_t col = n0 + wn * 64 + j * 32 + (lane & 31);
                    if (rok && col < p.N) epi_swiglu<uint16_t>(p.e, row, col, acc[i][j][e], acc[i][j + 2][e]);
                }
            } else {
#pragma clang loop unroll(full)
                for (int j = 0; j < 4; ++j) {
                    const int64_t col = n0 + wn * 128 + j * 32 + (lane & 31);
                    if (rok && col < p.N) epi_apply<EPI, uint16_t>(p.e, row, col, acc[i][j][e]);
                }
            }
        }
    }
}

template <bool AK, bool BKC, bool SWMAP, int EPI>
hipError_t launch(const Params& p, hipStream_t s) {
    const int grid = p.tiles_m * p.tiles_n;
    hipLaunchKernelGGL((gemm_bf16_kernel<AK, BKC, SWMAP, EPI>), dim3(grid), dim3(NTHREADS), 0, s, p);
    return hipGetLastError();
}

}  // namespace

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s) {
    Params p{};
    p.M = a.M;
    p.N = a.N;
    p.nseg = a.nseg;
    for (int i = 0; i < a.nseg; ++i) {
        p.A[i] = static_cast<const uint16_t*>(a.seg[i].A);
        p.B[i] = static_cast<const uint16_t*>(a.seg[i].B);
        p.B2[i] = static_cast<const uint16_t*>(a.seg[i].B2);
        p.lda[i] = a.seg[i].lda;
        p.ldb[i] = a.seg[i].ldb;
        p.K[i] = a.seg[i].K;
    }
    p.e = a.e;
    const int64_t ncols_per_tile = a.swiglu_map ? BN / 2 : BN;
    p.tiles_m = (int)((a.M + BM - 1) / BM);
    p.tiles_n = (int)((a.N + ncols_per_tile - 1) / ncols_per_tile);
    if (p.tiles_m == 0 || p.tiles_n == 0) return hipSuccess;

#define PPS_GEMM_CASE(AKV, BKV, SWV, EPV)                                                  \
    if (a.a_kcontig == AKV && a.b_kcontig == BKV && a.swiglu_map == SWV && a.epi == EPV) \
        return launch<AKV, BKV, SWV, EPV>(p, s);
    PPS_GEMM_CASE(true, false, true, EPI_SWIGLU)        // g,u = n [Wg|Wu]
    PPS_GEMM_CASE(true, false, false, EPI_RESID)        // y = x + h Wd
    PPS_GEMM_CASE(true, true, false, EPI_SWIGLU_BWD)    // dh = dy Wd^T
    PPS_GEMM_CASE(true, true, false, EPI_STORE_F32)     // dn = dg Wg^T + du Wu^T
    PPS_GEMM_CASE(false, false, false, EPI_ACC_F32)     // dW += X^T G
    PPS_GEMM_CASE(true, false, false, EPI_STORE)
    PPS_GEMM_CASE(true, true, false, EPI_STORE)
#undef PPS_GEMM_CASE
    return hipErrorInvalidValue;
}

}  // namespace pps
