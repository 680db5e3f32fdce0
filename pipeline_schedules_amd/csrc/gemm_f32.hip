// fp32 GEMM (vector ALU, fp32 storage and arithmetic) for the fp32 stage
// workloads, plus the dtype dispatcher of pps::gemm.
//
// Tile 64 x 64 x 16, 256 threads as 16 x 16; thread (tx, ty) owns rows
// ty + 16 i and columns tx + 16 j (i, j < 4), so the four columns of one
// thread pair up (j, j+2) for the SwiGLU gate/up map: tile column c < 32 is
// gate column tn*32 + c, c >= 32 the up column of the same hidden index.
#include "epilogue.h"
#include "pps.h"

namespace pps {

hipError_t gemm_bf16(const GemmArgs& a, hipStream_t s);

namespace {

constexpr int TB = 64, TK = 16;

struct Params32 {
    int64_t M, N;
    int tiles_m, tiles_n, nseg, pad;
    const float* A[2];
    const float* B[2];
    const float* B2[2];
    int64_t lda[2], ldb[2], K[2];
    EpiArgs e;
};

template <bool AK, bool BKC, bool SWMAP, int EPI>
__global__ __launch_bounds__(256) void gemm_f32_kernel(const Params32 p) {
    __shared__ float As[TK][TB + 4];
    __shared__ float Bs[TK][TB + 4];
    const int t = threadIdx.x, tx = t & 15, ty = t >> 4;
    const int tm = blockIdx.x % p.tiles_m, tn = blockIdx.x / p.tiles_m;
    const int64_t m0 = (int64_t)tm * TB;
    const int64_t n0 = (int64_t)tn * (SWMAP ? TB / 2 : TB);
    float acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = 0.0f;

    for (int s = 0; s < p.nseg; ++s) {
        const int64_t K = p.K[s];
        for (int64_t k0 = 0; k0 < K; k0 += TK) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int e = t + 256 * q;
                int m, k;
                if constexpr (AK) { m = e >> 4; k = e & 15; } else { k = e >> 6; m = e & 63; }
                const int64_t gm = m0 + m, gk = k0 + k;
                float v = 0.0f;
                if (gm < p.M && gk < K) v = AK ? p.A[s][gm * p.lda[s] + gk] : p.A[s][gk * p.lda[s] + gm];
                As[k][m] = v;
                int n;
                if constexpr (BKC) { n = e >> 4; k = e & 15; } else { k = e >> 6; n = e & 63; }
                const float* bb = p.B[s];
                int64_t gn = n0 + n;
                if constexpr (SWMAP) {
                    bb = (n >= 32) ? p.B2[s] : p.B[s];
                    gn = n0 + (n & 31);
                }
                const int64_t gk2 = k0 + k;
                float w = 0.0f;
                if (gn < p.N && gk2 < K) w = BKC ? bb[gn * p.ldb[s] + gk2] : bb[gk2 * p.ldb[s] + gn];
                Bs[k][n] = w;
            }
            __syncthreads();
#pragma unroll
            for (int k = 0; k < TK; ++k) {
                float a[4], b[4];
#pragma unroll
                for (int i = 0; i < 4; ++i) a[i] = As[k][ty + 16 * i];
#pragma unroll
                for (int j = 0; j < 4; ++j) b[j] = Bs[k][tx + 16 * j];
#pragma unroll
                for (int i = 0; i < 4; ++i)
#pragma unroll
                    for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
            }
            __syncthreads();
        }
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t row = m0 + ty + 16 * i;
        if (row >= p.M) continue;
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int64_t col = n0 + tx + 16 * j;
                if (col < p.N) epi_swiglu<float>(p.e, row, col, acc[i][j], acc[i][j + 2]);
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int64_t col = n0 + tx + 16 * j;
                if (col < p.N) epi_apply<EPI, float>(p.e, row, col, acc[i][j]);
            }
        }
    }
}

template <bool AK, bool BKC, bool SWMAP, int EPI>
hipError_t launch32(const Params32& p, hipStream_t s) {
    hipLaunchKernelGGL((gemm_f32_kernel<AK, BKC, SWMAP, EPI>), dim3(p.tiles_m * p.tiles_n), dim3(256), 0, s, p);
    return hipGetLastError();
}

hipError_t gemm_f32(const GemmArgs& a, hipStream_t s) {
    Params32 p{};
    p.M = a.M;
    p.N = a.N;
    p.nseg = a.nseg;
    for (int i = 0; i < a.nseg; ++i) {
        p.A[i] = static_cast<const float*>(a.seg[i].A);
        p.B[i] = static_cast<const float*>(a.seg[i].B);
        p.B2[i] = static_cast<const float*>(a.seg[i].B2);
        p.lda[i] = a.seg[i].lda;
        p.ldb[i] = a.seg[i].ldb;
        p.K[i] = a.seg[i].K;
    }
    p.e = a.e;
    p.tiles_m = (int)((a.M + TB - 1) / TB);
    p.tiles_n = (int)((a.N + (a.swiglu_map ? TB / 2 : TB) - 1) / (a.swiglu_map ? TB / 2 : TB));
    if (p.tiles_m == 0 || p.tiles_n == 0) return hipSuccess;
#define PPS_GEMM32_CASE(AKV, BKV, SWV, EPV)                                                \
    if (a.a_kcontig == AKV && a.b_kcontig == BKV && a.swiglu_map == SWV && a.epi == EPV) \
        return launch32<AKV, BKV, SWV, EPV>(p, s);
    PPS_GEMM32_CASE(true, false, true, EPI_SWIGLU)
    PPS_GEMM32_CASE(true, false, false, EPI_RESID)
    PPS_GEMM32_CASE(true, true, false, EPI_SWIGLU_BWD)
    PPS_GEMM32_CASE(true, true, false, EPI_STORE_F32)
    PPS_GEMM32_CASE(false, false, false, EPI_ACC_F32)
    PPS_GEMM32_CASE(true, false, false, EPI_BIAS_GELU)
    PPS_GEMM32_CASE(true, true, false, EPI_STORE)
    PPS_GEMM32_CASE(true, false, false, EPI_STORE)
#undef PPS_GEMM32_CASE
    return hipErrorInvalidValue;
}

}  // namespace

hipError_t gemm(int dtype, const GemmArgs& a, hipStream_t s) {
    if (a.M <= 0 || a.N <= 0) return hipSuccess;
    if (a.epi == EPI_ACC_F32) {
        int64_t ktot = 0;
        for (int i = 0; i < a.nseg; ++i) ktot += a.seg[i].K;
        if (ktot == 0) return hipSuccess;   // nothing to accumulate
    }
    return dtype == PPS_DTYPE_BF16 ? gemm_bf16(a, s) : gemm_f32(a, s);
}

}  // namespace pps
