// Memory-bound kernels of the stage: RMSNorm forward and backward, the
// deterministic dgamma reduction, the elementwise recomputation that feeds
// the weight-gradient GEMMs, the toy block's GELU backward and bias sum, and
// fill/copy.  All accesses are 16-byte vectors along rows (coalesced), with
// one workgroup per row (forward) or per block of rows (backward).
#include "device_common.h"
#include "kernels.h"
#include "pps.h"

namespace pps {
namespace {

// 8 consecutive elements <-> 8 floats.
template <typename S> struct Vec8;
template <> struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[8]) {
        const uint4 q = *reinterpret_cast<const uint4*>(p);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = bf2f(w[i] & 0xffffu);
            v[2 * i + 1] = bf2f(w[i] >> 16);
        }
    }
    static __device__ __forceinline__ void store(uint16_t* p, const float (&v)[8]) {
        uint32_t w[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) w[i] = f2bf(v[2 * i]) | (f2bf(v[2 * i + 1]) << 16);
        *reinterpret_cast<uint4*>(p) = make_uint4(w[0], w[1], w[2], w[3]);
    }
};
template <> struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
        const float4 a = *reinterpret_cast<const float4*>(p);
        const float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void store(float* p, const float (&v)[8]) {
        *reinterpret_cast<float4*>(p) = make_float4(v[0], v[1], v[2], v[3]);
        *reinterpret_cast<float4*>(p + 4) = make_float4(v[4], v[5], v[6], v[7]);
    }
};

__device__ __forceinline__ float block_sum(float v, float* red) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    float s = 0.0f;
    const int nw = blockDim.x >> 6;
    for (int w = 0; w < nw; ++w) s += red[w];
    return s;
}

// One workgroup per row; the row stays in registers between the sum of
// squares and the scaling (each thread holds Q chunks of 8 elements).
template <typename S, int Q>
__global__ __launch_bounds__(256) void rmsnorm_fwd_kernel(const S* __restrict__ x, const float* __restrict__ gamma,
                                                          float eps, int64_t d, float* __restrict__ r,
                                                          S* __restrict__ n, S* __restrict__ xcopy) {
    __shared__ float red[4];
    const int64_t row = blockIdx.x;
    const int64_t nchunk = d / 8;
    const S* xr = x + row * d;
    float v[Q][8];
    float ss = 0.0f;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t c = threadIdx.x + 256 * q;
        if (c < nchunk) {
            Vec8<S>::load(xr + c * 8, v[q]);
#pragma unroll
            for (int i = 0; i < 8; ++i) ss += v[q][i] * v[q][i];
        }
    }
    ss = block_sum(ss, red);
    const float rr = 1.0f / sqrtf(ss / (float)d + eps);
    if (threadIdx.x == 0) r[row] = rr;
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t c = threadIdx.x + 256 * q;
        if (c < nchunk) {
            if (xcopy) Vec8<S>::store(xcopy + row * d + c * 8, v[q]);
            if (n) {
                float gm[8], o[8];
                Vec8<float>::load(gamma + c * 8, gm);
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = (v[q][i] * rr) * gm[i];
                Vec8<S>::store(n + row * d + c * 8, o);
            }
        }
    }
}

constexpr int BWD_ROWS = 16;   // rows per workgroup in the RMSNorm backward

// a = dn gamma; dx = dy + r a - r^3 x (a.x)/d; dgamma partial of the
// workgroup's rows = sum dn x r (kept in registers, written once).  With n,
// also writes the block's RMSNorm output n = (x r) gamma again, computed as
// the forward computed it (same bits), for the weight gradients.
template <typename S, int Q>
__global__ __launch_bounds__(256) void rmsnorm_bwd_kernel(const float* __restrict__ dn, const S* __restrict__ x,
                                                          const float* __restrict__ r, const float* __restrict__ gamma,
                                                          const S* __restrict__ dy, int64_t T, int64_t d,
                                                          S* __restrict__ dx, float* __restrict__ partial,
                                                          S* __restrict__ n) {
    __shared__ float red[4];
    const int64_t nchunk = d / 8;
    float gam[Q][8], gp[Q][8];
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t c = threadIdx.x + 256 * q;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            gam[q][i] = c < nchunk ? gamma[c * 8 + i] : 0.0f;
            gp[q][i] = 0.0f;
        }
    }
    const int64_t r0 = (int64_t)blockIdx.x * BWD_ROWS;
    for (int rr = 0; rr < BWD_ROWS; ++rr) {
        const int64_t row = r0 + rr;
        if (row >= T) break;
        const float rv = r[row];
        float a[Q][8], xv[Q][8], dyv[Q][8];
        float dot = 0.0f;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t c = threadIdx.x + 256 * q;
            if (c < nchunk) {
                float dnv[8];
                Vec8<float>::load(dn + row * d + c * 8, dnv);
                Vec8<S>::load(x + row * d + c * 8, xv[q]);
                Vec8<S>::load(dy + row * d + c * 8, dyv[q]);   // issued before the reduction
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    a[q][i] = dnv[i] * gam[q][i];
                    dot += a[q][i] * xv[q][i];
                    gp[q][i] += dnv[i] * xv[q][i] * rv;
                }
            }
        }
        dot = block_sum(dot, red);
        const float coef = rv * rv * rv * dot / (float)d;
#pragma unroll
        for (int q = 0; q < Q; ++q) {
            const int64_t c = threadIdx.x + 256 * q;
            if (c < nchunk) {
                float o[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) o[i] = dyv[q][i] + rv * a[q][i] - coef * xv[q][i];
                Vec8<S>::store(dx + row * d + c * 8, o);
                if (n) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) o[i] = (xv[q][i] * rv) * gam[q][i];
                    Vec8<S>::store(n + row * d + c * 8, o);
                }
            }
        }
    }
#pragma unroll
    for (int q = 0; q < Q; ++q) {
        const int64_t c = threadIdx.x + 256 * q;
        if (c < nchunk) Vec8<float>::store(partial + (int64_t)blockIdx.x * d + c * 8, gp[q]);
    }
}

// out[j] += sum_w partial[w, j] in a fixed order: thread (c, g) of a workgroup
// sums rows g, g+8, g+16, ... of column j = 32*block + c, then the 8 partial
// sums are added in g order.  32 columns per workgroup: d/32 workgroups fill
// the chip where one thread per column would leave most CUs idle.
__global__ __launch_bounds__(256) void column_reduce_kernel(const float* __restrict__ partial, int rows, int64_t d,
                                                            float* __restrict__ out) {
    __shared__ float part[8][33];
    const int c = threadIdx.x & 31, g = threadIdx.x >> 5;
    const int64_t j = (int64_t)blockIdx.x * 32 + c;
    float s = 0.0f;
    if (j < d)
        for (int w = g; w < rows; w += 8) s += partial[(int64_t)w * d + j];
    part[g][c] = s;
    __syncthreads();
    if (g == 0 && j < d) {
        float t = part[0][c];
#pragma unroll
        for (int k = 1; k < 8; ++k) t += part[k][c];
        out[j] += t;
    }
}

// chunks [0, nx) recompute n = (x r) gamma on [T,d]; chunks [nx, nx+nh)
// recompute h = silu(g) u on [T,f].
template <typename S>
__global__ __launch_bounds__(256) void prep_w_kernel(const S* __restrict__ x, const float* __restrict__ r,
                                                     const float* __restrict__ gamma, const S* __restrict__ g,
                                                     const S* __restrict__ u, int64_t d, int64_t f, int64_t nx,
                                                     int64_t nh, S* __restrict__ n, S* __restrict__ h) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx < nx) {
        const int64_t e = idx * 8, row = e / d, col = e % d;
        float v[8], o[8];
        Vec8<S>::load(x + e, v);
        const float rv = r[row];
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = (v[i] * rv) * gamma[col + i];
        Vec8<S>::store(n + e, o);
    } else if (idx < nx + nh) {
        const int64_t e = (idx - nx) * 8;
        float gv[8], uv[8], o[8];
        Vec8<S>::load(g + e, gv);
        Vec8<S>::load(u + e, uv);
#pragma unroll
        for (int i = 0; i < 8; ++i) o[i] = swiglu_f(gv[i], uv[i]);
        Vec8<S>::store(h + e, o);
    }
}

__global__ __launch_bounds__(256) void gelu_bwd_kernel(const float* __restrict__ dy, const float* __restrict__ z,
                                                       int64_t count, float* __restrict__ dz) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < count) dz[i] = dy[i] * gelu_grad_f(z[i]);
}

__global__ __launch_bounds__(256) void colsum_kernel(const float* __restrict__ a, int64_t T, int64_t d,
                                                     float* __restrict__ out) {
    const int64_t j = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (j >= d) return;
    float s = 0.0f;
    for (int64_t t = 0; t < T; ++t) s += a[t * d + j];
    out[j] += s;
}

// 64 x 64 tile transposes of bf16 through LDS.  Source rows r < rows,
// columns c < cols (cols % 8 == 0); destination row map(c), column r, stride
// ldd (ldd % 8 == 0); destination columns in [rows, ldd) are written as zero.
// map(c) = c, or with grp > 0: (c / grp) * 2 grp + half * grp + c % grp
// (gate/up interleave of the forward weight copy).  The value moved is
// src[r, c] (x rowscale[r], then x colscale[c]: the RMSNorm output (x r) gamma
// as the forward computed it), or with src2 silu(src[r, c]) src2[r, c] (h from
// g and u, the expression the SwiGLU epilogues use).
__global__ __launch_bounds__(256) void tile_transpose_kernel(const uint16_t* __restrict__ src, int64_t rows, int64_t cols,
                                                             int64_t lds, uint16_t* __restrict__ dst, int64_t ldd,
                                                             int grp, int half, const float* __restrict__ rowscale,
                                                             const float* __restrict__ colscale,
                                                             const uint16_t* __restrict__ src2) {
    __shared__ float tile[64][65];
    const int64_t r0 = (int64_t)blockIdx.x * 64, c0 = (int64_t)blockIdx.y * 64;
    const int t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = t + 256 * i, rr = q >> 3, c8 = (q & 7) * 8;
        const int64_t row = r0 + rr, col = c0 + c8;
        float v[8];
        if (row < rows && col < cols) {
            Vec8<uint16_t>::load(src + row * lds + col, v);
            if (src2) {
                float w[8];
                Vec8<uint16_t>::load(src2 + row * lds + col, w);
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] = swiglu_f(v[j], w[j]);
            }
            if (rowscale) {
                const float sc = rowscale[row];
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] *= sc;   // rounded to bf16 by the store
            }
            if (colscale) {
#pragma unroll
                for (int j = 0; j < 8; ++j) v[j] *= colscale[col + j];
            }
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) tile[rr][c8 + j] = v[j];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 2; ++i) {
        const int q = t + 256 * i, cc = q >> 3, r8 = (q & 7) * 8;
        const int64_t col = c0 + cc, row = r0 + r8;
        if (col < cols && row < ldd) {
            float v[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = tile[r8 + j][cc];
            const int64_t drow = grp ? (col / grp) * 2 * grp + (int64_t)half * grp + col % grp : col;
            Vec8<uint16_t>::store(dst + drow * ldd + row, v);
        }
    }
}

template <typename S>
__global__ __launch_bounds__(256) void scale_kernel(S* __restrict__ dst, const S* __restrict__ src, int64_t n,
                                                    float sc) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i < n) Store<S>::store(dst + i, Store<S>::load(src + i) * sc);
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4* __restrict__ p, int64_t n16, uint8_t* __restrict__ tail,
                                                        int ntail) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t k = i; k < n16; k += stride) p[k] = make_uint4(0u, 0u, 0u, 0u);
    if (i < ntail) tail[i] = 0;
}

__global__ __launch_bounds__(256) void copy_kernel(uint4* __restrict__ dst, const uint4* __restrict__ src, int64_t n16,
                                                   uint8_t* __restrict__ dtail, const uint8_t* __restrict__ stail,
                                                   int ntail) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * 256;
    for (int64_t k = i; k < n16; k += stride) dst[k] = src[k];
    if (i < ntail) dtail[i] = stail[i];
}

inline unsigned grid_for(int64_t work, int64_t per_block = 256, int64_t cap = 1 << 20) {
    int64_t g = (work + per_block - 1) / per_block;
    if (g > cap) g = cap;
    return (unsigned)(g < 1 ? 1 : g);
}

}  // namespace

hipError_t rmsnorm_fwd(int dtype, const void* x, const float* gamma, float eps, int64_t T, int64_t d, float* r,
                       void* n, void* xcopy, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t q = (d / 8 + 255) / 256;   // chunks of 8 per thread
#define PPS_RF(S, Q)                                                                                       \
    hipLaunchKernelGGL((rmsnorm_fwd_kernel<S, Q>), dim3((unsigned)T), dim3(256), 0, s, static_cast<const S*>(x), \
                       gamma, eps, d, r, static_cast<S*>(n), static_cast<S*>(xcopy))
    if (dtype == PPS_DTYPE_BF16) {
        if (q <= 1) PPS_RF(uint16_t, 1); else if (q <= 2) PPS_RF(uint16_t, 2); else if (q <= 4) PPS_RF(uint16_t, 4);
        else if (q <= 8) PPS_RF(uint16_t, 8); else return hipErrorInvalidValue;
    } else {
        if (q <= 1) PPS_RF(float, 1); else if (q <= 2) PPS_RF(float, 2); else if (q <= 4) PPS_RF(float, 4);
        else if (q <= 8) PPS_RF(float, 8); else return hipErrorInvalidValue;
    }
#undef PPS_RF
    return hipGetLastError();
}

int rmsnorm_bwd_partial_rows(int64_t T) { return (int)((T + BWD_ROWS - 1) / BWD_ROWS); }

template <typename S>
static hipError_t rmsnorm_bwd_t(const float* dn, const void* x, const float* r, const float* gamma, const void* dy,
                                int64_t T, int64_t d, void* dx, float* partial, void* n, hipStream_t s) {
    const int64_t q = (d / 8 + 255) / 256;
    const dim3 grid((unsigned)rmsnorm_bwd_partial_rows(T));
    const S* xs = static_cast<const S*>(x);
    const S* dys = static_cast<const S*>(dy);
    S* dxs = static_cast<S*>(dx);
    S* ns = static_cast<S*>(n);
    if (q <= 1) hipLaunchKernelGGL((rmsnorm_bwd_kernel<S, 1>), grid, dim3(256), 0, s, dn, xs, r, gamma, dys, T, d, dxs, partial, ns);
    else if (q <= 2) hipLaunchKernelGGL((rmsnorm_bwd_kernel<S, 2>), grid, dim3(256), 0, s, dn, xs, r, gamma, dys, T, d, dxs, partial, ns);
    else if (q <= 4) hipLaunchKernelGGL((rmsnorm_bwd_kernel<S, 4>), grid, dim3(256), 0, s, dn, xs, r, gamma, dys, T, d, dxs, partial, ns);
    else if (q <= 8) hipLaunchKernelGGL((rmsnorm_bwd_kernel<S, 8>), grid, dim3(256), 0, s, dn, xs, r, gamma, dys, T, d, dxs, partial, ns);
    else return hipErrorInvalidValue;
    return hipGetLastError();
}

hipError_t rmsnorm_bwd(int dtype, const float* dn, const void* x, const float* r, const float* gamma, const void* dy,
                       int64_t T, int64_t d, void* dx, float* partial, int* n_partial, void* n, hipStream_t s) {
    *n_partial = 0;
    if (T <= 0) return hipSuccess;
    *n_partial = rmsnorm_bwd_partial_rows(T);
    return dtype == PPS_DTYPE_BF16 ? rmsnorm_bwd_t<uint16_t>(dn, x, r, gamma, dy, T, d, dx, partial, n, s)
                                   : rmsnorm_bwd_t<float>(dn, x, r, gamma, dy, T, d, dx, partial, n, s);
}

hipError_t column_reduce_acc(const float* partial, int rows, int64_t d, float* out, hipStream_t s) {
    if (rows <= 0 || d <= 0) return hipSuccess;
    hipLaunchKernelGGL(column_reduce_kernel, dim3((unsigned)((d + 31) / 32)), dim3(256), 0, s, partial, rows, d, out);
    return hipGetLastError();
}

hipError_t prep_w(int dtype, const void* x, const float* r, const float* gamma, const void* g, const void* u,
                  int64_t T, int64_t d, int64_t f, void* n, void* h, hipStream_t s) {
    if (T <= 0) return hipSuccess;
    const int64_t nx = T * d / 8, nh = T * f / 8;
    const dim3 grid(grid_for(nx + nh, 256, (int64_t)1 << 31));
    if (dtype == PPS_DTYPE_BF16)
        hipLaunchKernelGGL(prep_w_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<const uint16_t*>(x), r, gamma,
                           static_cast<const uint16_t*>(g), static_cast<const uint16_t*>(u), d, f, nx, nh,
                           static_cast<uint16_t*>(n), static_cast<uint16_t*>(h));
    else
        hipLaunchKernelGGL(prep_w_kernel<float>, grid, dim3(256), 0, s, static_cast<const float*>(x), r, gamma,
                           static_cast<const float*>(g), static_cast<const float*>(u), d, f, nx, nh,
                           static_cast<float*>(n), static_cast<float*>(h));
    return hipGetLastError();
}

hipError_t gelu_bwd(const float* dy, const float* z, int64_t count, float* dz, hipStream_t s) {
    if (count <= 0) return hipSuccess;
    hipLaunchKernelGGL(gelu_bwd_kernel, dim3(grid_for(count, 256, (int64_t)1 << 31)), dim3(256), 0, s, dy, z, count, dz);
    return hipGetLastError();
}

hipError_t colsum_acc(const float* a, int64_t T, int64_t d, float* out, hipStream_t s) {
    if (T <= 0 || d <= 0) return hipSuccess;
    hipLaunchKernelGGL(colsum_kernel, dim3(grid_for(d)), dim3(256), 0, s, a, T, d, out);
    return hipGetLastError();
}

hipError_t transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst, int64_t ldd, int grp,
                          int half, hipStream_t s, const float* rowscale, const float* colscale, const void* src2) {
    if (cols <= 0 || ldd <= 0) return hipSuccess;
    if (cols % 8 || ldd % 8 || lds % 8) return hipErrorInvalidValue;
    const dim3 grid((unsigned)((ldd + 63) / 64), (unsigned)((cols + 63) / 64));
    hipLaunchKernelGGL(tile_transpose_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(src), rows, cols, lds,
                       static_cast<uint16_t*>(dst), ldd, grp, half, rowscale, colscale,
                       static_cast<const uint16_t*>(src2));
    return hipGetLastError();
}

hipError_t scale(int dtype, void* dst, const void* src, int64_t n, float sc, hipStream_t s) {
    if (n <= 0) return hipSuccess;
    const dim3 grid(grid_for(n, 256, (int64_t)1 << 31));
    if (dtype == PPS_DTYPE_BF16)
        hipLaunchKernelGGL(scale_kernel<uint16_t>, grid, dim3(256), 0, s, static_cast<uint16_t*>(dst),
                           static_cast<const uint16_t*>(src), n, sc);
    else
        hipLaunchKernelGGL(scale_kernel<float>, grid, dim3(256), 0, s, static_cast<float*>(dst),
                           static_cast<const float*>(src), n, sc);
    return hipGetLastError();
}

hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s) {
    if (bytes <= 0) return hipSuccess;
    const int64_t n16 = bytes / 16;
    const int ntail = (int)(bytes % 16);
    uint8_t* tail = static_cast<uint8_t*>(p) + n16 * 16;
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid_for(n16 > 0 ? n16 : 1, 256, 8192)), dim3(256), 0, s,
                       static_cast<uint4*>(p), n16, tail, ntail);
    return hipGetLastError();
}

hipError_t copy_bytes(void* dst, const void* src, int64_t bytes, hipStream_t s) {
    if (bytes <= 0) return hipSuccess;
    const int64_t n16 = bytes / 16;
    const int ntail = (int)(bytes % 16);
    hipLaunchKernelGGL(copy_kernel, dim3(grid_for(n16 > 0 ? n16 : 1, 256, 8192)), dim3(256), 0, s,
                       static_cast<uint4*>(dst), static_cast<const uint4*>(src), n16,
                       static_cast<uint8_t*>(dst) + n16 * 16, static_cast<const uint8_t*>(src) + n16 * 16, ntail);
    return hipGetLastError();
}

}  // namespace pps
