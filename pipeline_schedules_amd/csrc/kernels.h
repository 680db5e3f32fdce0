// Host-side launch interface of the HIP kernels (library-internal).
//
// GEMM convention: C[M,N] = sum_k A[m,k] B[k,n], fp32 accumulation.
//   A "K-contiguous": A[m,k] at A + m*lda + k     (row-major activations)
//   A "M-contiguous": A[m,k] at A + k*lda + m     (activation transposed)
//   B "K-contiguous": B[k,n] at B + n*ldb + k     (weight used transposed)
//   B "N-contiguous": B[k,n] at B + k*ldb + n     (weight [in,out] / activation)
// Up to two K segments are summed into one accumulator (dn = dg Wg^T + du Wu^T).
// Every pointer is 16-byte aligned; the contiguous extent of every operand
// (K for K-contiguous, M or N otherwise) is a multiple of 8.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

namespace pps {

enum Epi {
    EPI_STORE_F32 = 0,   // out0[m*ld0+n] = acc                           (float)
    EPI_RESID = 1,       // out0[m*ld0+n] = in0[m*ldi0+n] + acc           (storage type)
    EPI_SWIGLU = 2,      // g,u pair -> out0=g, out1=u, out2=h=silu(g)*u  (storage type, ld0);
                         // bf16 GEMM: g, u = rowscale[m] * acc first, h from the unrounded g, u
    EPI_SWIGLU_BWD = 3,  // dh=acc; g=in0,u=in1 (ldi0) -> out0[m*ld0+n]=dg, out0[..+nsplit]=du,
                         // and if out2: h = silu(g) u at out2[m*ldi0+n] (fp32 GEMM) or
                         // out2[n*ld2+m] (bf16 GEMM; with out3 also dg, du transposed)
    EPI_ACC_F32 = 4,     // n <  nsplit: out0[m*ld0+n] += acc; else out1[m*ld1+n-nsplit] += acc
                         // (bf16: nsplit and ld1 multiples of 8)
    EPI_BIAS_GELU = 5,   // z = acc + bias[n]; out0 = z, out1 = GELU(z)   (fp32 only)
    EPI_STORE = 6,       // out0[m*ld0+n] = acc                           (storage type)
};

struct EpiArgs {
    void* out0 = nullptr;
    void* out1 = nullptr;
    void* out2 = nullptr;
    int64_t ld0 = 0, ld1 = 0;
    const void* in0 = nullptr;
    const void* in1 = nullptr;
    int64_t ldi0 = 0;
    int64_t nsplit = 0;
    const float* bias = nullptr;
    int64_t ld2 = 0;   // SwiGLU backward, bf16 GEMM: h is written transposed, out2[n*ld2 + m]
                       // (needs M and N multiples of 256, ld2 % 8 == 0)
    const float* rowscale = nullptr;   // SwiGLU, bf16 GEMM: per output row factor (RMSNorm r)
    void* out3 = nullptr;   // SwiGLU backward, bf16 GEMM: dg and du also written transposed,
                            // out3[n*ld2 + m] and out3[(nsplit + n)*ld2 + m] (full tiles, as out2)
};

struct GemmSeg {
    const void* A = nullptr;
    const void* B = nullptr;
    const void* B2 = nullptr;   // second B matrix of the SwiGLU gate/up map
    int64_t lda = 0, ldb = 0, K = 0;
};

struct GemmArgs {
    int64_t M = 0, N = 0;       // output rows / columns (SwiGLU map: N = ffn)
    int nseg = 1;
    GemmSeg seg[2];
    // bf16: both K-contiguous; fp32: any combination.
    bool a_kcontig = true;
    bool b_kcontig = false;
    bool swiglu_map = false;    // B columns: per 2*H group, H from B then H from B2
    int epi = EPI_STORE;
    EpiArgs e;
};

// dtype: PPS_DTYPE_BF16 (MFMA) or PPS_DTYPE_FP32.  Returns a hipError_t.
hipError_t gemm(int dtype, const GemmArgs& a, hipStream_t s);

// r[t] = (mean_j x[t,j]^2 + eps)^-1/2;  n[t,j] = x[t,j] r[t] gamma[j] (skipped
// when n is null: the bf16 forward folds gamma into its weight copy and applies
// r in the gate/up GEMM's epilogue); xcopy (optional) receives x.  One
// workgroup per row.
hipError_t rmsnorm_fwd(int dtype, const void* x, const float* gamma, float eps,
                       int64_t T, int64_t d, float* r, void* n, void* xcopy, hipStream_t s);

// a = dn gamma; dx = dy + r a - r^3 x (a.x)/d; partial[w, j] = sum over the
// rows of workgroup w of dn x r.  Returns the number of partial rows used.
// If n is given, also writes n = (x r) gamma [T, d] exactly as rmsnorm_fwd.
hipError_t rmsnorm_bwd(int dtype, const float* dn, const void* x, const float* r,
                       const float* gamma, const void* dy, int64_t T, int64_t d,
                       void* dx, float* partial, int* n_partial, void* n, hipStream_t s);
int rmsnorm_bwd_partial_rows(int64_t T);

// out[j] += sum_{w < rows} partial[w, j]   (fixed order)
hipError_t column_reduce_acc(const float* partial, int rows, int64_t d, float* out, hipStream_t s);

// n = x r gamma  ([T,d]);  h = silu(g) u  ([T,f]).
hipError_t prep_w(int dtype, const void* x, const float* r, const float* gamma,
                  const void* g, const void* u, int64_t T, int64_t d, int64_t f,
                  void* n, void* h, hipStream_t s);

// dz = dy * GELU'(z)   (fp32)
hipError_t gelu_bwd(const float* dy, const float* z, int64_t count, float* dz, hipStream_t s);

// out[j] += sum_t a[t, j]  (fp32, fixed order)
hipError_t colsum_acc(const float* a, int64_t T, int64_t d, float* out, hipStream_t s);

// Tiled bf16 transpose: dst[map(c), r] = v(r, c) rounded to bf16, for
// r < rows, c < cols; dst columns in [rows, ldd) are zeroed.  v = src[r, c],
// times rowscale[r] and then colscale[c] when given; with src2 (same layout
// as src) v = silu(src[r, c]) src2[r, c] instead (h from g and u).
// map(c) = c, or (c/grp)*2grp + half*grp + c%grp with grp > 0.  cols, lds and
// ldd must be multiples of 8.
hipError_t transpose_bf16(const void* src, int64_t rows, int64_t cols, int64_t lds, void* dst, int64_t ldd, int grp,
                          int half, hipStream_t s, const float* rowscale = nullptr, const float* colscale = nullptr,
                          const void* src2 = nullptr);

// Rows of the interleaved gate/up weight copy used by the forward GEMM.
int64_t swiglu_b_rows(int64_t ffn);

// Workgroups (256 x 256 output tiles, one per CU at a time) of a bf16 GEMM
// with M x N outputs.
int64_t gemm_bf16_tiles(int64_t M, int64_t N);

// dst = src * scale (n elements of the storage type)
hipError_t scale(int dtype, void* dst, const void* src, int64_t n, float scale, hipStream_t s);

hipError_t fill_zero(void* p, int64_t bytes, hipStream_t s);

// Device address of this device's fixed no-alloc array (PPS_NOALLOC_MAX_BYTES),
// looked up once per device.  Returns a PPS_* status.
int noalloc_scratch(char** out);
hipError_t copy_bytes(void* dst, const void* src, int64_t bytes, hipStream_t s);

}  // namespace pps
