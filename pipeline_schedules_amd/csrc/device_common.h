// Device helpers shared by the HIP kernels of the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pps {

// bf16 <-> fp32.  bf16 is the upper half of an IEEE fp32 word; conversion
// to bf16 rounds to nearest, ties to even, and keeps NaN a NaN (gfx950's
// v_cvt_pk_bf16_f32 does both in one instruction for two values).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf2f(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Two fp32 values -> packed bf16 pair (a in the low half).
__device__ __forceinline__ uint32_t pack2_bf(float a, float b) {
    const bf16x2_t v = {(__bf16)a, (__bf16)b};
    return __builtin_bit_cast(uint32_t, v);
}

__device__ __forceinline__ uint32_t f2bf(float f) { return pack2_bf(f, 0.0f) & 0xffffu; }

// Round an fp32 value to the nearest bf16 value, returned as fp32.
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

template <typename S> struct Store;
template <> struct Store<uint16_t> {
    static __device__ __forceinline__ float load(const uint16_t* p) { return bf2f(*p); }
    static __device__ __forceinline__ void store(uint16_t* p, float v) { *p = (uint16_t)f2bf(v); }
    static __device__ __forceinline__ float round(float v) { return round_bf(v); }
};
template <> struct Store<float> {
    static __device__ __forceinline__ float load(const float* p) { return *p; }
    static __device__ __forceinline__ void store(float* p, float v) { *p = v; }
    static __device__ __forceinline__ float round(float v) { return v; }
};

// sigmoid with the hardware reciprocal (about 1 ulp), not an IEEE divide.
__device__ __forceinline__ float sigmoid_f(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// h = silu(g) * u with silu(g) = g * sigmoid(g).
__device__ __forceinline__ float swiglu_f(float g, float u) { return g * sigmoid_f(g) * u; }

// Gradient of h = silu(g) u: du = dh silu(g); dg = dh u s (1 + g (1 - s)).
__device__ __forceinline__ void swiglu_bwd_f(float dh, float g, float u, float& dg, float& du) {
    const float s = sigmoid_f(g);
    du = dh * g * s;
    dg = dh * u * s * (1.0f + g * (1.0f - s));
}

// Both at once with one sigmoid: h = silu(g) u, and dg, du for dh.  Same
// expressions, so the same bits, as swiglu_f and swiglu_bwd_f.
__device__ __forceinline__ void swiglu_h_bwd_f(float dh, float g, float u, float& h, float& dg, float& du) {
    const float s = sigmoid_f(g);
    h = g * s * u;
    du = dh * g * s;
    dg = dh * u * s * (1.0f + g * (1.0f - s));
}

// Exact (erf-based) GELU and its derivative Phi(z) + z phi(z).
__device__ __forceinline__ float gelu_f(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}
__device__ __forceinline__ float gelu_grad_f(float z) {
    const float cdf = 0.5f * (1.0f + erff(z * 0.70710678118654752f));
    const float pdf = 0.39894228040143268f * expf(-0.5f * z * z);
    return cdf + z * pdf;
}

}  // namespace pps
