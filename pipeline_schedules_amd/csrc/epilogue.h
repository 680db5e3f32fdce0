// GEMM epilogues, shared by the bf16 (MFMA) and fp32 GEMM kernels.
//
// Each epilogue consumes one fp32 accumulator value at output (row, col).
// The SwiGLU epilogue consumes a (gate, up) pair for one hidden column.
// The block math is the stage's: y = x + h Wd (residual); h = silu(g) u;
// the SwiGLU backward dg, du; fp32 in-place weight-gradient accumulation
// (gradients are summed over micro-batches, then one step: [1F1B §5.1]).
#pragma once

#include "device_common.h"
#include "kernels.h"

namespace pps {

template <int EPI, typename S>
__device__ __forceinline__ void epi_apply(const EpiArgs& e, int64_t row, int64_t col, float v) {
    if constexpr (EPI == EPI_STORE_F32) {
        static_cast<float*>(e.out0)[row * e.ld0 + col] = v;
    } else if constexpr (EPI == EPI_STORE) {
        Store<S>::store(static_cast<S*>(e.out0) + row * e.ld0 + col, v);
    } else if constexpr (EPI == EPI_RESID) {
        const float x = Store<S>::load(static_cast<const S*>(e.in0) + row * e.ldi0 + col);
        Store<S>::store(static_cast<S*>(e.out0) + row * e.ld0 + col, x + v);
    } else if constexpr (EPI == EPI_SWIGLU_BWD) {
        const float g = Store<S>::load(static_cast<const S*>(e.in0) + row * e.ldi0 + col);
        const float u = Store<S>::load(static_cast<const S*>(e.in1) + row * e.ldi0 + col);
        float dg, du;
        swiglu_bwd_f(v, g, u, dg, du);
        S* o = static_cast<S*>(e.out0) + row * e.ld0;
        Store<S>::store(o + col, dg);
        Store<S>::store(o + e.nsplit + col, du);
        if (e.out2) Store<S>::store(static_cast<S*>(e.out2) + row * e.ldi0 + col, swiglu_f(g, u));
    } else if constexpr (EPI == EPI_ACC_F32) {
        if (col < e.nsplit) static_cast<float*>(e.out0)[row * e.ld0 + col] += v;
        else static_cast<float*>(e.out1)[row * e.ld1 + (col - e.nsplit)] += v;
    } else if constexpr (EPI == EPI_BIAS_GELU) {
        const float z = v + e.bias[col];
        static_cast<float*>(e.out0)[row * e.ld0 + col] = z;
        static_cast<float*>(e.out1)[row * e.ld1 + col] = gelu_f(z);
    }
}

// Gate/up pair of hidden column `col`: stores g and u (rounded to the storage
// type) and h = silu(g) u computed from the stored values, so a later
// recomputation of h from the stash gives the same bits.
template <typename S>
__device__ __forceinline__ void epi_swiglu(const EpiArgs& e, int64_t row, int64_t col, float g, float u) {
    const float gs = Store<S>::round(g);
    const float us = Store<S>::round(u);
    const int64_t o = row * e.ld0 + col;
    Store<S>::store(static_cast<S*>(e.out0) + o, gs);
    Store<S>::store(static_cast<S*>(e.out1) + o, us);
    Store<S>::store(static_cast<S*>(e.out2) + o, swiglu_f(gs, us));
}

}  // namespace pps
