// fma_rate.hpp -- the rate at which gfx950 issues non-packed FP32 FMAs, for
// the roofline of the register-tiled VALU kernel (page aerisun.top, section
// "Register Tiling 与线程内复用": the inner loop is an outer product of r_m A
// values and r_n B values held in registers).
//
// Two loops, no memory traffic but one store per thread at the end:
//   kFmaOuter  an 8 x 8 outer product per iteration, every operand in a VGPR
//              (the shape of sgemm_valu_kernel's inner loop), and 8 multiplies
//              that change the A values so nothing is loop-invariant;
//   kFmaScalar 16 independent FMA chains x = x * a + b with a and b kernel
//              arguments (SGPR operands).
// FLOP per thread per iteration: kFmaOuter 2 * 64 + 8 = 136, kFmaScalar
// 2 * 8 * 16 = 256 (8 rounds of the 16 chains).
#pragma once

#include <hip/hip_runtime.h>

namespace mi {

constexpr int kFmaOuter = 0, kFmaScalar = 1;

__global__ __launch_bounds__(256) void fma_outer_kernel(float *out, int iters) {
    float a[8], b[8], c[8][8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        a[j] = threadIdx.x * 1e-3f + j;
        b[j] = 1.0f - j * 1e-4f;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) c[i][j] = 0.f;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 8; ++j) c[i][j] = __builtin_fmaf(a[i], b[j], c[i][j]);
#pragma unroll
        for (int j = 0; j < 8; ++j) a[j] *= 0.999f;
    }
    float s = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) s += c[i][j];
    out[256 * (long long)blockIdx.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void fma_scalar_kernel(float *out, int iters, float a, float b) {
    float x[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = threadIdx.x * 1e-3f + j;
    for (int it = 0; it < iters; ++it) {
#pragma unroll
        for (int r = 0; r < 8; ++r)
#pragma unroll
            for (int j = 0; j < 16; ++j) x[j] = __builtin_fmaf(x[j], a, b);
    }
    float s = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) s += x[j];
    out[256 * (long long)blockIdx.x + threadIdx.x] = s;
}

}  // namespace mi
