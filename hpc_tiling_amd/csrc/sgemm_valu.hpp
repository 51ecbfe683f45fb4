// sgemm_valu.hpp -- FP32 GEMM on the vector ALUs, register-tiled.
//
// The geometry is the worked example of page "GEMM优化原理" (section
// 一个具体的例子): 128 x 128 tiles of C per workgroup, k step 8, 256 threads,
// each thread accumulating an 8 x 8 block of C as 8 outer products of 8 A
// values by 8 B values per k step (64 FMAs per "small iteration"; page
// aerisun.top, section "Register Tiling 与线程内复用").  It is kept as a
// measured comparison for the matrix-core path: on gfx950 a wave64 FP32 FMA
// retires 128 FLOP per clock per CU, half the FP32 MFMA rate.
//
// Layout on gfx950:
//   * A is stored in LDS k-major (transposed while staging) so that a thread's
//     8 A values for one k are two 16-byte reads; B stays k-major as in
//     memory.  Rows hold 128 (+8 pad) floats.
//   * A thread owns rows {4ty..4ty+3} U {64+4ty..64+4ty+3} and the same split
//     of columns with tx, so the 16 threads of a row group read 16
//     consecutive float4 of B (no bank conflict) and broadcast A.
//   * Global loads of step t+1 go to VGPRs before the FMAs of step t and to
//     the other LDS buffer after them (page "gemm优化", section on prefetch).
#pragma once

#include "common.hpp"

namespace mi {

struct ValuTile {
    static constexpr int BM = 128, BN = 128, BK = 8, RM = 8, RN = 8;
    static constexpr int NT = (BM / RM) * (BN / RN);  // 256
    static constexpr int LDS_S = 128 + 8;
};

template <bool VEC>
__global__ __launch_bounds__(256) void sgemm_valu_kernel(GemmArgs p) {
    using T = ValuTile;
    __shared__ __attribute__((aligned(16))) float As[2][T::BK * T::LDS_S];
    __shared__ __attribute__((aligned(16))) float Bs[2][T::BK * T::LDS_S];

    const int tid = threadIdx.x;
    const int tx = tid & 15, ty = tid >> 4;

    int tm, tn;
    grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int nsteps = (p.k + T::BK - 1) / T::BK;
    const bool full_m = m0 + T::BM <= p.m;
    const bool full_n = n0 + T::BN <= p.n;

    // A slot: row tid/2, k quad tid%2; B slot: k row tid/32, column quad tid%32.
    const int ar = tid >> 1, ac = 4 * (tid & 1);
    const int br = tid >> 5, bc = 4 * (tid & 31);
    const float *asrc = p.A + (long long)(m0 + ar) * p.lda + ac;
    const float *bsrc = p.B + (long long)br * p.ldb + n0 + bc;
    f32x4 ra, rb;

    auto load_step = [&](int step) {
        const int k0 = step * T::BK;
        const bool full_k = k0 + T::BK <= p.k;
        if (VEC && full_m && full_k) {
            ra = *reinterpret_cast<const f32x4 *>(asrc + k0);
        } else {
            const int valid = (m0 + ar < p.m) ? min(4, p.k - (k0 + ac)) : 0;
            ra = load4_masked<VEC>(asrc + k0, valid);
        }
        const float *b = bsrc + (long long)k0 * p.ldb;
        if (VEC && full_n && full_k) {
            rb = *reinterpret_cast<const f32x4 *>(b);
        } else {
            const int valid = (k0 + br < p.k) ? min(4, p.n - (n0 + bc)) : 0;
            rb = load4_masked<VEC>(b, valid);
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int c = 0; c < 4; ++c) As[buf][(ac + c) * T::LDS_S + ar] = ra[c];
        *reinterpret_cast<f32x4 *>(&Bs[buf][br * T::LDS_S + bc]) = rb;
    };

    float acc[T::RM][T::RN];
#pragma unroll
    for (int i = 0; i < T::RM; ++i)
#pragma unroll
        for (int j = 0; j < T::RN; ++j) acc[i][j] = 0.f;

    if (nsteps > 0) {
        load_step(0);
        store_step(0);
        __syncthreads();
    }
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const bool more = step + 1 < nsteps;
        if (more) load_step(step + 1);
#pragma unroll
        for (int kk = 0; kk < T::BK; ++kk) {
            const float *arow = &As[buf][kk * T::LDS_S];
            const float *brow = &Bs[buf][kk * T::LDS_S];
            const f32x4 a0 = *reinterpret_cast<const f32x4 *>(arow + 4 * ty);
            const f32x4 a1 = *reinterpret_cast<const f32x4 *>(arow + 64 + 4 * ty);
            const f32x4 b0 = *reinterpret_cast<const f32x4 *>(brow + 4 * tx);
            const f32x4 b1 = *reinterpret_cast<const f32x4 *>(brow + 64 + 4 * tx);
            const float av[8] = {a0[0], a0[1], a0[2], a0[3], a1[0], a1[1], a1[2], a1[3]};
            const float bv[8] = {b0[0], b0[1], b0[2], b0[3], b1[0], b1[1], b1[2], b1[3]};
#pragma unroll
            for (int i = 0; i < T::RM; ++i)
#pragma unroll
                for (int j = 0; j < T::RN; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
        }
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // Epilogue: row i of the micro tile is C row m0 + 4ty + i (i < 4) or
    // m0 + 64 + 4ty + i - 4; columns likewise with tx.
#pragma unroll
    for (int i = 0; i < T::RM; ++i) {
        const int row = m0 + (i < 4 ? 4 * ty + i : 64 + 4 * ty + i - 4);
        if (row >= p.m) continue;
        float *crow = p.C + (long long)row * p.ldc;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int col = n0 + 64 * h + 4 * tx;
            f32x4 v;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = p.alpha * acc[i][4 * h + j];
            if (p.c_vec && col + 3 < p.n) {
                f32x4 *dst = reinterpret_cast<f32x4 *>(crow + col);
                if (p.beta != 0.f) {
                    const f32x4 c = *dst;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(p.beta, c[j], v[j]);
                }
                *dst = v;
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (col + j < p.n) {
                        float r = v[j];
                        if (p.beta != 0.f) r = __builtin_fmaf(p.beta, crow[col + j], r);
                        crow[col + j] = r;
                    }
                }
            }
        }
    }
}

}  // namespace mi
