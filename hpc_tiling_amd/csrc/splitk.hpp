// splitk.hpp -- combine of split-K partials, and the beta-only update.
//
// Combine: C_ij = alpha * sum_s ws[s][i*n + j] + beta * C_ij.
// The partial sums are reduced in two levels (page aerisun.top, sections
// "先在线程内累加，再交换部分和" and "Warp shuffle 的数据交换"): first inside
// a lane over a strided subset of the slices, then across lanes with
// register exchanges instead of LDS.
//
// One wave handles a chunk of 64 consecutive outputs (in the dense m x n
// order of the workspace), then the chunk a grid's worth of waves further
// on (the block count is capped at kCombineMaxBlocks).  Lane (q, v) = (lane / 16, lane % 16) loads the
// float4 at chunk offset 4v from slices s = q, q+4, q+8, ...: every load
// instruction of the wave reads four 256-byte runs, one per slice group.
// The four lanes v, v+16, v+32, v+48 then hold partial sums of the same four
// outputs; two butterfly steps add them:
//     x += (x from lane ^ 32)   -- v_permlane32_swap_b32
//     x += (x from lane ^ 16)   -- v_permlane16_swap_b32
// after which all four lanes hold the total, and lane (q, v) stores output
// 4v + q, so the 64 lanes write the chunk's 64 outputs once each.  Lanes past
// the end of the output add zeros and still take part in every exchange.
// The order of additions is fixed, so results are deterministic.
#pragma once

#include "common.hpp"

namespace mi {

constexpr long long kCombineMaxBlocks = 1 << 20;

__global__ __launch_bounds__(256) void splitk_combine_kernel(const float *__restrict__ ws,
                                                             long long ws_slice, int splits,
                                                             int m, int n, float alpha,
                                                             float beta, float *C,
                                                             long long ldc) {
    const long long mn = (long long)m * n;
    const long long chunks = (mn + 63) / 64;
    const int lane = threadIdx.x & 63;
    const int q = lane >> 4, v = lane & 15;
    // the chunk is the same for the whole wave: every lane takes part in the
    // exchanges below, or none does
    for (long long chunk = (long long)blockIdx.x * 4 + (threadIdx.x >> 6); chunk < chunks;
         chunk += (long long)gridDim.x * 4) {
        const long long f = chunk * 64 + 4 * v;

        f32x4 s4 = {0.f, 0.f, 0.f, 0.f};
        if (f < mn) {
            // Slices are padded to a multiple of 64 floats, so the whole float4
            // is inside slice s even when mn is not a multiple of 4.
            const float *src = ws + f;
            auto at = [&](int s) {
                return *reinterpret_cast<const f32x4 *>(src + (long long)s * ws_slice);
            };
            int s = q;
#pragma unroll 4
            for (; s + 12 < splits; s += 16) {
                const f32x4 x0 = at(s), x1 = at(s + 4), x2 = at(s + 8), x3 = at(s + 12);
                s4 += (x0 + x1) + (x2 + x3);
            }
            for (; s < splits; s += 4) s4 += at(s);
        }
        const float t0 = sum_over_lane_quarters(s4[0]);
        const float t1 = sum_over_lane_quarters(s4[1]);
        const float t2 = sum_over_lane_quarters(s4[2]);
        const float t3 = sum_over_lane_quarters(s4[3]);
        const float tot = q == 0 ? t0 : q == 1 ? t1 : q == 2 ? t2 : t3;

        const long long o = chunk * 64 + 4 * v + q;
        if (o < mn) {
            const long long i = o / n, j = o - i * n;
            float *dst = C + i * ldc + j;
            float r = alpha * tot;
            if (beta != 0.f) r = __builtin_fmaf(beta, *dst, r);
            *dst = r;
        }
    }
}

// C <- beta * C over the m x n logical extent (beta == 0 writes zeros without
// reading C).  Used when k == 0 or alpha == 0.
__global__ __launch_bounds__(256) void scale_c_kernel(int m, int n, float beta, float *C,
                                                      long long ldc) {
    const long long total = (long long)m * n;
    for (long long e = (long long)blockIdx.x * 256 + threadIdx.x; e < total;
         e += (long long)gridDim.x * 256) {
        const long long i = e / n, j = e - i * n;
        float *dst = C + i * ldc + j;
        *dst = beta != 0.f ? beta * *dst : 0.f;
    }
}

}  // namespace mi
