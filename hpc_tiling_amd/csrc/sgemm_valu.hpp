// sgemm_valu.hpp -- FP32 GEMM on the vector ALUs, register-tiled.
//
// The geometry is the worked example of page "GEMM优化原理" (section
// 一个具体的例子): 128 x 128 tiles of C per workgroup, k step 8, 256 threads,
// each thread accumulating an 8 x 8 block of C as 8 outer products of 8 A
// values by 8 B values per k step (64 FMAs per "small iteration"; page
// aerisun.top, section "Register Tiling 与线程内复用").  It is kept as a
// measured comparison for the matrix-core path.  Its bound is the FP32
// vector peak (157.3 TFLOP/s on MI355X, the same as the FP32 matrix peak):
// on gfx950 a non-packed v_fma_f32 with all operands in VGPRs issues every
// two cycles per SIMD, 256 FLOP per clock per CU (an 8 x 8 outer-product
// loop without memory sustains 136 TFLOP/s), while FMA chains with an SGPR
// operand issue every four cycles.
//
// Layout on gfx950:
//   * A is stored in LDS k-major (transposed while staging) so that a thread's
//     8 A values for one k are two 16-byte reads; B stays k-major as in
//     memory.  Rows hold 128 (+8 pad) floats.
//   * A thread owns rows {4ty..4ty+3} U {64+4ty..64+4ty+3} and the same split
//     of columns with tx, so the 16 threads of a row group read 16
//     consecutive float4 of B (no bank conflict) and broadcast A.
//   * Global loads run two k steps ahead through two register sets (page
//     "gemm优化", section on prefetch, with one more step of distance): the
//     tile of step t+2 is loaded before the FMAs of step t, and the tile of
//     step t+1 (loaded a step earlier) goes to the other LDS buffer after
//     them.  With one k group (below) at 2048^3 each SIMD holds a single
//     wave of this kernel, so the load latency must fit in the FMAs of a
//     step or more: one step (2048 FMA cycles) was not enough.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mi {

struct ValuTile {
    static constexpr int BM = 128, BN = 128, BK = 8, RM = 8, RN = 8;
    static constexpr int NT = (BM / RM) * (BN / RN);  // 256 threads per k group
    static constexpr int LDS_S = 128 + 8;
    static constexpr int STAGE = BK * LDS_S;           // floats of one A or B stage
};

// KG k groups of 256 threads share a tile: group g takes the k steps
// g, g + KG, g + 2 KG, ... with LDS buffers of its own, and at the end group 0
// adds the other groups' sums, in group order, through LDS.  With KG = 2 a
// CU's one workgroup of a one-round grid has two waves per SIMD, so that one
// wave's LDS waits and barriers are covered by the other's FMAs.
template <bool VEC, int KG>
__global__ __launch_bounds__(256 * KG) void sgemm_valu_kernel(GemmArgs p) {
    using T = ValuTile;
    // KG groups x two buffers x (A, B) stages; with KG > 1 the same memory
    // later holds the sums of groups 1 .. KG-1 (64 per thread).
    constexpr int STAGES_F = KG * 2 * 2 * T::STAGE;
    constexpr int XCH_F = (KG - 1) * T::RM * T::RN * T::NT;
    __shared__ __attribute__((aligned(16))) float smem[STAGES_F > XCH_F ? STAGES_F : XCH_F];

    const int g = KG > 1 ? __builtin_amdgcn_readfirstlane((int)threadIdx.x / T::NT) : 0;
    const int tid = (int)threadIdx.x % T::NT;
    const int tx = tid & 15, ty = tid >> 4;
    // buffer b of the group: its A stage, then its B stage
    auto As = [&](int b) { return smem + (g * 2 + b) * 2 * T::STAGE; };
    auto Bs = [&](int b) { return smem + (g * 2 + b) * 2 * T::STAGE + T::STAGE; };

    int tm, tn;
    grouped_tile(xcd_contiguous(blockIdx.x, gridDim.x), p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int nsteps = (p.k + T::BK - 1) / T::BK;
    // every group runs the same number of steps (and barriers); steps past
    // the end load zeros
    const int nloc = (nsteps + KG - 1) / KG;
    auto gstep = [&](int j) { return KG * j + g; };
    const bool full_m = m0 + T::BM <= p.m;
    const bool full_n = n0 + T::BN <= p.n;

    // A slot: row tid/2, k quad tid%2; B slot: k row tid/32, column quad tid%32.
    const int ar = tid >> 1, ac = 4 * (tid & 1);
    const int br = tid >> 5, bc = 4 * (tid & 31);
    const float *asrc = p.A + (long long)(m0 + ar) * p.lda + ac;
    const float *bsrc = p.B + (long long)br * p.ldb + n0 + bc;
    struct Regs {
        f32x4 a, b;
    };
    Regs r0, r1;  // the staged tiles of two consecutive steps

    auto load_step = [&](Regs &r, int step) {
        const int k0 = step * T::BK;
        const bool full_k = k0 + T::BK <= p.k;
        if (VEC && full_m && full_k) {
            r.a = *reinterpret_cast<const f32x4 *>(asrc + k0);
        } else {
            const int valid = (m0 + ar < p.m) ? min(4, p.k - (k0 + ac)) : 0;
            r.a = load4_masked<VEC>(asrc + k0, valid);
        }
        const float *b = bsrc + (long long)k0 * p.ldb;
        if (VEC && full_n && full_k) {
            r.b = *reinterpret_cast<const f32x4 *>(b);
        } else {
            const int valid = (k0 + br < p.k) ? min(4, p.n - (n0 + bc)) : 0;
            r.b = load4_masked<VEC>(b, valid);
        }
    };
    // Interior tile, all k of the step in range: plain 16-byte loads.
    auto load_full = [&](Regs &r, int step) {
        const int k0 = step * T::BK;
        r.a = *reinterpret_cast<const f32x4 *>(asrc + k0);
        r.b = *reinterpret_cast<const f32x4 *>(bsrc + (long long)k0 * p.ldb);
    };
    auto store_step = [&](const Regs &r, int buf) {
#pragma unroll
        for (int c = 0; c < 4; ++c) As(buf)[(ac + c) * T::LDS_S + ar] = r.a[c];
        *reinterpret_cast<f32x4 *>(Bs(buf) + br * T::LDS_S + bc) = r.b;
    };

    float acc[T::RM][T::RN];
#pragma unroll
    for (int i = 0; i < T::RM; ++i)
#pragma unroll
        for (int j = 0; j < T::RN; ++j) acc[i][j] = 0.f;

    if (nloc > 0) {
        load_step(r0, gstep(0));
        if (nloc > 1) load_step(r1, gstep(1));
        store_step(r0, 0);
        __syncthreads();
    }
    // Step `step` computes from LDS buffer step % 2.  On entry `cur` holds
    // nothing live and `nxt` holds the tile of step+1; `cur` is refilled with
    // the tile of step+2, and `nxt` is written to the other buffer.
    // Fragments: the 8 A and 8 B values of one k, read one k ahead of the
    // FMAs that use them (two sets); the fences keep the compiler from
    // hoisting every read of a step to its top, which would hold 128 VGPRs.
    struct Frag {
        f32x4 a0, a1, b0, b1;
    };
    auto read_frag = [&](Frag &f, int buf, int kk) {
        const float *arow = As(buf) + kk * T::LDS_S;
        const float *brow = Bs(buf) + kk * T::LDS_S;
        f.a0 = *reinterpret_cast<const f32x4 *>(arow + 4 * ty);
        f.a1 = *reinterpret_cast<const f32x4 *>(arow + 64 + 4 * ty);
        f.b0 = *reinterpret_cast<const f32x4 *>(brow + 4 * tx);
        f.b1 = *reinterpret_cast<const f32x4 *>(brow + 64 + 4 * tx);
    };
    auto fma_block = [&](const Frag &f) {
        const float av[8] = {f.a0[0], f.a0[1], f.a0[2], f.a0[3], f.a1[0], f.a1[1], f.a1[2], f.a1[3]};
        const float bv[8] = {f.b0[0], f.b0[1], f.b0[2], f.b0[3], f.b1[0], f.b1[1], f.b1[2], f.b1[3]};
#pragma unroll
        for (int i = 0; i < T::RM; ++i)
#pragma unroll
            for (int j = 0; j < T::RN; ++j) acc[i][j] = __builtin_fmaf(av[i], bv[j], acc[i][j]);
    };
    // FULL: the steady state of an interior tile (the tile of step+2 exists
    // and is whole), without any branch in the step.
    // `step` counts the group's own steps (global step gstep(step)).
    auto one_step = [&](int step, Regs &cur, Regs &nxt, auto full_tag) {
        constexpr bool FULL = decltype(full_tag)::value;
        const int buf = step & 1;
        if (FULL)
            load_full(cur, gstep(step + 2));
        else if (step + 2 < nloc)
            load_step(cur, gstep(step + 2));
        Frag f[2];
        read_frag(f[0], buf, 0);
#pragma unroll
        for (int kk = 0; kk < T::BK; ++kk) {
            if (kk + 1 < T::BK) read_frag(f[(kk + 1) & 1], buf, kk + 1);
            __builtin_amdgcn_sched_barrier(0);
            fma_block(f[kk & 1]);
            __builtin_amdgcn_sched_barrier(0);
        }
        if (FULL || step + 1 < nloc) store_step(nxt, buf ^ 1);
        __syncthreads();
    };
    // Two steps per iteration, so the register sets alternate at compile
    // time; the steady loop stops while the group's tile three steps ahead
    // is whole.
    int step = 0;
    if (VEC && full_m && full_n) {
        const int nfull = p.k / T::BK;
        for (; gstep(step + 3) < nfull; step += 2) {
            one_step(step, r0, r1, std::true_type{});
            one_step(step + 1, r1, r0, std::true_type{});
        }
    }
    for (; step + 1 < nloc; step += 2) {
        one_step(step, r0, r1, std::false_type{});
        one_step(step + 1, r1, r0, std::false_type{});
    }
    if (step < nloc) one_step(step, r0, r1, std::false_type{});

    if constexpr (KG > 1) {
        // The last step ended with a barrier: no wave reads a stage any more.
        // Value (i, j) of thread t of group q sits at (q-1, i, j, t): a wave
        // writes and reads 64 consecutive floats.
        float *xch = smem;
        if (g > 0) {
#pragma unroll
            for (int i = 0; i < T::RM; ++i)
#pragma unroll
                for (int j = 0; j < T::RN; ++j)
                    xch[(((g - 1) * T::RM + i) * T::RN + j) * T::NT + tid] = acc[i][j];
        }
        __syncthreads();
        if (g > 0) return;
#pragma unroll
        for (int q = 1; q < KG; ++q)
#pragma unroll
            for (int i = 0; i < T::RM; ++i)
#pragma unroll
                for (int j = 0; j < T::RN; ++j)
                    acc[i][j] += xch[(((q - 1) * T::RM + i) * T::RN + j) * T::NT + tid];
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
                // C is touched once: nontemporal access.
                f32x4 *dst = reinterpret_cast<f32x4 *>(crow + col);
                if (p.beta != 0.f) {
                    const f32x4 c = __builtin_nontemporal_load(dst);
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(p.beta, c[j], v[j]);
                }
                __builtin_nontemporal_store(v, dst);
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
