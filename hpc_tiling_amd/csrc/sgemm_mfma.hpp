// sgemm_mfma.hpp -- FP32 GEMM on the CDNA4 matrix cores.
//
// Blocking (page "GEMM优化原理", sections 基于 shared memory 计算,
// 基于 register 计算 and prefetch 和双缓冲, re-planned for gfx950):
//   * a workgroup of WGM x WGN waves owns a BM x BN tile of C and walks k in
//     steps of BK ("big iterations");
//   * each step stages a BM x BK tile of A and a BK x BN tile of B from HBM
//     through VGPRs into one of two LDS buffers with 16-byte loads whose
//     adjacent lanes read adjacent addresses (page aerisun.top, sections on
//     coalescing and float4); out-of-range elements are stored as zeros
//     (page aerisun.top, section "Shared Tiling 与 block 内复用");
//   * each wave owns a (BM/WGM) x (BN/WGN) sub-tile held as 32 x 32 blocks
//     of v_mfma_f32_32x32x2_f32 accumulators and reads its A and B fragments
//     from LDS;
//   * the global loads of step t+1 are issued before the MFMAs of step t and
//     written to the other LDS buffer after them, so one barrier per step
//     suffices.
//
// k ordering inside a step.  One 16-byte LDS read gives lane (i, h)
// (i = lane % 32, h = lane / 32) the four A values A[i][8g+4h .. 8g+4h+3] of a
// group g of 8 k values.  MFMA s (s = 0..3) of the group takes A[i][8g+4h+s]
// and B[8g+4h+s][j] from lane (i or j, h): the instruction's two k rows are
// k = 8g+s and 8g+4+s, so the four MFMAs cover the eight k values of the
// group exactly once with matching A and B indices.
//
// LDS layout.  A: BM rows of BK (+4 pad) floats (m-major, as in memory); with
// the pad, the 16-byte fragment reads of 16 consecutive rows fall on
// disjoint bank quads.  B: BK rows of BN (+8 pad) floats (k-major, as in
// memory); the pad puts rows k and k+4 (read by the two lane halves) half a
// bank cycle apart.
#pragma once

#include "common.hpp"

namespace mi {

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int WAVES = WGM * WGN;
    static constexpr int NT = 64 * WAVES;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // per-wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 blocks per wave
    static constexpr int LDA_S = BK + 4;                  // LDS row stride of A
    static constexpr int LDB_S = BN + 8;                  // LDS row stride of B
    static constexpr int A_Q = BK / 4;                    // float4 per A row
    static constexpr int B_Q = BN / 4;                    // float4 per B row
    static constexpr int A_PER = BM * BK / 4 / NT;        // A float4 per thread
    static constexpr int B_PER = BK * BN / 4 / NT;        // B float4 per thread
    static constexpr int LDS_BYTES = 2 * (BM * LDA_S + BK * LDB_S) * 4;
    static_assert(BK % 8 == 0, "k step must hold whole groups of 8");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BM * BK / 4 % NT == 0 && BK * BN / 4 % NT == 0, "load slots must divide evenly");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup");
};

// SPLIT: workgroup (tile, slice) sums k in [slice*k_per_split, ...) into the
// raw partial ws[slice] (no alpha/beta); otherwise the full k range is summed
// and C = alpha*acc + beta*C is written.  VEC: A and B allow 16-byte loads.
template <class T, bool VEC, bool SPLIT>
__global__ __launch_bounds__(T::NT) void sgemm_mfma_kernel(GemmArgs p) {
    __shared__ __attribute__((aligned(16))) float As[2][T::BM * T::LDA_S];
    __shared__ __attribute__((aligned(16))) float Bs[2][T::BK * T::LDB_S];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WGN, wn = wave % T::WGN;

    // ---- which tile (and slice) this workgroup computes -------------------
    int id = xcd_contiguous(blockIdx.x, gridDim.x);
    int slice = 0;
    if (SPLIT) {
        const int tiles = p.tiles_m * p.tiles_n;
        slice = id / tiles;
        id -= slice * tiles;
    }
    int tm, tn;
    grouped_tile(id, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
    const int m0 = tm * T::BM, n0 = tn * T::BN;
    const int kbeg = SPLIT ? slice * p.k_per_split : 0;
    const int kend = SPLIT ? min(p.k, kbeg + p.k_per_split) : p.k;
    const int nsteps = (kend - kbeg + T::BK - 1) / T::BK;
    const bool full_m = m0 + T::BM <= p.m;
    const bool full_n = n0 + T::BN <= p.n;

    // ---- global -> VGPR staging ------------------------------------------
    f32x4 ra[T::A_PER], rb[T::B_PER];
    const float *Ablk = p.A + (long long)m0 * p.lda;
    const float *Bblk = p.B + n0;

    auto load_step = [&](int step) {
        const int k0 = kbeg + step * T::BK;
        const bool full_k = k0 + T::BK <= kend;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const int s = tid + i * T::NT;
            const int r = s / T::A_Q, c = 4 * (s % T::A_Q);
            const float *src = Ablk + (long long)r * p.lda + k0 + c;
            if (VEC && full_m && full_k) {
                ra[i] = *reinterpret_cast<const f32x4 *>(src);
            } else {
                const int valid = (m0 + r < p.m) ? min(4, kend - (k0 + c)) : 0;
                ra[i] = load4_masked<VEC>(src, valid);
            }
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int s = tid + i * T::NT;
            const int r = s / T::B_Q, c = 4 * (s % T::B_Q);
            const float *src = Bblk + (long long)(k0 + r) * p.ldb + c;
            if (VEC && full_n && full_k) {
                rb[i] = *reinterpret_cast<const f32x4 *>(src);
            } else {
                const int valid = (k0 + r < kend) ? min(4, p.n - (n0 + c)) : 0;
                rb[i] = load4_masked<VEC>(src, valid);
            }
        }
    };
    auto store_step = [&](int buf) {
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            const int s = tid + i * T::NT;
            const int r = s / T::A_Q, c = 4 * (s % T::A_Q);
            *reinterpret_cast<f32x4 *>(&As[buf][r * T::LDA_S + c]) = ra[i];
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            const int s = tid + i * T::NT;
            const int r = s / T::B_Q, c = 4 * (s % T::B_Q);
            *reinterpret_cast<f32x4 *>(&Bs[buf][r * T::LDB_S + c]) = rb[i];
        }
    };

    // ---- accumulators -----------------------------------------------------
    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int a = 0; a < T::FM; ++a)
#pragma unroll
        for (int b = 0; b < T::FN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int li = lane & 31, lh = lane >> 5;
    const int a_off = (wm * T::WTM + li) * T::LDA_S + 4 * lh;
    const int b_off = 4 * lh * T::LDB_S + wn * T::WTN + li;

    if (nsteps > 0) {
        load_step(0);
        store_step(0);
        __syncthreads();
    }
    for (int step = 0; step < nsteps; ++step) {
        const int buf = step & 1;
        const bool more = step + 1 < nsteps;
        if (more) load_step(step + 1);

        const float *as = &As[buf][a_off];
        const float *bs = &Bs[buf][b_off];
#pragma unroll
        for (int g = 0; g < T::BK / 8; ++g) {
            f32x4 af[T::FM];
            float bf[T::FN][4];
#pragma unroll
            for (int a = 0; a < T::FM; ++a)
                af[a] = *reinterpret_cast<const f32x4 *>(as + a * 32 * T::LDA_S + 8 * g);
#pragma unroll
            for (int b = 0; b < T::FN; ++b)
#pragma unroll
                for (int s = 0; s < 4; ++s) bf[b][s] = bs[(8 * g + s) * T::LDB_S + 32 * b];
#pragma unroll
            for (int s = 0; s < 4; ++s)
#pragma unroll
                for (int a = 0; a < T::FM; ++a)
#pragma unroll
                    for (int b = 0; b < T::FN; ++b)
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(af[a][s], bf[b][s],
                                                                         acc[a][b], 0, 0, 0);
        }
        if (more) store_step(buf ^ 1);
        __syncthreads();
    }

    // ---- epilogue -----------------------------------------------------------
    // Accumulator register r of lane (j, h) holds C row 8*(r/4) + 4*h + r%4,
    // column j of its 32x32 block.
#pragma unroll
    for (int a = 0; a < T::FM; ++a) {
#pragma unroll
        for (int b = 0; b < T::FN; ++b) {
            const int col = n0 + wn * T::WTN + 32 * b + li;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * T::WTM + 32 * a + 8 * (r >> 2) + 4 * lh + (r & 3);
                if (row < p.m && col < p.n) {
                    if (SPLIT) {
                        p.ws[(long long)slice * p.ws_slice + (long long)row * p.n + col] = acc[a][b][r];
                    } else {
                        float *dst = p.C + (long long)row * p.ldc + col;
                        float v = p.alpha * acc[a][b][r];
                        if (p.beta != 0.f) v = __builtin_fmaf(p.beta, *dst, v);
                        *dst = v;
                    }
                }
            }
        }
    }
}

}  // namespace mi
