// sgemm_mfma.hpp -- FP32 GEMM on the CDNA4 matrix cores.
//
// Blocking (page "GEMM优化原理", sections 基于 shared memory 计算,
// 基于 register 计算 and prefetch 和双缓冲, re-planned for gfx950):
//   * a workgroup of WGM x WGN waves owns a BM x BN tile of C and walks k in
//     steps of BK ("big iterations");
//   * each step stages a BM x BK tile of A and a BK x BN tile of B in one of
//     three LDS buffers.  Whole k steps of aligned operands use gfx950's
//     direct global->LDS loads (buffer_load_dwordx4 ... lds: 16 bytes per
//     lane, no VGPRs involved), issued two steps ahead; the partial last k
//     step and unaligned operands use 16-byte (or element) loads through
//     VGPRs with out-of-range elements stored as zeros (page aerisun.top,
//     section "Shared Tiling 与 block 内复用");
//   * each wave owns a (BM/WGM) x (BN/WGN) sub-tile held as 32 x 32 blocks
//     of v_mfma_f32_32x32x2_f32 accumulators and reads its A and B fragments
//     from LDS one group of 8 k ahead of the MFMAs that use them.
//
// k ordering inside a step.  One 16-byte LDS read gives lane (i, h)
// (i = lane % 32, h = lane / 32) the four A values A[i][8g+4h .. 8g+4h+3] of a
// group g of 8 k values.  MFMA s (s = 0..3) of the group takes A[i][8g+4h+s]
// and B[8g+4h+s][j] from lane (i or j, h): the instruction's two k rows are
// k = 8g+s and 8g+4+s, so the four MFMAs cover the eight k values of the
// group exactly once with matching A and B indices.
//
// LDS layout (64 banks of 4 bytes; a direct load writes 64 lanes x 16 bytes
// to 1 KiB of consecutive LDS, so tiles are unpadded and XOR-swizzled in
// 16-byte chunks instead):
//   * A: BM rows of BK floats (m-major, as in memory); logical chunk c of row
//     r sits at chunk c ^ swz(r), swz(r) = (r * CA / 16) % CA with CA = BK / 4
//     chunks per row.  The 16 lanes of a fragment read (16 consecutive rows,
//     same logical chunk) then cover all 16 bank quads.
//   * B: BK rows of BN floats (k-major, as in memory); rows with bit 2 set
//     swap the two 32-float halves of every 64 floats.  The lane halves of a
//     fragment read take rows k and k+4, which then fall on disjoint banks.
#pragma once

#include <type_traits>

#include "common.hpp"

namespace mi {

template <int BM_, int BN_, int BK_, int WGM_, int WGN_>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int STAGES = 3;                      // LDS buffers in the ring
    static constexpr int WAVES = WGM * WGN;
    static constexpr int NT = 64 * WAVES;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // per-wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 blocks per wave
    static constexpr int GROUPS = BK / 8;                 // groups of 8 k per step
    static constexpr int CA = BK / 4;                     // 16-byte chunks per A row
    static constexpr int CB = BN / 4;                     // 16-byte chunks per B row
    static constexpr int A_PER = BM * CA / NT;            // A chunks per thread per step
    static constexpr int B_PER = BK * CB / NT;            // B chunks per thread per step
    static constexpr int LDS_BYTES = STAGES * (BM * BK + BK * BN) * 4;
    static_assert(BK == 16 || BK == 32, "A swizzle assumes 4 or 8 chunks per row");
    static_assert(BN % 64 == 0, "B swizzle swaps 32-float halves of 64-float blocks");
    static_assert(GROUPS % 2 == 0, "fragment double-buffering needs an even group count");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(BM * CA % NT == 0 && BK * CB % NT == 0, "load slots must divide evenly");
    static_assert(LDS_BYTES <= 160 * 1024, "LDS budget of one workgroup");

    __device__ static constexpr int a_swz(int row) { return (row * CA / 16) % CA; }
    __device__ static constexpr int b_swz(int krow) { return 8 * ((krow >> 2) & 1); }
};

// Word 3 of a raw (untyped) buffer resource on gfx9-class parts: 32-bit data
// format, no swizzling; with stride 0 the range check is a byte count.
constexpr int kBufferWord3 = 0x00020000;

__device__ __forceinline__ __attribute__((address_space(3))) void *lds_ptr(float *p) {
    return (__attribute__((address_space(3))) void *)p;
}

// One buffer_load_dwordx4 ... lds: 16 bytes from base + voffset (per lane)
// into LDS at lds + 16 * lane.  The resource covers 2^31 - 1 bytes from base.
// (Kept out of the kernel template: the host compilation pass drops the
// launch stub of a kernel whose body builds a buffer resource.)
__device__ __forceinline__ void load_lds16(const float *base, float *lds, int voffset) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff,
                                                        kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds), 16, voffset, 0, 0, 0);
}

// Epilogue modes.  kFull: the whole k range, C = alpha*acc + beta*C.
// kPartial: workgroup (tile, slice) sums k in [slice*k_per_split, ...) into
// the raw partial ws[slice] (no alpha/beta).  kAtomic: the same slice sum,
// added as alpha*acc to C with hardware float atomics (C already holds
// beta*C; the order of the additions, hence the last bits, varies from run
// to run).  VEC: A and B allow 16-byte loads.
//
// Pipeline (one barrier per step, buffers used round-robin):
//   top of step t    issue the tile of step t+2 into buffer (t+2) % 3 (direct
//                    loads, or VGPR loads for the masked cases)
//   body             MFMAs of step t on buffer t % 3; the last group also reads
//                    the first fragments of step t+1 from buffer (t+1) % 3
//   end of step t    (VGPR case) write the staged tile; barrier
// Buffer (t+2) % 3 was last read during step t-1, before the barrier that
// ended it; buffer (t+1) % 3 was filled during step t-1 and completed by the
// same barrier (which waits for the direct loads), so the first fragments of
// step t+1 can be read before the barrier of step t and the MFMA stream does
// not wait for LDS at a step boundary.
template <class T, bool VEC, int MODE>
__global__ __launch_bounds__(T::NT) void sgemm_mfma_kernel(GemmArgs p) {
    constexpr bool SPLIT = MODE != kFull;
    // One LDS object per ring stage, always indexed at compile time: the
    // compiler can then tell the buffer a direct load writes from the buffers
    // being read, and does not hold the MFMAs back until the load lands.
    __shared__ __attribute__((aligned(1024))) float As0[T::BM * T::BK];
    __shared__ __attribute__((aligned(1024))) float As1[T::BM * T::BK];
    __shared__ __attribute__((aligned(1024))) float As2[T::BM * T::BK];
    __shared__ __attribute__((aligned(1024))) float Bs0[T::BK * T::BN];
    __shared__ __attribute__((aligned(1024))) float Bs1[T::BK * T::BN];
    __shared__ __attribute__((aligned(1024))) float Bs2[T::BK * T::BN];
    auto a_buf = [&](auto s) -> float * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return As0;
        else if constexpr (S == 1) return As1;
        else return As2;
    };
    auto b_buf = [&](auto s) -> float * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return Bs0;
        else if constexpr (S == 1) return Bs1;
        else return Bs2;
    };

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
    // Whole k steps of aligned operands are loaded directly into LDS (byte
    // offsets inside one tile step must fit the 31-bit buffer offset).  On
    // the m / n edge, rows of A past m and chunks of B past n are clamped to
    // the last valid row / chunk: they only feed outputs that are never
    // stored, and every address stays inside the operands.
    const bool direct_ok = VEC && p.lda < (1LL << 31) / (4LL * T::BM) &&
                           p.ldb < (1LL << 31) / (4LL * T::BK);
    const int ndirect = direct_ok ? (kend - kbeg) / T::BK : 0;
    const int a_row_max = min(T::BM, p.m - m0) - 1;           // last valid row of the A tile
    const int b_chunk_max = (min(T::BN, p.n - n0) - 1) >> 2;  // chunk holding column n-1

    const float *Ablk = p.A + (long long)m0 * p.lda;
    const float *Bblk = p.B + n0;

    // Chunk q = tid + i * NT of a tile (the chunk lane `lane` of wave `wave`
    // writes in the i-th load instruction): its row and logical chunk.
    auto a_chunk = [&](int i, int &row, int &c) {
        const int q = tid + i * T::NT;
        row = q / T::CA;
        c = (q % T::CA) ^ T::a_swz(row);
    };
    auto b_chunk = [&](int i, int &row, int &c) {
        const int q = tid + i * T::NT;
        row = q / T::CB;
        c = (q % T::CB) ^ T::b_swz(row);
    };

    // ---- direct global -> LDS loads (complete, aligned tiles) ---------------
    // buffer_load_dwordx4 ... lds through a per-step buffer resource whose
    // base is the step's first element; each lane supplies a byte offset.
    // (The MUBUF form rather than global_load_lds: the compiler treats a FLAT
    // access that may touch LDS as unordered and would then wait for every
    // outstanding LDS read before each MFMA group.)
    auto load_direct = [&](int step, auto buf) {
        float *as = a_buf(buf), *bs = b_buf(buf);
        const int k0 = kbeg + step * T::BK;
        const float *abase = Ablk + k0;
        const float *bbase = Bblk + (long long)k0 * p.ldb;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            int row, c;
            a_chunk(i, row, c);
            load_lds16(abase, as + (i * T::WAVES + wave) * 256,
                       (int)(4 * ((long long)min(row, a_row_max) * p.lda + 4 * c)));
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            int row, c;
            b_chunk(i, row, c);
            load_lds16(bbase, bs + (i * T::WAVES + wave) * 256,
                       (int)(4 * ((long long)row * p.ldb + 4 * min(c, b_chunk_max))));
        }
    };

    // ---- masked loads through VGPRs (edges, k tail, unaligned) -------------
    struct Stage {
        f32x4 a[T::A_PER], b[T::B_PER];
    };
    auto load_regs = [&](Stage &st, int step) {
        const int k0 = kbeg + step * T::BK;
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i) {
            int row, c;
            a_chunk(i, row, c);
            const float *src = Ablk + (long long)row * p.lda + k0 + 4 * c;
            const int valid = (m0 + row < p.m) ? min(4, kend - (k0 + 4 * c)) : 0;
            st.a[i] = load4_masked<VEC>(src, valid);
        }
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i) {
            int row, c;
            b_chunk(i, row, c);
            const float *src = Bblk + (long long)(k0 + row) * p.ldb + 4 * c;
            const int valid = (k0 + row < kend) ? min(4, p.n - (n0 + 4 * c)) : 0;
            st.b[i] = load4_masked<VEC>(src, valid);
        }
    };
    auto store_regs = [&](const Stage &st, auto buf) {
        float *as = a_buf(buf), *bs = b_buf(buf);
#pragma unroll
        for (int i = 0; i < T::A_PER; ++i)
            *reinterpret_cast<f32x4 *>(as + 4 * (tid + i * T::NT)) = st.a[i];
#pragma unroll
        for (int i = 0; i < T::B_PER; ++i)
            *reinterpret_cast<f32x4 *>(bs + 4 * (tid + i * T::NT)) = st.b[i];
    };

    // ---- accumulators and fragments ----------------------------------------
    f32x16 acc[T::FM][T::FN];
#pragma unroll
    for (int a = 0; a < T::FM; ++a)
#pragma unroll
        for (int b = 0; b < T::FN; ++b)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;

    const int li = lane & 31, lh = lane >> 5;
    int a_row_off[T::FM], a_swz[T::FM], b_col[T::FN];
#pragma unroll
    for (int a = 0; a < T::FM; ++a) {
        const int row = wm * T::WTM + 32 * a + li;
        a_row_off[a] = row * T::BK;
        a_swz[a] = T::a_swz(row);
    }
#pragma unroll
    for (int b = 0; b < T::FN; ++b)
        b_col[b] = ((wn * T::WTN + 32 * b + li) ^ (32 * lh)) + 4 * lh * T::BN;

    struct Frag {
        f32x4 a[T::FM];
        float b[T::FN][4];
    };
    auto read_frag = [&](Frag &f, auto buf, int g) {
        const float *as = a_buf(buf), *bs = b_buf(buf);
#pragma unroll
        for (int a = 0; a < T::FM; ++a)
            f.a[a] = *reinterpret_cast<const f32x4 *>(
                as + a_row_off[a] + 4 * ((2 * g + lh) ^ a_swz[a]));
#pragma unroll
        for (int b = 0; b < T::FN; ++b)
#pragma unroll
            for (int s = 0; s < 4; ++s) f.b[b][s] = bs[b_col[b] + (8 * g + s) * T::BN];
    };
    auto mfma_group = [&](const Frag &f) {
#pragma unroll
        for (int s = 0; s < 4; ++s)
#pragma unroll
            for (int a = 0; a < T::FM; ++a)
#pragma unroll
                for (int b = 0; b < T::FN; ++b)
                    acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x2f32(f.a[a][s], f.b[b][s],
                                                                     acc[a][b], 0, 0, 0);
    };

    // ---- main loop -----------------------------------------------------------
    using S0 = std::integral_constant<int, 0>;
    using S1 = std::integral_constant<int, 1>;
    if (nsteps > 0) {
        Frag f[2];
        // make the tiles of steps 0 and 1 resident
        auto fill = [&](int step, auto buf) {
            if (step < ndirect) {
                load_direct(step, buf);
            } else {
                Stage st;
                load_regs(st, step);
                store_regs(st, buf);
            }
        };
        fill(0, S0{});
        if (nsteps > 1) fill(1, S1{});
        __syncthreads();
        read_frag(f[0], S0{}, 0);

        // One step with its ring position CUR = step % 3 fixed at compile time.
        // DIRECT: the tile two steps ahead is loaded directly (the steady
        // state of interior tiles -- no VGPR loads in that loop, so the
        // compiler's wait counts never hold back the MFMAs); otherwise it goes
        // through VGPRs (edge tiles, unaligned operands, the last k steps).
        auto one_step = [&](int step, auto direct_tag, auto cur) {
            constexpr bool DIRECT = decltype(direct_tag)::value;
            constexpr int CUR = decltype(cur)::value;
            using NXT = std::integral_constant<int, (CUR + 1) % 3>;  // (step + 1) % 3
            using WRT = std::integral_constant<int, (CUR + 2) % 3>;  // (step + 2) % 3
            const bool ahead = step + 2 < nsteps;
            Stage st;
            if (DIRECT)
                load_direct(step + 2, WRT{});
            else if (ahead)
                load_regs(st, step + 2);
            // The fences keep the scheduler from sinking the loads and the
            // next group's LDS reads below the MFMAs that hide them.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < T::GROUPS; ++g) {
                if (g + 1 < T::GROUPS) {
                    read_frag(f[(g + 1) & 1], cur, g + 1);
                } else if (DIRECT || step + 1 < nsteps) {
                    read_frag(f[0], NXT{}, 0);  // GROUPS is even: step+1 starts on set 0
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(f[g & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (!DIRECT && ahead) store_regs(st, WRT{});
            __syncthreads();
        };
        auto dispatch = [&](int step, auto direct_tag) {
            switch (step % 3) {
                case 0: one_step(step, direct_tag, S0{}); break;
                case 1: one_step(step, direct_tag, S1{}); break;
                default: one_step(step, direct_tag, std::integral_constant<int, 2>{}); break;
            }
        };
        using S2 = std::integral_constant<int, 2>;
        int step = 0;
        // Steady state: three steps per iteration, so each ring position is a
        // compile-time constant and the accumulators keep their registers
        // (a runtime switch per step makes the compiler copy them around).
        for (; step + 4 < ndirect; step += 3) {
            one_step(step, std::true_type{}, S0{});
            one_step(step + 1, std::true_type{}, S1{});
            one_step(step + 2, std::true_type{}, S2{});
        }
        for (; step + 2 < ndirect; ++step) dispatch(step, std::true_type{});
        for (; step < nsteps; ++step) dispatch(step, std::false_type{});
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
                    if constexpr (MODE == kPartial) {
                        p.ws[(long long)slice * p.ws_slice + (long long)row * p.n + col] = acc[a][b][r];
                    } else if constexpr (MODE == kAtomic) {
                        unsafeAtomicAdd(p.C + (long long)row * p.ldc + col, p.alpha * acc[a][b][r]);
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
