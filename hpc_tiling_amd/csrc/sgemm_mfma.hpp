// sgemm_mfma.hpp -- FP32 GEMM on the CDNA4 matrix cores.
//
// Blocking (page "GEMM优化原理", sections 基于 shared memory 计算,
// 基于 register 计算 and prefetch 和双缓冲, re-planned for gfx950):
//   * a workgroup of WGM x WGN waves owns a BM x BN tile of C and walks k in
//     steps of BK ("big iterations");
//   * each step stages a BM x BK tile of A and a BK x BN tile of B in a ring
//     of three LDS buffers (two for tiles built for two workgroups per CU,
//     four for the 16-wave 128 x 128 x 32 tile).  Whole k steps use gfx950's
//     direct global->LDS loads (buffer_load_dwordx4 ... lds, 16 bytes per
//     lane, for aligned operands; buffer_load_dword ... lds, 4 bytes per
//     lane, otherwise; no VGPRs involved), issued one step ahead per buffer
//     beyond the first; the partial last k step (and
//     tiles whose byte offsets exceed the buffer range) use masked 16-byte
//     or element loads through VGPRs with out-of-range elements stored as
//     zeros (page aerisun.top, section "Shared Tiling 与 block 内复用");
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
// Operand layouts.  Each operand supplies an E x BK slice per k step (E = BM
// for A, BN for B) and sits in memory in one of two layouts:
//   * k-contiguous: element (e, t) at X[e*ld + t] -- A as given, or B given
//     transposed (B^T stored n x k);
//   * e-contiguous: element (e, t) at X[t*ld + e] -- B as given, or A given
//     transposed (A^T stored k x m).
// The LDS tile keeps the memory layout (a direct load cannot transpose), and
// the fragment read adapts to it: from a k-contiguous tile one 16-byte read
// gives the four k values above; from an e-contiguous tile four 4-byte reads
// (one per k row) do.  Transposed reads are the bank-conflict case of page
// "GEMM优化原理" (section 基于 register 计算); the swizzles below remove them.
//
// LDS layout (64 banks of 4 bytes; a direct load writes 64 lanes x 16 bytes
// to 1 KiB of consecutive LDS, so tiles are unpadded and XOR-swizzled in
// 16-byte chunks instead):
//   * k-contiguous tile: E rows of BK floats; logical chunk c of row r sits
//     at chunk c ^ swz(r), swz(r) = (r * CH / 16) % CH with CH = BK / 4
//     chunks per row.  The 16 lanes of a fragment read (16 consecutive rows,
//     same logical chunk) then cover all 16 bank quads.
//   * e-contiguous tile: BK rows of E floats; rows with bit 2 set swap the two
//     32-float halves of every 64 floats.  The lane halves of a fragment read
//     take rows k and k+4, which then fall on disjoint banks.
#pragma once

#include <type_traits>

#include "common.hpp"
#include "kloop.hpp"

namespace mi {

template <int BM_, int BN_, int BK_, int WGM_, int WGN_, int STAGES_ = 3,
          int WGS_ = (STAGES_ == 2 ? 2 : 1)>
struct MfmaTile {
    static constexpr int BM = BM_, BN = BN_, BK = BK_, WGM = WGM_, WGN = WGN_;
    static constexpr int STAGES = STAGES_;                // LDS buffers in the ring (2 to 4)
    static constexpr int DIST = STAGES - 1;               // steps a load runs ahead
    static constexpr int WAVES = WGM * WGN;
    static constexpr int NT = 64 * WAVES;
    // Workgroups per CU the register allocation must allow (a two-stage ring
    // relies on another resident workgroup to cover its barrier stalls), and
    // the waves per SIMD that makes.
    static constexpr int WGS = WGS_;
    static constexpr int WAVES_PER_SIMD = (WAVES * WGS + 3) / 4;
    static constexpr int WTM = BM / WGM, WTN = BN / WGN;  // per-wave tile
    static constexpr int FM = WTM / 32, FN = WTN / 32;    // 32x32 blocks per wave
    static constexpr int GROUPS = BK / 8;                 // groups of 8 k per step
    static constexpr int LDS_BYTES = STAGES * (BM * BK + BK * BN) * 4;
    static_assert(GROUPS % 2 == 0, "fragment double-buffering needs an even group count");
    static_assert(WTM % 32 == 0 && WTN % 32 == 0, "wave tile must be whole 32x32 blocks");
    static_assert(WGS * lds_granules(LDS_BYTES) <= kLdsGranulesPerCu,
                  "WGS workgroups must fit one CU's LDS");
    // the LDS holds only one workgroup per CU
    static constexpr bool ONE_PER_CU = 2 * lds_granules(LDS_BYTES) > kLdsGranulesPerCu;
    static_assert(STAGES >= 2 && STAGES <= 4, "ring of two to four buffers");
};

// Four floats of an e-contiguous fragment (read one by one).
struct Vals4 {
    float v[4];
    __device__ float &operator[](int s) { return v[s]; }
    __device__ float operator[](int s) const { return v[s]; }
};

// Staging and fragment reads of one operand (E = BM or BN) of tile T.
// KROWS: the operand is e-contiguous, so LDS rows are k rows.
template <class T, int E, bool KROWS>
struct Operand {
    static constexpr bool K_ROWS = KROWS;
    static constexpr int ROWS = KROWS ? T::BK : E;         // LDS tile rows
    static constexpr int CH = KROWS ? E / 4 : T::BK / 4;   // 16-byte chunks per row
    static constexpr int PER = ROWS * CH / T::NT;          // chunks per thread per step
    static constexpr int ROW_WORDS = 4 * CH;               // floats per LDS row
    static constexpr int PER4 = ROWS * ROW_WORDS / T::NT;  // 4-byte direct loads per lane per step
    static constexpr int ELEMS = E * T::BK;
    using Frag = std::conditional_t<KROWS, Vals4, f32x4>;  // four k values of one lane
    static_assert(KROWS ? E % 64 == 0 : (T::BK == 16 || T::BK == 32),
                  "swizzle assumes 64-float rows (e-contiguous) or 4 or 8 chunks per row");
    static_assert(ROWS * CH % T::NT == 0, "load slots must divide evenly");

    __device__ static constexpr int swz(int row) {
        return KROWS ? 8 * ((row >> 2) & 1) : (row * CH / 16) % CH;
    }
    // Chunk q = tid + i * NT of a tile (the chunk lane `lane` of wave `wave`
    // writes in the i-th load instruction): its LDS row and logical chunk.
    __device__ static void chunk(int tid, int i, int &row, int &c) {
        const int q = tid + i * T::NT;
        row = q / CH;
        c = (q % CH) ^ swz(row);
    }
    // Largest in-range coordinate on the e edge, in the unit the clamp of a
    // direct load uses: a row (k-contiguous) or a chunk (e-contiguous).
    __device__ static int clamp_limit(int e_valid) { return KROWS ? (e_valid - 1) >> 2 : e_valid - 1; }
    // First element of the workgroup's e range (e0 = its first row of op(X)),
    // and from there the first element of the tile of k step k0.
    __device__ static const float *block_base(const float *X, long long ld, int e0) {
        return KROWS ? X + e0 : X + (long long)e0 * ld;
    }
    __device__ static const float *tile_base(const float *blk, long long ld, int k0) {
        return KROWS ? blk + (long long)k0 * ld : blk + k0;
    }
    // Byte offset from the tile base of chunk (row, c), edge rows or chunks
    // clamped to `lim` (they feed only outputs that are never stored).
    __device__ static int direct_offset(int row, int c, long long ld, int lim) {
        return KROWS ? (int)(4 * ((long long)row * ld + 4 * min(c, lim)))
                     : (int)(4 * ((long long)min(row, lim) * ld + 4 * c));
    }
    // 4-byte direct loads (operands not 16-byte aligned): word w of the
    // swizzled LDS tile is loaded from the element the layout puts there (the
    // chunk swizzle undone), e clamped to e_last.  The lanes of one load cover
    // one or two row segments, only in permuted chunk order.
    __device__ static int word_offset(int w, long long ld, int e_last) {
        const int r = w / ROW_WORDS, u = w % ROW_WORDS;
        const int col = 4 * ((u >> 2) ^ swz(r)) + (u & 3);
        return KROWS ? (int)(4 * ((long long)r * ld + min(col, e_last)))
                     : (int)(4 * ((long long)min(r, e_last) * ld + col));
    }
    // k index, within its step, of word w of the swizzled LDS tile (the word
    // word_offset(w, ...) loads).
    __device__ static int word_k(int w) {
        const int r = w / ROW_WORDS, u = w % ROW_WORDS;
        return KROWS ? r : 4 * ((u >> 2) ^ swz(r)) + (u & 3);
    }
    // Direct loads need every byte offset of a tile to fit the 31-bit range.
    __device__ static bool direct_fits(long long ld) {
        return ld < (1LL << 31) / (4LL * (KROWS ? T::BK : E));
    }
    // Masked 16-byte load of chunk (row, c) of the tile at (e0, k0): elements
    // with e >= e_end or k >= k_end read as zero.
    template <bool VEC>
    __device__ static f32x4 load_masked(const float *X, long long ld, int e0, int e_end, int k0,
                                        int k_end, int row, int c) {
        if (KROWS) {
            const float *src = X + (long long)(k0 + row) * ld + e0 + 4 * c;
            const int valid = (k0 + row < k_end) ? min(4, e_end - (e0 + 4 * c)) : 0;
            return load4_masked<VEC>(src, valid);
        } else {
            const float *src = X + (long long)(e0 + row) * ld + k0 + 4 * c;
            const int valid = (e0 + row < e_end) ? min(4, k_end - (k0 + 4 * c)) : 0;
            return load4_masked<VEC>(src, valid);
        }
    }
    // Per-lane fragment addressing for the 32-row block starting at wave-tile
    // coordinate e_blk: lane (l, h) = (lane % 32, lane / 32).
    __device__ static void frag_setup(int e_blk, int li, int lh, int &off, int &sw) {
        const int e = e_blk + li;
        if (KROWS) {
            off = (e ^ (32 * lh)) + 4 * lh * E;
            sw = 0;
        } else {
            off = e * T::BK;
            sw = swz(e);
        }
    }
    // The four values lane (l, h) feeds MFMAs s = 0..3 of group g: X[e][8g+4h+s],
    // from word frag_addr(...) of the tile on.
    __device__ static int frag_addr(int off, int sw, int g, int lh) {
        return KROWS ? off + 8 * g * E : off + 4 * ((2 * g + lh) ^ sw);
    }
    __device__ static void frag_read(Frag &f, const float *buf, int addr) {
        if constexpr (KROWS) {
#pragma unroll
            for (int s = 0; s < 4; ++s) f[s] = buf[addr + s * E];
        } else {
            f = *reinterpret_cast<const f32x4 *>(buf + addr);
        }
    }
};

// Word 3 of a raw (untyped) buffer resource on gfx9-class parts: 32-bit data
// format, no swizzling; with stride 0 the range check is a byte count.
constexpr int kBufferWord3 = 0x00020000;

// A lane offset past the 2^31 - 1 bytes every buffer resource here covers:
// the load is out of range, reads nothing and returns zero.
constexpr int kOutOfRange = (int)0x80000000u;

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

// The same with buffer_load_dword ... lds: 4 bytes per lane into LDS at
// lds + 4 * lane.
__device__ __forceinline__ void load_lds4(const float *base, float *lds, int voffset) {
    const auto rsrc = __builtin_amdgcn_make_buffer_rsrc(const_cast<float *>(base), 0, 0x7fffffff,
                                                        kBufferWord3);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, lds_ptr(lds), 4, voffset, 0, 0, 0);
}

// The barrier at the end of a step of a four-buffer ring: this wave's LDS
// reads and all but its newest N vector-memory operations (the direct loads
// just issued, for the step three ahead) complete, then the workgroup meets.
// s_waitcnt fields on gfx9-class parts: vmcnt in bits 3:0 and 15:14, expcnt
// in bits 6:4 (7: no wait), lgkmcnt in bits 11:8.  The empty asm statements
// keep the compiler from moving memory accesses across the wait or the
// barrier (the barrier intrinsic alone does not order them).
template <int N>
__device__ __forceinline__ void barrier_keep_newest() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    constexpr int kImm = (N & 15) | ((N >> 4) << 14) | (7 << 4);
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(kImm);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Epilogue modes.  kFull: the whole k range, C = alpha*acc + beta*C.
// kPartial: workgroup (tile, slice) sums k in [slice*k_per_split, ...) into
// the raw partial ws[slice] (no alpha/beta).  kAtomic: the same slice sum,
// added as alpha*acc to C with hardware float atomics (C already holds
// beta*C; the order of the additions, hence the last bits, varies from run
// to run).  kStreamK: whole tiles, then even shares of the (tile, k step)
// iterations of the rest, cut tiles left in workspace slots for the fixup
// kernel (see the stream-K branch at the end).  VEC: A and B allow 16-byte
// loads.
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
// not wait for LDS at a step boundary.  A two-buffer ring (T::STAGES == 2)
// loads one step ahead instead: buffer (t+1) % 2 was read during step t-1,
// and step t+1's first fragments are read after the barrier of step t; the
// other workgroup resident on the CU keeps the matrix cores busy meanwhile.
// A four-buffer ring loads three steps ahead, into buffer (t+3) % 4 (read
// during step t-1), behind the first MFMA group of step t, and its barrier
// waits only for the loads issued a step earlier: every load has nearly two
// steps to land instead of one (the three-buffer barrier waits for all of
// them), and the loads' issue no longer holds back the first MFMAs after the
// barrier.
template <class T, bool VEC, int MODE, bool TA = false, bool TB = false>
__global__ __launch_bounds__(T::NT) __attribute__((amdgpu_waves_per_eu(T::WAVES_PER_SIMD)))
void sgemm_mfma_kernel(GemmArgs p) {
    constexpr bool SPLIT = MODE == kPartial || MODE == kAtomic;
    using OA = Operand<T, T::BM, TA>;    // A: k-contiguous unless given transposed
    using OB = Operand<T, T::BN, !TB>;   // B: n-contiguous unless given transposed
    // One LDS object per ring stage, always indexed at compile time: the
    // compiler can then tell the buffer a direct load writes from the buffers
    // being read, and does not hold the MFMAs back until the load lands.
    __shared__ __attribute__((aligned(1024))) float As0[OA::ELEMS];
    __shared__ __attribute__((aligned(1024))) float As1[OA::ELEMS];
    __shared__ __attribute__((aligned(1024))) float As2[T::STAGES > 2 ? OA::ELEMS : 4];
    __shared__ __attribute__((aligned(1024))) float As3[T::STAGES > 3 ? OA::ELEMS : 4];
    __shared__ __attribute__((aligned(1024))) float Bs0[OB::ELEMS];
    __shared__ __attribute__((aligned(1024))) float Bs1[OB::ELEMS];
    __shared__ __attribute__((aligned(1024))) float Bs2[T::STAGES > 2 ? OB::ELEMS : 4];
    __shared__ __attribute__((aligned(1024))) float Bs3[T::STAGES > 3 ? OB::ELEMS : 4];
    auto a_buf = [&](auto s) -> float * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return As0;
        else if constexpr (S == 1) return As1;
        else if constexpr (S == 2) return As2;
        else return As3;
    };
    auto b_buf = [&](auto s) -> float * {
        constexpr int S = decltype(s)::value;
        if constexpr (S == 0) return Bs0;
        else if constexpr (S == 1) return Bs1;
        else if constexpr (S == 2) return Bs2;
        else return Bs3;
    };

    // (not const: the stream-K segment loop launders them, see there)
    int tid = threadIdx.x;
    int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / T::WGN, wn = wave % T::WGN;

    // ---- the tile (and k range) being computed ------------------------------
    // Set once per workgroup, or once per segment of its stream-K range.
    int m0 = 0, n0 = 0, kbeg = 0, kend = 0, nsteps = 0, ndirect = 0, a_lim = 0, b_lim = 0;
    const float *Ablk = p.A, *Bblk = p.B;
    // Whole k steps are loaded directly into LDS (byte offsets inside one
    // tile step must fit the 31-bit buffer offset): 16 bytes per lane for
    // aligned operands, 4 bytes otherwise.  On the m / n edge, rows, chunks
    // or elements past the edge are clamped to the last valid one: they only
    // feed outputs that are never stored, and every address stays inside the
    // operands.
    const bool direct_ok = OA::direct_fits(p.lda) && OB::direct_fits(p.ldb);
    auto set_tile = [&](int tile, int kb, int ke) {
        int tm, tn;
        grouped_tile(tile, p.tiles_m, p.tiles_n, p.group_m, tm, tn);
        m0 = tm * T::BM;
        n0 = tn * T::BN;
        kbeg = kb;
        kend = ke;
        nsteps = (kend - kbeg + T::BK - 1) / T::BK;
        ndirect = direct_ok ? (kend - kbeg) / T::BK : 0;
        a_lim = VEC ? OA::clamp_limit(min(T::BM, p.m - m0)) : min(T::BM, p.m - m0) - 1;
        b_lim = VEC ? OB::clamp_limit(min(T::BN, p.n - n0)) : min(T::BN, p.n - n0) - 1;
        // (the k offset is folded in here so that a step's base below is the
        // same expression in every mode)
        Ablk = OA::tile_base(OA::block_base(p.A, p.lda, m0), p.lda, kbeg);
        Bblk = OB::tile_base(OB::block_base(p.B, p.ldb, n0), p.ldb, kbeg);
    };

    // ---- direct global -> LDS loads (complete, aligned tiles) ---------------
    // buffer_load_dwordx4 ... lds through a per-step buffer resource whose
    // base is the step's first element; each lane supplies a byte offset.
    // (The MUBUF form rather than global_load_lds: the compiler treats a FLAT
    // access that may touch LDS as unordered and would then wait for every
    // outstanding LDS read before each MFMA group.)
    auto load_direct = [&](int step, auto buf) {
        float *as = a_buf(buf), *bs = b_buf(buf);
        const float *abase = OA::tile_base(Ablk, p.lda, step * T::BK);
        const float *bbase = OB::tile_base(Bblk, p.ldb, step * T::BK);
        if constexpr (VEC) {
#pragma unroll
            for (int i = 0; i < OA::PER; ++i) {
                int row, c;
                OA::chunk(tid, i, row, c);
                load_lds16(abase, as + (i * T::WAVES + wave) * 256, OA::direct_offset(row, c, p.lda, a_lim));
            }
#pragma unroll
            for (int i = 0; i < OB::PER; ++i) {
                int row, c;
                OB::chunk(tid, i, row, c);
                load_lds16(bbase, bs + (i * T::WAVES + wave) * 256, OB::direct_offset(row, c, p.ldb, b_lim));
            }
        } else {
            // 64-word window `win` of the tile is filled by one wave's load
#pragma unroll
            for (int i = 0; i < OA::PER4; ++i) {
                const int win = i * T::WAVES + wave;
                load_lds4(abase, as + win * 64, OA::word_offset(win * 64 + lane, p.lda, a_lim));
            }
#pragma unroll
            for (int i = 0; i < OB::PER4; ++i) {
                const int win = i * T::WAVES + wave;
                load_lds4(bbase, bs + win * 64, OB::word_offset(win * 64 + lane, p.ldb, b_lim));
            }
        }
    };

    // The partial last k step, directly as well: four bytes per lane (a
    // 16-byte chunk may straddle the end of k), the words whose k lies past
    // the end given an offset out of the buffer's range, so that they land in
    // LDS as zeros (both operands: a NaN in a pad must not meet a zero).  The
    // words go where the swizzled layout puts them, as in the 4-byte loads of
    // unaligned operands; m / n edges are clamped the same way.
    auto load_direct_masked = [&](int step, auto buf) {
        float *as = a_buf(buf), *bs = b_buf(buf);
        const float *abase = OA::tile_base(Ablk, p.lda, step * T::BK);
        const float *bbase = OB::tile_base(Bblk, p.ldb, step * T::BK);
        const int kv = kend - kbeg - step * T::BK;  // k values left in this step
        const int a_last = min(T::BM, p.m - m0) - 1, b_last = min(T::BN, p.n - n0) - 1;
        // (computed here, once per tile: kept from being hoisted to the
        // kernel's start, where the offsets would hold registers throughout)
        int ln = lane;
        asm volatile("" : "+v"(ln));
#pragma unroll
        for (int i = 0; i < OA::PER4; ++i) {
            const int win = i * T::WAVES + wave, w = win * 64 + ln;
            load_lds4(abase, as + win * 64,
                      OA::word_k(w) < kv ? OA::word_offset(w, p.lda, a_last) : kOutOfRange);
        }
#pragma unroll
        for (int i = 0; i < OB::PER4; ++i) {
            const int win = i * T::WAVES + wave, w = win * 64 + ln;
            load_lds4(bbase, bs + win * 64,
                      OB::word_k(w) < kv ? OB::word_offset(w, p.ldb, b_last) : kOutOfRange);
        }
    };

    // ---- masked loads through VGPRs (edges, k tail, unaligned) -------------
    struct Stage {
        f32x4 a[OA::PER], b[OB::PER];
    };
    auto load_regs = [&](Stage &st, int step) {
        const int k0 = kbeg + step * T::BK;
#pragma unroll
        for (int i = 0; i < OA::PER; ++i) {
            int row, c;
            OA::chunk(tid, i, row, c);
            st.a[i] = OA::template load_masked<VEC>(p.A, p.lda, m0, p.m, k0, kend, row, c);
        }
#pragma unroll
        for (int i = 0; i < OB::PER; ++i) {
            int row, c;
            OB::chunk(tid, i, row, c);
            st.b[i] = OB::template load_masked<VEC>(p.B, p.ldb, n0, p.n, k0, kend, row, c);
        }
    };
    auto store_regs = [&](const Stage &st, auto buf) {
        float *as = a_buf(buf), *bs = b_buf(buf);
#pragma unroll
        for (int i = 0; i < OA::PER; ++i)
            *reinterpret_cast<f32x4 *>(as + 4 * (tid + i * T::NT)) = st.a[i];
#pragma unroll
        for (int i = 0; i < OB::PER; ++i)
            *reinterpret_cast<f32x4 *>(bs + 4 * (tid + i * T::NT)) = st.b[i];
    };

    // ---- accumulators and fragments ----------------------------------------
    f32x16 acc[T::FM][T::FN];
    auto clear_acc = [&]() {
#pragma unroll
        for (int a = 0; a < T::FM; ++a)
#pragma unroll
            for (int b = 0; b < T::FN; ++b)
#pragma unroll
                for (int r = 0; r < 16; ++r) acc[a][b][r] = 0.f;
    };

    int li = lane & 31, lh = lane >> 5;

    struct Frag {
        typename OA::Frag a[T::FM];
        typename OB::Frag b[T::FN];
    };
    // Word offsets of every group's fragment reads.  Set at the start of each
    // run of k steps: (for an operand whose reads are swizzled per group)
    // they then live only through the loop, which keeps a persistent
    // workgroup's compiler from rebuilding them inside the loop to free
    // registers for the epilogue.
    int a_addr[T::FM][T::GROUPS], b_addr[T::FN][T::GROUPS];
    auto set_frag_addr = [&]() {
        int a_off[T::FM], a_sw[T::FM], b_off[T::FN], b_sw[T::FN];
#pragma unroll
        for (int a = 0; a < T::FM; ++a) OA::frag_setup(wm * T::WTM + 32 * a, li, lh, a_off[a], a_sw[a]);
#pragma unroll
        for (int b = 0; b < T::FN; ++b) OB::frag_setup(wn * T::WTN + 32 * b, li, lh, b_off[b], b_sw[b]);
#pragma unroll
        for (int g = 0; g < T::GROUPS; ++g) {
#pragma unroll
            for (int a = 0; a < T::FM; ++a) {
                a_addr[a][g] = OA::frag_addr(a_off[a], a_sw[a], g, lh);
                if constexpr (MODE == kStreamK && !OA::K_ROWS) asm volatile("" : "+v"(a_addr[a][g]));
            }
#pragma unroll
            for (int b = 0; b < T::FN; ++b) {
                b_addr[b][g] = OB::frag_addr(b_off[b], b_sw[b], g, lh);
                if constexpr (MODE == kStreamK && !OB::K_ROWS) asm volatile("" : "+v"(b_addr[b][g]));
            }
        }
    };
    auto read_frag = [&](Frag &f, auto buf, int g) {
        const float *as = a_buf(buf), *bs = b_buf(buf);
#pragma unroll
        for (int a = 0; a < T::FM; ++a) OA::frag_read(f.a[a], as, a_addr[a][g]);
#pragma unroll
        for (int b = 0; b < T::FN; ++b) OB::frag_read(f.b[b], bs, b_addr[b][g]);
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
    auto run_steps = [&]() {
    if (nsteps > 0) {
        set_frag_addr();
        Frag f[2];
        // Stream-K runs a four-buffer tile as a three-buffer ring: its
        // segments restart the pipeline mid-kernel, and the deeper ring
        // measured slower there.
        constexpr int NS = MODE == kStreamK && T::STAGES > 3 ? 3 : T::STAGES, D = NS - 1;
        // direct loads one wave issues per step (a whole step; the partial one)
        constexpr int DIRECT_LOADS = VEC ? OA::PER + OB::PER : OA::PER4 + OB::PER4;
        constexpr int MASKED_LOADS = OA::PER4 + OB::PER4;
        // the partial last k step goes straight to LDS too (four buffers)
        const bool direct_on = partial_step_direct(NS, direct_ok);
        // load the tile of one of the first D steps
        auto fill = [&](int step, auto buf) {
            const int load = load_of(step, nsteps, ndirect);
            if (load == kLoadDirect) {
                load_direct(step, buf);
            } else if (loads_directly(load, direct_on)) {
                load_direct_masked(step, buf);
            } else {
                Stage st;
                load_regs(st, step);
                store_regs(st, buf);
            }
        };
        fill(0, S0{});
        if (D >= 2 && nsteps > 1) fill(1, S1{});
        if (D >= 3 && nsteps > 2) fill(2, std::integral_constant<int, 2>{});
        // Four buffers: the first two tiles must be resident (step 0 reads
        // step 1's first fragments before its barrier); the third may still
        // be on its way, if it was loaded directly.
        if (D >= 3 && 2 < ndirect)
            barrier_keep_newest<DIRECT_LOADS>();
        else
            __syncthreads();
        // Group of a step before which its direct loads are issued: with four
        // buffers a load has nearly two steps to land, and issued behind the
        // first MFMA group it no longer delays that group after the barrier.
        constexpr int LOAD_GROUP = NS == 4 ? 1 : 0;
        static_assert(LOAD_GROUP < T::GROUPS, "the loads must be issued in the step");
        read_frag(f[0], S0{}, 0);

        // One step with its ring position CUR = step % NS fixed at compile
        // time.  DIRECT: the tile D steps ahead is loaded directly (the steady
        // state -- no VGPR loads in that loop, so the compiler's wait counts
        // never hold back the MFMAs); otherwise the step decides: directly
        // while whole k steps remain, else through VGPRs (the partial last k
        // step, or no direct loads at all), or nothing past the end.
        // LOAD: what the step loads for step + D -- kLoadDirect, kLoadRegs
        // (the partial last k step), kLoadNone (past the end), or kLoadAuto
        // (decided at run time).
        auto one_step = [&](int step, auto load_tag, auto cur) {
            constexpr int LOAD = decltype(load_tag)::value;
            constexpr int CUR = decltype(cur)::value;
            using NXT = std::integral_constant<int, (CUR + 1) % NS>;  // (step + 1) % NS
            using WRT = std::integral_constant<int, (CUR + D) % NS>;  // (step + D) % NS
            const int load = LOAD == kLoadAuto ? load_of(step + D, nsteps, ndirect) : LOAD;
            const bool ahead = load != kLoadNone;
            const bool direct = load == kLoadDirect;
            const bool masked = load == kLoadRegs && direct_on;  // partial step, directly
            const bool staged = ahead && !direct && !masked;
            auto issue = [&]() {
                if (direct)
                    load_direct(step + D, WRT{});
                else if (masked)
                    load_direct_masked(step + D, WRT{});
            };
            Stage st;
            if (staged) load_regs(st, step + D);
            if (LOAD_GROUP == 0) issue();
            // The fences keep the scheduler from sinking the loads and the
            // next group's LDS reads below the MFMAs that hide them.
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int g = 0; g < T::GROUPS; ++g) {
                if (g > 0 && g == LOAD_GROUP && (direct || masked)) {
                    issue();
                    __builtin_amdgcn_sched_barrier(0);
                }
                // (the last step reads the next buffer too: stale, unused, and
                // without a branch in front of the last MFMA group)
                if (g + 1 < T::GROUPS) {
                    read_frag(f[(g + 1) & 1], cur, g + 1);
                } else if (D >= 2) {
                    read_frag(f[0], NXT{}, 0);  // GROUPS is even: step+1 starts on set 0
                }
                __builtin_amdgcn_sched_barrier(0);
                mfma_group(f[g & 1]);
                __builtin_amdgcn_sched_barrier(0);
            }
            if (staged) store_regs(st, WRT{});
            // Four buffers: the loads just issued (for step + 3) keep running
            // across the barrier; the ones issued a step earlier (step + 2)
            // must be complete, in every wave, before it.
            if (keeps_load_in_flight(NS, load, direct_on) && direct)
                barrier_keep_newest<DIRECT_LOADS>();
            else if (keeps_load_in_flight(NS, load, direct_on))
                barrier_keep_newest<MASKED_LOADS>();
            else
                __syncthreads();
            // two buffers: step + 1's tile is complete only after the barrier
            if (D == 1) read_frag(f[0], NXT{}, 0);
        };
        using S2 = std::integral_constant<int, 2>;
        using S3 = std::integral_constant<int, 3>;
        using LD = std::integral_constant<int, kLoadDirect>;
        using LA = std::integral_constant<int, kLoadAuto>;
        // The phases of the run and its tail sequence (kloop.hpp).
        const KLoop kl = kloop_schedule(nsteps, ndirect, NS);
        int step = 0;
        // Steady state: NS steps per iteration, so each ring position is a
        // compile-time constant and the accumulators keep their registers
        // (a runtime switch per step makes the compiler copy them around).
        for (; step < kl.steady_end; step += NS) {
            one_step(step, LD{}, S0{});
            one_step(step + 1, LD{}, S1{});
            if constexpr (NS > 2) one_step(step + 2, LD{}, S2{});
            if constexpr (NS > 3) one_step(step + 3, LD{}, S3{});
        }
        // Without direct loads (huge leading dimensions) whole rounds of the
        // ring go through the deciding step too, so step % NS stays 0.
        for (; step < kl.auto_end; step += NS) {
            one_step(step, LA{}, S0{});
            one_step(step + 1, LA{}, S1{});
            if constexpr (NS > 2) one_step(step + 2, LA{}, S2{});
            if constexpr (NS > 3) one_step(step + 3, LA{}, S3{});
        }
        // The last R <= kTailMax steps (step % NS == 0 here), ND of them whole k
        // steps, as one of a few sequences fixed at compile time: step i
        // loads step i + D directly, through VGPRs (the partial step) or not
        // at all.  Decided in each step at run time, they ran about a
        // quarter of a step slower each.
        auto tail = [&](auto seq_tag) {
            constexpr TailSeq SEQ = kTailSequences[decltype(seq_tag)::value];
            auto at = [&](auto i_tag) {
                constexpr int I = decltype(i_tag)::value;
                if constexpr (I < SEQ.r) {
                    one_step(step + I,
                             std::integral_constant<int, load_of(I + D, SEQ.r, SEQ.nd)>{},
                             std::integral_constant<int, I % NS>{});
                }
            };
            at(std::integral_constant<int, 0>{});
            at(std::integral_constant<int, 1>{});
            at(std::integral_constant<int, 2>{});
            at(std::integral_constant<int, 3>{});
            at(std::integral_constant<int, 4>{});
        };
        static_assert(kTailMax == 5, "the tail steps cover five steps");
        auto tail_auto = [&]() {
            using Q2 = std::integral_constant<int, 2 % NS>;
            using Q3 = std::integral_constant<int, 3 % NS>;
            using Q4 = std::integral_constant<int, 4 % NS>;
            if (step < nsteps) one_step(step, LA{}, S0{});
            if (step + 1 < nsteps) one_step(step + 1, LA{}, S1{});
            if (step + 2 < nsteps) one_step(step + 2, LA{}, Q2{});
            if (step + 3 < nsteps) one_step(step + 3, LA{}, Q3{});
            if (step + 4 < nsteps) one_step(step + 4, LA{}, Q4{});
        };
        // The sequence kl.tail, each one compiled in its own branch.
        auto dispatch = [&](auto self, auto idx_tag) {
            constexpr int IDX = decltype(idx_tag)::value;
            if constexpr (IDX < kNumTailSequences) {
                if (kl.tail == IDX)
                    tail(idx_tag);
                else
                    self(self, std::integral_constant<int, IDX + 1>{});
            } else {
                tail_auto();
            }
        };
        // Two-buffer rings (long k steps per tile, registers to the limit)
        // keep the run-time tail (kloop_schedule never picks a sequence
        // for them).
        if constexpr (NS == 2) {
            tail_auto();
        } else {
            dispatch(dispatch, std::integral_constant<int, 0>{});
        }
    }
    };

    // ---- epilogue -----------------------------------------------------------
    // Accumulator register r of lane (j, h) holds C row 8*(r/4) + 4*h + r%4,
    // column j of its 32x32 block.  `store(row, col, v)` gets every in-range
    // element of the tile.
    auto for_each_output = [&](auto store) {
#pragma unroll
        for (int a = 0; a < T::FM; ++a) {
#pragma unroll
            for (int b = 0; b < T::FN; ++b) {
                const int col = n0 + wn * T::WTN + 32 * b + li;
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                    const int row = m0 + wm * T::WTM + 32 * a + 8 * (r >> 2) + 4 * lh + (r & 3);
                    if (row < p.m && col < p.n) store(row, col, acc[a][b][r]);
                }
            }
        }
    };
    // Tiles that lie inside the output (most of them) can take a lean path:
    // `corner` is the tile's first element, each lane adds one 32-bit byte
    // offset and each accumulator register a row offset the whole wave shares,
    // with no bounds checks, 64-bit index products or branches per element
    // (the checked path costs about 15 instructions per element).  Byte
    // offsets stay below 2^32 when BM * ld < 2^30.
    auto lean_ok = [&](int ld) {
        return m0 + T::BM <= p.m && n0 + T::BN <= p.n && (long long)T::BM * ld < (1ll << 30);
    };
    // `block(addr, v)` gets each 32 x 32 block's registers v and addr(r), the
    // address of register r's element.
    auto for_each_lean = [&](float *corner, int ld, auto block) {
        const unsigned lane_off = (unsigned)((wm * T::WTM + 4 * lh) * ld + wn * T::WTN + li);
#pragma unroll
        for (int a = 0; a < T::FM; ++a) {
#pragma unroll
            for (int b = 0; b < T::FN; ++b) {
                auto addr = [&](int r) {
                    const unsigned e =
                        lane_off + (unsigned)((32 * a + 8 * (r >> 2) + (r & 3)) * ld + 32 * b);
                    return reinterpret_cast<float *>(reinterpret_cast<char *>(corner) + 4u * e);
                };
                block(addr, acc[a][b]);
            }
        }
    };
    auto store_lean = [&](float *corner, int ld) {
        for_each_lean(corner, ld, [&](auto addr, const f32x16 &v) {
#pragma unroll
            for (int r = 0; r < 16; ++r) *addr(r) = v[r];
        });
    };
    // C = alpha * acc + beta * C.  C is touched once: nontemporal access
    // (measured about 1 % faster at 2048^3 and 8192^3, probably less dirty L2
    // to write back when the kernel ends).  The lean path is for tiles of
    // which a CU holds several workgroups, whose epilogues overlap the
    // others' matrix work (ragged-tail shape +2 %, 8192^3 with beta +1 %);
    // with one 16-wave workgroup per CU the checked path measured 0.4 %
    // faster at 2048^3 (four pairs of runs back to back).
    auto store_c = [&]() {
        if (!T::ONE_PER_CU && lean_ok(p.ldc)) {
            float *corner = p.C + (long long)m0 * p.ldc + n0;
            if (p.beta == 0.f) {
                for_each_lean(corner, p.ldc, [&](auto addr, const f32x16 &v) {
#pragma unroll
                    for (int r = 0; r < 16; ++r) __builtin_nontemporal_store(p.alpha * v[r], addr(r));
                });
            } else {
                // a block's 16 loads in flight together, then its stores
                for_each_lean(corner, p.ldc, [&](auto addr, const f32x16 &v) {
                    float c[16];
#pragma unroll
                    for (int r = 0; r < 16; ++r) c[r] = __builtin_nontemporal_load(addr(r));
#pragma unroll
                    for (int r = 0; r < 16; ++r)
                        __builtin_nontemporal_store(__builtin_fmaf(p.beta, c[r], p.alpha * v[r]),
                                                    addr(r));
                });
            }
            return;
        }
        for_each_output([&](int row, int col, float v) {
            float *dst = p.C + (long long)row * p.ldc + col;
            float r = p.alpha * v;
            if (p.beta != 0.f) r = __builtin_fmaf(p.beta, __builtin_nontemporal_load(dst), r);
            __builtin_nontemporal_store(r, dst);
        });
    };

    if constexpr (MODE == kStreamK) {
        // Data-parallel tiles, then stream-K.  The first sk_dp_tiles
        // workgroups each compute one whole tile, in the order of the
        // one-tile-per-workgroup launch (the hardware hands them to CUs as
        // CUs free up, which balances the load); the remaining `grid` share
        // the (tile, k step) iterations of the tiles after those evenly, one
        // segment per tile a workgroup's range touches.  A segment that
        // covers its tile's whole k range is finished here; the others leave
        // their raw sums in the workgroup's slot 0 (a segment that starts
        // inside its tile) or slot 1 (one that starts at the tile's first step
        // and stops inside it), for the fixup kernel.  A workgroup has at most
        // one segment of each kind.
        const int h = blockIdx.x;
        const int dp = p.sk_dp_tiles;
        long long w = -1, it, end, tile0 = 0;
        if (h < dp) {
            it = (long long)xcd_contiguous(h, dp) * p.sk_ksteps;
            end = it + p.sk_ksteps;
        } else {
            const long long grid = gridDim.x - dp;
            w = xcd_contiguous(h - dp, (int)grid);
            it = sk_begin(w, p.sk_iters, grid);
            end = sk_begin(w + 1, p.sk_iters, grid);
            tile0 = dp;
        }
        while (it < end) {
            // Per-lane indices pass through an empty asm statement at the top
            // of each segment, so that addresses derived from them are
            // computed per segment instead of being hoisted out of the loop
            // and held in registers across every k step (which made this
            // instance spill).
            asm volatile("" : "+v"(tid), "+v"(lane), "+v"(li), "+v"(lh));
            const long long t = it / p.sk_ksteps;
            const int ks = (int)(it - t * p.sk_ksteps);
            const int ke = (int)min((long long)p.sk_ksteps, ks + (end - it));
            set_tile((int)(tile0 + t), ks * T::BK, min(p.k, ke * T::BK));
            clear_acc();
            run_steps();
            if (ks == 0 && ke == p.sk_ksteps) {
                store_c();
            } else {
                // (the whole slot is written; entries outside C are never
                // stored by the fixup)
                float *slot = p.ws + (w * 2 + (ks > 0 ? 0 : 1)) * (long long)(T::BM * T::BN);
                store_lean(slot, T::BN);
            }
            it += ke - ks;
        }
    } else {
        int id = p.xcd_remap ? xcd_contiguous(blockIdx.x, gridDim.x) : (int)blockIdx.x;
        int slice = 0;
        if (SPLIT) {
            const int tiles = p.tiles_m * p.tiles_n;
            slice = id / tiles;
            id -= slice * tiles;
        }
        const int kb = SPLIT ? slice * p.k_per_split : 0;
        set_tile(id, kb, SPLIT ? min(p.k, kb + p.k_per_split) : p.k);
        clear_acc();
        run_steps();
        if constexpr (MODE == kPartial) {
            // Ordinary stores (unlike C): the combine that reads the partials
            // next finds them in cache.  At 512 x 512 x 262144 (16 slices) the
            // combine took 4.82 us after ordinary stores against 5.24 us after
            // nontemporal ones, with the partial kernel unchanged (932 us).
            if (lean_ok(p.n)) {
                float *corner = p.ws + (long long)slice * p.ws_slice + (long long)m0 * p.n + n0;
                store_lean(corner, p.n);
            } else {
                for_each_output([&](int row, int col, float v) {
                    p.ws[(long long)slice * p.ws_slice + (long long)row * p.n + col] = v;
                });
            }
        } else if constexpr (MODE == kAtomic) {
            for_each_output([&](int row, int col, float v) {
                unsafeAtomicAdd(p.C + (long long)row * p.ldc + col, p.alpha * v);
            });
        } else {
            store_c();
        }
    }
}

}  // namespace mi
