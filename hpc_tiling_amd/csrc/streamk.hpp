// streamk.hpp -- the fixup kernel of the stream-K schedule (gfx950).
#pragma once

#include <hip/hip_runtime.h>

#include "common.hpp"

namespace mi {

// Stream-K fixup over the shared tiles tile0, tile0 + 1, ... (`iters` is
// their count times `ksteps`).  Blocks come in groups of kFixupSplit, one per
// band of rows of a tile.  Group b - 1 (b = 1 .. grid - 1) looks at the
// iteration where workgroup b's range starts; if that is inside a tile, and b
// is the first workgroup starting inside it, the tile was shared: its parts
// sit in the slots of workgroups first .. last (the owners of the tile's first
// and last iterations), and the group adds them in that order -- which is
// also k order, so the result is fixed -- then writes C = alpha * sum +
// beta * C.  At most kFixupMaxParts workgroups may share one tile (the host
// keeps the grid below that).
constexpr int kFixupMaxParts = 2048;
constexpr int kFixupSplit = 4;
constexpr int kFixupThreads = 256;

template <int BM, int BN>
__global__ __launch_bounds__(kFixupThreads) void streamk_fixup_kernel(
    const float *__restrict__ ws, long long iters, int ksteps, int grid, int tile0, int tiles_m,
    int tiles_n, int group_m, int m, int n, float alpha, float beta, float *C, long long ldc) {
    const long long b = (long long)(blockIdx.x / kFixupSplit) + 1;
    const int band = blockIdx.x % kFixupSplit;
    // The index arithmetic sits in front of every block's first load: while
    // every numerator below (at most iters * (grid + 1)) fits in 32 bits, the
    // divisions are done in 32-bit unsigned arithmetic (same quotients, a
    // fraction of the instructions of a 64-bit division).
    const bool narrow = iters * (grid + 1) < (1ll << 32);
    auto div = [narrow](long long a, long long d) -> long long {
        return narrow ? (long long)((unsigned)a / (unsigned)d) : a / d;
    };
    auto begin = [&](long long w) { return div(w * iters, grid); };
    auto owner = [&](long long x) { return div((x + 1) * grid + iters - 1, iters) - 1; };
    const long long x = begin(b);
    if (x >= iters) return;
    const long long t = div(x, ksteps);
    if (x == t * ksteps) return;
    const long long first = owner(t * ksteps);
    if (first + 1 != b) return;
    const long long last = owner(t * ksteps + ksteps - 1);
    const int parts = (int)(last - first + 1);

    // slot offset of every part (-1: a workgroup with an empty range)
    __shared__ long long part_off[kFixupMaxParts];
    for (int q = threadIdx.x; q < parts; q += kFixupThreads) {
        const long long w = first + q;
        const long long wb = begin(w);
        part_off[q] = begin(w + 1) == wb
                          ? -1
                          : (w * 2 + (wb > t * ksteps ? 0 : 1)) * (long long)(BM * BN);
    }
    __syncthreads();

    // Lane l of band j holds float4 groups j * BAND + l, j * BAND + l + 256,
    // ... of the tile (row-major, BN a multiple of 4).  The parts are added in
    // order, the loads of PG parts in flight together (a tile is usually
    // shared by two or three workgroups: one round trip to memory).  Entries
    // of the slots outside C's extent are added like the others but never
    // stored.
    constexpr int BAND = BM * BN / 4 / kFixupSplit;
    constexpr int PER = BAND / kFixupThreads;
    static_assert(PER >= 1 && BAND % kFixupThreads == 0, "a band must fill the block");
    const int g0 = band * BAND + threadIdx.x;
    auto part = [&](long long off, int u) -> f32x4 {
        if (off < 0) return f32x4{0.f, 0.f, 0.f, 0.f};
        return reinterpret_cast<const f32x4 *>(ws + off)[g0 + u * kFixupThreads];
    };
    f32x4 acc[PER];
#pragma unroll
    for (int u = 0; u < PER; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
    // Positions past the last part add +0, which leaves every sum unchanged
    // (a sum that starts at +0 is never -0).
    constexpr int PG = 4;
    for (int q = 0; q < parts; q += PG) {
        f32x4 v[PG][PER];
#pragma unroll
        for (int i = 0; i < PG; ++i) {
            const long long o = q + i < parts ? part_off[q + i] : -1;
#pragma unroll
            for (int u = 0; u < PER; ++u) v[i][u] = part(o, u);
        }
#pragma unroll
        for (int i = 0; i < PG; ++i)
#pragma unroll
            for (int u = 0; u < PER; ++u) acc[u] += v[i][u];
    }
    int tm, tn;
    grouped_tile(tile0 + (int)t, tiles_m, tiles_n, group_m, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    // Columns come in groups of four from a multiple of 4, so with C 16-byte
    // aligned and ldc a multiple of 4 a whole group is one 16-byte access.
    const bool vec = (reinterpret_cast<unsigned long long>(C) & 15) == 0 && ldc % 4 == 0;
#pragma unroll
    for (int u = 0; u < PER; ++u) {
        const int e = 4 * (g0 + u * kFixupThreads);
        const int row = m0 + e / BN, col = n0 + e % BN;
        if (row >= m) continue;
        if (vec && col + 3 < n) {
            f32x4 *dst = reinterpret_cast<f32x4 *>(C + (long long)row * ldc + col);
            f32x4 v = alpha * acc[u];
            if (beta != 0.f) {
                const f32x4 c = *dst;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = __builtin_fmaf(beta, c[j], v[j]);
            }
            *dst = v;
            continue;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            if (col + j >= n) break;
            float *dst = C + (long long)row * ldc + col + j;
            float v = alpha * acc[u][j];
            if (beta != 0.f) v = __builtin_fmaf(beta, *dst, v);
            *dst = v;
        }
    }
}

}  // namespace mi
