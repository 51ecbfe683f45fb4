// common.hpp -- argument block and workgroup-order helpers shared by the
// SGEMM kernels (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace mi {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// Epilogue modes of the matrix-core kernel (see sgemm_mfma.hpp).
constexpr int kFull = 0, kPartial = 1, kAtomic = 2, kStreamK = 3;

// MI355X places workgroups on its 8 XCDs (each with a private L2) round-robin
// by workgroup id.
constexpr int kXcds = 8;

// LDS is handed to workgroups in granules of 1280 bytes, 128 per CU (its
// 160 KiB).  Probed on MI355X with workgroups of a given LDS size, the
// workgroups that ran on one CU at once were floor(128 / granules) for every
// size tried from 24 to 54 KiB: five of 32000 bytes (25 granules) but four of
// 32256 or 32768 (26), four of 40960 (32), three of 53248 (42), two of 54272
// (43).
constexpr int kLdsGranuleBytes = 1280;
constexpr int kLdsGranulesPerCu = 128;
constexpr int lds_granules(long long bytes) {
    return (int)((bytes + kLdsGranuleBytes - 1) / kLdsGranuleBytes);
}

// Everything a GEMM kernel needs; passed by value as the single kernel
// argument.  Leading dimensions and slice strides are 64-bit so that row
// offsets never overflow.
struct GemmArgs {
    int m, n, k;
    float alpha, beta;
    const float *A;
    long long lda;
    const float *B;
    long long ldb;
    float *C;
    long long ldc;
    int tiles_m, tiles_n;  // C tiles along m and n
    int group_m;           // height (in tiles) of one group of the grouped order
    int k_per_split;       // split-K: length of a k slice (multiple of the k step)
    float *ws;             // split-K: partials, slice s at ws + s * ws_slice
    long long ws_slice;    // split-K: floats per slice (>= m * n, multiple of 64)
    int c_vec;             // 1 when C is 16-byte aligned and ldc % 4 == 0
    long long sk_iters;    // stream-K: (shared tiles) * k steps per tile
    int sk_ksteps;         // stream-K: k steps per tile
    int sk_dp_tiles;       // stream-K: leading tiles computed whole, one per workgroup
    int xcd_remap;         // 1: logical ids contiguous per XCD (xcd_contiguous); 0: the
                           // hardware order (measured comparisons only)
};

// Stream-K partition of `iters` (tile, k step) iterations over `grid`
// workgroups: workgroup w takes [sk_begin(w), sk_begin(w + 1)), and the
// iteration x belongs to workgroup sk_owner(x) (the last w whose range starts
// at or before x).
__host__ __device__ __forceinline__ long long sk_begin(long long w, long long iters, long long grid) {
    return w * iters / grid;
}
__host__ __device__ __forceinline__ long long sk_owner(long long x, long long iters, long long grid) {
    return ((x + 1) * grid + iters - 1) / iters - 1;
}

// Renumbers workgroups so that each XCD owns one contiguous range of logical
// ids: hardware id w runs on XCD w % 8 as that XCD's (w / 8)-th workgroup.
// The map is a bijection of [0, count) for every count.
__device__ __forceinline__ int xcd_contiguous(int w, int count) {
    const int q = count / kXcds, r = count % kXcds;
    const int x = w % kXcds, idx = w / kXcds;
    return x * q + (x < r ? x : r) + idx;
}

// Grouped tile order (page "gemm优化", section on L2 swizzle): consecutive
// logical ids walk down a group of `group_m` tile rows before moving to the
// next tile column, so neighbouring workgroups share both B columns and A
// rows in L2.  A bijection of [0, tiles_m * tiles_n).
__device__ __forceinline__ void grouped_tile(int id, int tiles_m, int tiles_n,
                                             int group_m, int &tm, int &tn) {
    const int per_group = group_m * tiles_n;
    const int g = id / per_group;
    const int first = g * group_m;
    const int rows = min(tiles_m - first, group_m);
    const int local = id - g * per_group;
    tm = first + local % rows;
    tn = local / rows;
}

// Four consecutive floats src[0..3]; elements at index >= valid read as 0
// (never dereferenced).  `vec` allows one 16-byte load when all 4 are valid.
template <bool VEC>
__device__ __forceinline__ f32x4 load4_masked(const float *src, int valid) {
    if (VEC && valid >= 4) return *reinterpret_cast<const f32x4 *>(src);
    f32x4 v = {0.f, 0.f, 0.f, 0.f};
    if (valid > 0) v[0] = src[0];
    if (valid > 1) v[1] = src[1];
    if (valid > 2) v[2] = src[2];
    if (valid > 3) v[3] = src[3];
    return v;
}

// Sum of x over the four lanes {l, l^16, l^32, l^48}, returned in all of them:
// two butterfly steps with gfx950's row-swap instructions.
__device__ __forceinline__ float sum_over_lane_quarters(float x) {
    const unsigned u = __float_as_uint(x);
    const auto h = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    // h[0] holds x of lanes (l < 32 ? l : l - 32), h[1] of (l < 32 ? l + 32 : l).
    const float y = __uint_as_float(h[0]) + __uint_as_float(h[1]);
    const unsigned w = __float_as_uint(y);
    const auto q = __builtin_amdgcn_permlane16_swap(w, w, false, false);
    return __uint_as_float(q[0]) + __uint_as_float(q[1]);
}

// x rotated right by N lanes within each row of 16 (DPP row_ror:N).
template <int N>
__device__ __forceinline__ float row_ror(float x) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x120 + N, 0xf, 0xf, false));
}

// Sum of x over the whole wave, returned in every lane.  Rotating a row of
// 16 by 8, 4, 2, 1 and adding leaves the row sum in all its lanes (after the
// first step the values are symmetric under lane ^ 8, so a rotation by 4
// pairs each lane with lane ^ 4, and so on); the row-swap butterflies then
// add the four rows.  6 addition levels; the order is fixed.
__device__ __forceinline__ float wave_sum(float x) {
    x += row_ror<8>(x);
    x += row_ror<4>(x);
    x += row_ror<2>(x);
    x += row_ror<1>(x);
    return sum_over_lane_quarters(x);
}

}  // namespace mi
