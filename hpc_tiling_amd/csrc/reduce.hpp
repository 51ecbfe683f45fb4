// reduce.hpp -- sum of a float array (page aerisun.top, section
// "Reduce 的分层归约"): every lane first accumulates many inputs in registers
// (section "先在线程内累加，再交换部分和"; here a contiguous run of the input per
// workgroup, its lanes striding through it), then the wave
// adds its lanes with register exchanges instead of LDS (section
// "Warp shuffle 的数据交换", on wave64 with DPP rotations and row swaps), the
// four waves of a workgroup meet in LDS, and a second single-workgroup kernel
// adds the per-workgroup partials -- two passes and no atomics, so the
// result is the same bits on every run.
#pragma once

#include "common.hpp"

namespace mi {

constexpr int kReduceThreads = 256;

// Workgroup partial sums.  The input is seen as n / 4 groups of four
// consecutive floats (plus n % 4 trailing floats, added by the first lanes of
// workgroup 0); workgroup b takes the contiguous run of `per` groups from
// b * per, and its lanes walk that run 256 groups apart, four deep for loads
// in flight, each keeping four accumulators (one per position in a group).
// VEC: x is 16-byte aligned and a group is one 16-byte load; otherwise the
// same groups are read as four 4-byte loads, so both paths add the same
// values in the same order.  The input is read once, so the loads are
// nontemporal.  On MI355X a contiguous run per workgroup sums 1 GiB at
// 7.0 TB/s, against 6.2 for runs interleaved across the grid (DRAM pages
// stay open longer).
template <bool VEC>
__device__ __forceinline__ f32x4 load_group(const float *x, long long j) {
    if constexpr (VEC) {
        return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(x) + j);
    } else {
        const float *q = x + 4 * j;
        return f32x4{__builtin_nontemporal_load(q), __builtin_nontemporal_load(q + 1),
                     __builtin_nontemporal_load(q + 2), __builtin_nontemporal_load(q + 3)};
    }
}

template <bool VEC>
__global__ __launch_bounds__(kReduceThreads) void reduce_partial_kernel(const float *__restrict__ x,
                                                                      long long n, long long per,
                                                                      float *__restrict__ partials) {
    const long long groups = n >> 2;
    const long long beg = (long long)blockIdx.x * per;
    const long long end = min(beg + per, groups);
    constexpr int NT = kReduceThreads;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    long long j = beg + threadIdx.x;
    for (; j + 3 * NT < end; j += 4 * NT) {
        const f32x4 a = load_group<VEC>(x, j);
        const f32x4 b = load_group<VEC>(x, j + NT);
        const f32x4 c = load_group<VEC>(x, j + 2 * NT);
        const f32x4 d = load_group<VEC>(x, j + 3 * NT);
        acc += a;
        acc += b;
        acc += c;
        acc += d;
    }
    for (; j < end; j += NT) acc += load_group<VEC>(x, j);
    if (blockIdx.x == 0) {
        const long long rest = n - 4 * groups;  // 0..3 trailing floats
        if (threadIdx.x < rest) acc[0] += x[4 * groups + threadIdx.x];
    }
    float s = wave_sum((acc[0] + acc[1]) + (acc[2] + acc[3]));
    __shared__ float wave_part[kReduceThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x == 0) partials[blockIdx.x] = (wave_part[0] + wave_part[1]) + (wave_part[2] + wave_part[3]);
}

// out[0] = sum of the `count` partials (0 <= count <= kFinalThreads *
// kFinalPer), one workgroup of kFinalThreads.  Lane t loads partials t,
// t + kFinalThreads, ... all at once (independent loads, one memory round
// trip) and adds them in that order; the waves then add their lanes, and
// wave 0 adds the per-wave sums.  The order is fixed, so the result is too.
constexpr int kFinalThreads = 1024;
constexpr int kFinalPer = 8;

__global__ __launch_bounds__(kFinalThreads) void reduce_final_kernel(const float *__restrict__ partials,
                                                                   int count, float *out) {
    float v[kFinalPer];
#pragma unroll
    for (int j = 0; j < kFinalPer; ++j) {
        const int i = threadIdx.x + j * kFinalThreads;
        v[j] = i < count ? partials[i] : 0.f;
    }
    float s = v[0];
#pragma unroll
    for (int j = 1; j < kFinalPer; ++j) s += v[j];
    s = wave_sum(s);
    __shared__ float wave_part[kFinalThreads / 64];
    if ((threadIdx.x & 63) == 0) wave_part[threadIdx.x >> 6] = s;
    __syncthreads();
    if (threadIdx.x < 64) {
        float w = threadIdx.x < kFinalThreads / 64 ? wave_part[threadIdx.x] : 0.f;
        w = wave_sum(w);
        if (threadIdx.x == 0) out[0] = w;
    }
}

}  // namespace mi
