// reduce.hpp -- sum of a float array (page aerisun.top, section
// "Reduce 的分层归约"): every lane first accumulates many inputs in registers
// (grid-stride loop, section "先在线程内累加，再交换部分和"), then the wave
// adds its lanes with register exchanges instead of LDS (section
// "Warp shuffle 的数据交换", on wave64 with DPP rotations and row swaps), the
// four waves of a workgroup meet in LDS, and a second single-workgroup kernel
// adds the per-workgroup partials -- two passes and no atomics, so the
// result is the same bits on every run.
#pragma once

#include "common.hpp"

namespace mi {

constexpr int kReduceThreads = 256;

// Workgroup partial sums.  VEC: x is 16-byte aligned (float4 loads; the last
// n % 4 elements are added by the first threads).  Each lane keeps four
// accumulators (one per float4 component) and adds one float4 per stride,
// unrolled four deep for loads in flight.  The input is read once, so the
// loads are marked nontemporal (streamed past the caches); on gfx950 that
// raised the 1 GiB sum from 5.3 to 6.2 TB/s.
template <bool VEC>
__global__ __launch_bounds__(kReduceThreads) void reduce_partial_kernel(const float *__restrict__ x,
                                                                      long long n,
                                                                      float *__restrict__ partials) {
    const long long tid = (long long)blockIdx.x * kReduceThreads + threadIdx.x;
    const long long stride = (long long)gridDim.x * kReduceThreads;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    if (VEC) {
        const f32x4 *xv = reinterpret_cast<const f32x4 *>(x);
        const long long nv = n >> 2;
        long long i = tid;
        for (; i + 3 * stride < nv; i += 4 * stride) {
            const f32x4 a = __builtin_nontemporal_load(xv + i);
            const f32x4 b = __builtin_nontemporal_load(xv + i + stride);
            const f32x4 c = __builtin_nontemporal_load(xv + i + 2 * stride);
            const f32x4 d = __builtin_nontemporal_load(xv + i + 3 * stride);
            acc += a;
            acc += b;
            acc += c;
            acc += d;
        }
        for (; i < nv; i += stride) acc += __builtin_nontemporal_load(xv + i);
        const long long rest = n - 4 * nv;  // 0..3 trailing elements
        if (tid < rest) acc[0] += x[4 * nv + tid];
    } else {
        for (long long i = tid; i < n; i += stride) acc[0] += __builtin_nontemporal_load(x + i);
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
