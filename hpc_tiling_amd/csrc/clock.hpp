// clock.hpp -- the shader clock, measured on the GPU (gfx950).
//
// Page "gemm优化" (blog.lightlisten.com), section 关于GPU频率影响, shows a
// GEMM's ranking against the vendor library flip with the core clock, so every
// timing is reported with the clock it ran at.  Each workgroup of this kernel
// reads the 64-bit shader-cycle counter (s_memtime, counting at the core
// clock of its CU) and the constant-rate reference counter (s_memrealtime)
// together, waits until the reference counter has advanced by `spin` ticks,
// and reads both again: the ratio of the two advances times the reference rate
// is the average core clock over the wait.  Workgroups are placed on the XCDs
// round-robin, so a launch of 8 measures each XCD once.
#pragma once

#include <hip/hip_runtime.h>

namespace mi {

constexpr int kClockProbeMaxWorkgroups = 1024;
constexpr long long kClockProbeMaxIters = 1 << 22;  // bounds the wait (~0.2 s)

// ticks[4 w + 0..3] = shader cycles and reference ticks at the start, then
// at the end, of workgroup w's wait.
__global__ __launch_bounds__(64) void clock_probe_kernel(unsigned long long *ticks,
                                                         long long spin) {
    const unsigned long long r0 = __builtin_amdgcn_s_memrealtime();
    const unsigned long long c0 = __builtin_amdgcn_s_memtime();
    unsigned long long r1 = r0;
    for (long long i = 0; i < kClockProbeMaxIters && (long long)(r1 - r0) < spin; ++i) {
        __builtin_amdgcn_s_sleep(1);
        r1 = __builtin_amdgcn_s_memrealtime();
    }
    const unsigned long long c1 = __builtin_amdgcn_s_memtime();
    // lanes 0..3 store one value each (a per-lane vector store)
    const int lane = threadIdx.x;
    if (lane < 4) {
        const unsigned long long v = lane == 0 ? c0 : lane == 1 ? r0 : lane == 2 ? c1 : r1;
        ticks[4 * (long long)blockIdx.x + lane] = v;
    }
}

}  // namespace mi
