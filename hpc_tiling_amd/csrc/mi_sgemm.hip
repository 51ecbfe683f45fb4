// mi_sgemm.hip -- C-ABI entry points: argument checks, planning and launch
// of the SGEMM kernels for gfx950.  Declarations and semantics are in
// include/mi_sgemm.h.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <climits>
#include <cstdint>
#include <cstring>
#include <mutex>

#include "mi_sgemm.h"
#include "mfma_configs.hpp"
#include "sgemm_valu.hpp"
#include "reduce.hpp"
#include "splitk.hpp"
#include "clock.hpp"
#include "fma_rate.hpp"

// Scratch of mi_sgemm_splitk_noalloc: the split-K partial sums (or stream-K
// slots) of callers that cannot allocate device memory.  Each device the
// library runs on holds its own copy until the process ends.  Host code never
// uses this name as an address (on the host it is only a stand-in): the
// device address comes from hipGetSymbolAddress, once per device
// (mi::scratch_address).
static __device__ __align__(256) float scratch[MI_SGEMM_NOALLOC_SCRATCH_BYTES / sizeof(float)];

namespace mi {
namespace {

constexpr size_t kScratchBytes = MI_SGEMM_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch is a whole number of 256-byte blocks");

// The device address of `scratch` on the current device, looked up on the
// first call for each device (with that device current) and kept; nullptr
// when the runtime cannot give it.
void *scratch_address() {
    static std::mutex mu;
    static void *addr[128] = {};
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 128) return nullptr;
    std::lock_guard<std::mutex> lock(mu);
    if (!addr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess) return nullptr;
        addr[dev] = p;
    }
    return addr[dev];
}

// ---------------------------------------------------------------------------
// Tile configurations of the matrix-core kernel (mfma_configs.hpp).
// ---------------------------------------------------------------------------
const MfmaConfig *const kMfmaConfigTable[kNumMfmaConfigs] = {
    &kMfmaConfig0, &kMfmaConfig1, &kMfmaConfig2, &kMfmaConfig3, &kMfmaConfig4, &kMfmaConfig5,
    &kMfmaConfig6, &kMfmaConfig7, &kMfmaConfig8, &kMfmaConfig9, &kMfmaConfig10, &kMfmaConfig11,
    &kMfmaConfig12, &kMfmaConfig13, &kMfmaConfig14,
};
const MfmaConfig &mfma_config(int id) { return *kMfmaConfigTable[id]; }

constexpr int kGroupM = 8;  // grouped-order height (the pages use groups of 8)
constexpr int kCUs = 256;   // MI355X compute units

long long ceil_div(long long a, long long b) { return (a + b - 1) / b; }

long long tile_count(int m, int n, int id) {
    return ceil_div(m, mfma_config(id).bm) * ceil_div(n, mfma_config(id).bn);
}

// Tile choice: a small cost model.  The workgroups of a launch are spread
// evenly over the CUs, so the busiest CU runs ceil(tiles / CUs) tiles; its
// time is that count times the tile area over the configuration's efficiency
// when every CU is busy.  The efficiencies are measured on MI355X at 4096^3,
// where every configuration divides the grid evenly (fraction of the FP32
// matrix peak); ties go to the earlier entry.
struct Candidate {
    int id;
    double efficiency;
};
constexpr Candidate kCandidates[] = {
    {9, 0.946},  // 128 x 128 x 32, 16 waves
    {0, 0.941},  // 128 x 128 x 16, 4 waves
    {7, 0.937},  // 256 x 128 x 32, 8 waves
    {8, 0.922},  // 128 x 64 x 32, 4 waves
    {6, 0.906},  // 64 x 64 x 32, 4 waves
};

double tile_cost(int m, int n, int id, double efficiency) {
    const MfmaConfig &c = mfma_config(id);
    const long long per_cu = ceil_div(tile_count(m, n, id), kCUs);
    return (double)per_cu * c.bm * c.bn / efficiency;
}

// Two resident workgroups of an 8-wave 128 x 128 x 16 tile (id 14, 4 x 2
// waves, a four-buffer ring in 64 KB of LDS each) cover each other's barrier
// waits.  Forced against the 16-wave tile and against the earlier two-buffer
// 128 x 128 x 32 tile (id 11), back to back on one MI355X, it won from three
// rounds of 128 x 128 tiles on: 4096^3 148.9 -> 149.7, 8192^3 151.9 ->
// 152.5 (id 11), 8192^2 x 2048 146.4 -> 148.1 (id 11), 3072 x 4096^2 149.0
// -> 149.5.  It was mixed at two rounds and lost at one (2048^3 145.2 ->
// 143.1: half of the two-per-CU slots stay empty).
constexpr int kTwoWorkgroupId = 14;
constexpr long long kTwoWorkgroupMinRounds = 3;

// When k leaves a partial 32-wide step, the 64 x 64 x 16 tile built for six
// workgroups per CU (id 12) beats the 64 x 64 x 32 one on grids of 8 or more
// rounds of 64 x 64 tiles: 3001 x 4997 x 1023 +4 %, 5000^2 x 2047 +4 %,
// 3000^2 x 700 +3 %, 2500 x 6000 x 777 with unaligned rows +15 % (back to
// back on one MI355X).  With a whole number of 32-wide steps, or a short
// grid (1000^3: -3 %), it loses.
constexpr int kSmallStepId = 12;
constexpr long long kSmallStepMinRounds = 8;

// The same tile with a four-buffer ring (id 13; four workgroups of 32 KiB
// fit a CU's LDS; a load has nearly two k steps to land) wins once k is long enough to
// pay for the deeper prologue: over k = 257 .. 4095 at 3000 x 5000,
// 2500 x 6000 and 8000^2 it lost 1-4 % up to k = 777 and won 0.5-2 % from
// k = 900 on (3000 x 5000 x 1023: 123.5 -> 125.0, x 2047: 127.9 -> 130.5;
// forced configurations, back to back on one MI355X).
constexpr int kSmallStepDeepId = 13;
// stream-K with one workgroup per CU (see plan_split)
constexpr int kStreamKOnePerCuId = 6;
constexpr int kStreamKOnePerCuMinK = 1024;
constexpr int kStreamKOnePerCuMaxK = 2048;
constexpr double kStreamKOnePerCuEfficiency = 0.97;  // one 4-wave workgroup per CU
constexpr int kSmallStepDeepMinK = 848;

int choose_mfma_config(int m, int n, int k) {
    int best = kCandidates[0].id;
    double best_cost = tile_cost(m, n, best, kCandidates[0].efficiency);
    for (const Candidate &cand : kCandidates) {
        const double cost = tile_cost(m, n, cand.id, cand.efficiency);
        if (cost < best_cost * 0.999) {
            best = cand.id;
            best_cost = cost;
        }
    }
    if (best == 9 && tile_count(m, n, kTwoWorkgroupId) >= kTwoWorkgroupMinRounds * kCUs)
        best = kTwoWorkgroupId;
    if (best == 6 && k % 32 != 0 && tile_count(m, n, kSmallStepId) >= kSmallStepMinRounds * kCUs)
        best = k >= kSmallStepDeepMinK ? kSmallStepDeepId : kSmallStepId;
    return best;
}

// ---------------------------------------------------------------------------
// Split-K planning.
// ---------------------------------------------------------------------------
struct SplitPlan {
    int config;        // tile configuration of the partial (or full-k) kernel
    int splits;        // slices actually used (1: the full-k kernel, no workspace)
    int k_per_split;   // multiple of the k step
    long long slice;   // floats per workspace slice
    size_t bytes;      // workspace bytes including alignment slack (0 for one slice)
    int sk_grid;       // > 0: a stream-K schedule with this many workgroups instead
    long long sk_iters;  // stream-K: shared tiles * k steps
    int sk_ksteps;       // stream-K: k steps per tile
    long long sk_dp_tiles;  // stream-K: leading tiles computed whole, one per workgroup
    int sk_workers;         // stream-K: workgroups sharing the other tiles (0 or sk_grid)
};

constexpr size_t kWsAlign = 256;

// Slices of k for a request of `want` (>= 1): whole k steps per slice; the
// slice count that results may be smaller than asked.
SplitPlan make_plan(int m, int n, int k, long long want, int config) {
    SplitPlan sp{config, 0, 0, 0, 0, 0, 0, 0};
    if (m <= 0 || n <= 0 || k <= 0) return sp;
    const MfmaConfig &c = mfma_config(config);
    const long long kps = ceil_div(ceil_div(k, want), c.bk) * c.bk;
    sp.k_per_split = (int)kps;
    sp.splits = (int)ceil_div(k, kps);
    if (sp.splits == 1) sp.k_per_split = k;
    sp.slice = ceil_div((long long)m * n, 64) * 64;
    sp.bytes = sp.splits > 1 ? (size_t)sp.splits * (size_t)sp.slice * sizeof(float) + kWsAlign : 0;
    return sp;
}

// Modelled time (us) of a split plan.  Workgroups spread evenly over the
// CUs; the busiest CU runs ceil(tiles * S / CUs) of them, each for its k
// steps at the configuration's efficiency plus a fixed prologue / epilogue
// cost (divided among the workgroups one CU holds at once).  More than one
// slice adds the combine: a launch and 4 m n (S + 1) bytes at HBM speed.
// The constants are MI355X measurements: 2.4 GHz, ~3 us of prologue and
// epilogue per workgroup, ~3 us of fixed combine cost, ~6 TB/s.
constexpr double kClockMHz = 2400.0;
constexpr double kWorkgroupOverheadUs = 3.0;
constexpr double kCombineFixedUs = 3.0;
constexpr double kCombineBytesPerUs = 6.0e6;
constexpr size_t kAutoWorkspaceCap = size_t(512) << 20;  // automatic plans stay below this

long long resident_per_cu(int config);

double split_cost_us(int m, int n, const SplitPlan &sp, double efficiency) {
    const MfmaConfig &c = mfma_config(sp.config);
    const long long resident = resident_per_cu(sp.config);
    const long long per_cu = ceil_div(tile_count(m, n, sp.config) * sp.splits, kCUs);
    const double step_us = 2.0 * c.bm * c.bn * c.bk / 256.0 / efficiency / kClockMHz;
    double t = (double)per_cu *
               ((double)ceil_div(sp.k_per_split, c.bk) * step_us + kWorkgroupOverheadUs / resident);
    if (sp.splits > 1)
        t += kCombineFixedUs + 4.0 * (double)m * n * (sp.splits + 1) / kCombineBytesPerUs;
    return t;
}

double config_efficiency(int id) {
    for (const Candidate &cand : kCandidates)
        if (cand.id == id) return cand.efficiency;
    return 0.9;
}

// Workgroups of configuration `config` one CU holds at once (LDS, wave
// slots, and the register budget the kernel was built for).  LDS goes to
// workgroups in 1280-byte granules, 128 per CU (lds_granules): for
// workgroups of 32256 bytes and more, and of 53248 and 54272,
// hipOccupancyMaxActiveBlocksPerMultiprocessor reported one more resident
// workgroup (five, three) than ran on a CU at once on MI355X.
long long resident_per_cu(int config) {
    const MfmaConfig &c = mfma_config(config);
    const long long lds = (long long)c.stages * (c.bm * c.bk + c.bk * c.bn) * 4;
    const long long waves = (long long)c.wgm * c.wgn;
    long long r = kLdsGranulesPerCu / lds_granules(lds);
    if (r > 32 / waves) r = 32 / waves;
    if (c.max_wgs > 0 && r > c.max_wgs) r = c.max_wgs;
    return r < 1 ? 1 : r;
}

// A stream-K schedule for `grid` workgroups' worth of concurrent work (0: one
// per resident slot of every CU; never more than the iteration count or the
// fixup's part limit).  When the tiles fill whole rounds of the grid, every
// tile gets a workgroup of its own (no stream-K part).  Otherwise all rounds
// but the last full one do (data-parallel tiles), and `grid` more workgroups
// share the (tile, k step) iterations of the remaining tiles evenly (between
// one and two rounds' worth of tiles, or all of them when there are fewer
// than two rounds).  Workspace: two tile-sized slots per stream-K
// workgroup.
SplitPlan make_sk_plan(int m, int n, int k, int config, long long grid) {
    SplitPlan sp{config, 1, k, 0, 0, 0, 0, 0, 0};
    if (m <= 0 || n <= 0 || k <= 0) return sp;
    const MfmaConfig &c = mfma_config(config);
    const long long ksteps = ceil_div(k, c.bk);
    const long long tiles = tile_count(m, n, config);
    if (grid <= 0) grid = kCUs * resident_per_cu(config);
    if (grid > tiles * ksteps) grid = tiles * ksteps;
    if (grid > kFixupMaxParts) grid = kFixupMaxParts;
    long long dp = 0;
    if (tiles % grid == 0) dp = tiles;
    else if (tiles >= 2 * grid) dp = (tiles / grid - 1) * grid;
    sp.sk_grid = (int)grid;
    sp.sk_workers = dp == tiles ? 0 : (int)grid;
    sp.sk_dp_tiles = dp;
    sp.sk_iters = (tiles - dp) * ksteps;
    sp.sk_ksteps = (int)ksteps;
    sp.bytes = sp.sk_workers > 0
                   ? (size_t)sp.sk_workers * 2 * (size_t)c.bm * c.bn * sizeof(float) + kWsAlign
                   : 0;
    return sp;
}

// Modelled time (us) of a stream-K schedule: every workgroup runs its whole
// tiles and ceil(shared iterations / grid) k steps (the CUs' resident
// workgroups share the matrix cores), one prologue / epilogue per tile or
// segment, and the fixup reads the parts of at most grid - 1 shared tiles
// (about ksteps / share + 1 parts each).
double sk_cost_us(int m, int n, const SplitPlan &sp, double efficiency,
                  double seg_us = kWorkgroupOverheadUs) {
    (void)m;
    (void)n;
    const MfmaConfig &c = mfma_config(sp.config);
    const double step_us = 2.0 * c.bm * c.bn * c.bk / 256.0 / efficiency / kClockMHz;
    const long long rounds = sp.sk_dp_tiles / sp.sk_grid;
    const long long share = ceil_div(sp.sk_iters, sp.sk_grid);
    const long long per_wg = rounds * sp.sk_ksteps + share;
    const long long per_cu = ceil_div(sp.sk_grid, kCUs);
    double t = (double)per_cu * per_wg * step_us;
    if (share == 0) return t + (double)rounds * seg_us;
    const long long segments = rounds + ceil_div(share, sp.sk_ksteps) + 1;
    long long shared = sp.sk_grid - 1;
    if (shared > sp.sk_iters / sp.sk_ksteps) shared = sp.sk_iters / sp.sk_ksteps;
    const double parts = (double)sp.sk_ksteps / (double)share + 1.0;
    return t + (double)segments * seg_us + kCombineFixedUs +
           4.0 * c.bm * c.bn * (double)shared * parts / kCombineBytesPerUs;
}

// The split plan for a call: `splits` > 0 fixes the slice count (rounded to
// whole k steps), 0 lets the model choose it; `config` >= 0 fixes the tile
// configuration.  A plan of one slice runs the full-k kernel, and then (when
// the configuration is free) with the tiles mi_sgemm would choose.  Measured
// on MI355X at 512 x 512 x 262144: 16 slices of the 128 x 128 x 32 tile, one
// round of 256 workgroups.
SplitPlan plan_split(int m, int n, int k, int splits, int config, bool allow_sk = true,
                     size_t cap = kAutoWorkspaceCap) {
    if (m <= 0 || n <= 0 || k <= 0) return SplitPlan{config < 0 ? 0 : config, 0, 0, 0, 0};
    SplitPlan best{};
    double best_cost = 0.0;
    bool have = false;
    auto consider = [&](int id, long long want) {
        const SplitPlan sp = make_plan(m, n, k, want, id);
        if (splits == 0 && sp.bytes > cap) return;
        const double cost = split_cost_us(m, n, sp, config_efficiency(id));
        if (!have || cost < best_cost * 0.99) {
            best = sp;
            best_cost = cost;
            have = true;
        }
    };
    for (const Candidate &cand : kCandidates) {
        const int id = cand.id;
        if (config >= 0 && id != config) continue;
        if (splits > 0) {
            consider(id, splits);
            continue;
        }
        const long long ksteps = ceil_div(k, mfma_config(id).bk);
        for (long long want = 1; want <= 256 && want <= ksteps; want += (want < 32 ? 1 : 4))
            consider(id, want);
        // stream-K, when every workgroup's share spans at least a quarter of
        // a tile's k steps (a shared tile then has at most about five parts)
        const SplitPlan sk = make_sk_plan(m, n, k, id, 0);
        if (allow_sk && 4 * (sk.sk_iters / sk.sk_grid) >= sk.sk_ksteps &&
            sk.bytes <= cap) {
            const double cost = sk_cost_us(m, n, sk, config_efficiency(id));
            if (cost < best_cost * 0.97) {
                best = sk;
                best_cost = cost;
            }
        }
        // The 64 x 64 x 32 tile on stream-K with one workgroup per CU
        // instead of three: fewer, longer shares, and a segment's prologue
        // and epilogue move a quarter of a 128 x 128 tile's data.  From
        // k = 1024 on it beat the plans above on small grids (768^2 x 1024
        // 47.2 -> 57.8, 1536^2 x 1536 107.1 -> 116.5 TFLOP/s, one MI355X);
        // at k = 512 it lost.
        if (allow_sk && id == kStreamKOnePerCuId && k >= kStreamKOnePerCuMinK &&
            k <= kStreamKOnePerCuMaxK) {
            const SplitPlan sk1 = make_sk_plan(m, n, k, id, kCUs);
            if (sk1.sk_grid > 0 && 4 * (sk1.sk_iters / sk1.sk_grid) >= sk1.sk_ksteps &&
                sk1.bytes <= cap) {
                const MfmaConfig &c1 = mfma_config(id);
                const double seg = kWorkgroupOverheadUs * (double)(c1.bm * c1.bn) / (128.0 * 128.0);
                // (discounted only against a single pass or slices: where the
                // plan so far is stream-K itself, the one-per-CU form won every
                // measured case in this k range undiscounted)
                const double eff = config_efficiency(id) *
                                   (best.sk_grid > 0 ? 1.0 : kStreamKOnePerCuEfficiency);
                const double cost = sk_cost_us(m, n, sk1, eff, seg);
                if (cost < best_cost * 0.97) {
                    best = sk1;
                    best_cost = cost;
                }
            }
        }
    }
    if (!have) best = make_plan(m, n, k, splits > 0 ? splits : 1, config);  // forced non-candidate
    if (best.splits == 1 && best.sk_grid == 0 && config < 0) best.config = choose_mfma_config(m, n, k);
    return best;
}

// ---------------------------------------------------------------------------
// Checks shared by every entry point.
// ---------------------------------------------------------------------------
// Transpose flags are 0 (operand as given) or 1 (given transposed).  A
// stored row width is k for A and n for B, or m and k when transposed.
int check_sizes(int m, int n, int k, int lda, int ldb, int ldc, int ta = 0, int tb = 0) {
    if (m < 0 || n < 0 || k < 0) return MI_SGEMM_ERROR_INVALID_VALUE;
    if ((ta != 0 && ta != 1) || (tb != 0 && tb != 1)) return MI_SGEMM_ERROR_INVALID_VALUE;
    const int wa = ta ? m : k, wb = tb ? k : n;
    if (lda < (wa > 1 ? wa : 1) || ldb < (wb > 1 ? wb : 1) || ldc < (n > 1 ? n : 1))
        return MI_SGEMM_ERROR_INVALID_LD;
    return MI_SGEMM_SUCCESS;
}

int check_pointers(int m, int n, int k, float alpha, const float *A, const float *B,
                   const float *C) {
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    if (!C) return MI_SGEMM_ERROR_NULL_POINTER;
    if (k > 0 && alpha != 0.f && (!A || !B)) return MI_SGEMM_ERROR_NULL_POINTER;
    return MI_SGEMM_SUCCESS;
}

// The kernels are built for gfx950 only: refuse anything else up front.
int check_device() {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0) return MI_SGEMM_ERROR_DEVICE;
    static std::atomic<signed char> state[128];  // 0 unknown, 1 gfx950, -1 other
    if (dev >= 128) return MI_SGEMM_ERROR_DEVICE;
    const signed char s = state[dev].load(std::memory_order_acquire);
    if (s != 0) return s > 0 ? MI_SGEMM_SUCCESS : MI_SGEMM_ERROR_DEVICE;
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return MI_SGEMM_ERROR_DEVICE;
    const bool ok = std::strncmp(prop.gcnArchName, "gfx950", 6) == 0;
    state[dev].store(ok ? 1 : -1, std::memory_order_release);
    return ok ? MI_SGEMM_SUCCESS : MI_SGEMM_ERROR_DEVICE;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool vector_ok(const float *A, int lda, const float *B, int ldb) {
    return aligned16(A) && aligned16(B) && lda % 4 == 0 && ldb % 4 == 0;
}

// A dispatch describes its grid in work-items with 32 bits: launches beyond
// that are refused.  Only a C of about 2^36 elements and more, or a forced
// slice count of that order, comes near it; multi-kernel paths check their
// first large launch before anything is enqueued, so a refusal writes nothing.
bool launch_fits(long long grid, int threads) {
    return grid <= INT_MAX && grid * threads <= (long long)UINT32_MAX;
}

// Every launch reports the status hipLaunchKernel itself returns (not a
// sticky error another library may have left behind).
int launch_raw(const void *fn, long long grid, int threads, void **args, hipStream_t stream) {
    if (grid <= 0) return MI_SGEMM_SUCCESS;
    if (!launch_fits(grid, threads)) return MI_SGEMM_ERROR_INVALID_VALUE;
    return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), args, 0, stream) == hipSuccess
               ? MI_SGEMM_SUCCESS
               : MI_SGEMM_ERROR_LAUNCH;
}

int launch(KernelFn fn, long long grid, int threads, hipStream_t stream, GemmArgs args) {
    void *kargs[] = {&args};
    return launch_raw(reinterpret_cast<const void *>(fn), grid, threads, kargs, stream);
}

int launch_scale(int m, int n, float beta, float *C, int ldc, hipStream_t stream) {
    long long blocks = ceil_div((long long)m * n, 256);
    if (blocks > 4096) blocks = 4096;
    long long ldc64 = ldc;
    void *args[] = {&m, &n, &beta, &C, &ldc64};
    return launch_raw(reinterpret_cast<const void *>(&scale_c_kernel), blocks, 256, args, stream);
}

// The combine of `splits` partial slices (arguments checked).  It walks its
// chunks grid-stride, so the block count is capped.
int launch_combine(int m, int n, int splits, const float *ws, long long slice, float alpha,
                   float beta, float *C, int ldc, hipStream_t s) {
    const long long blocks =
        std::min(ceil_div(ceil_div((long long)m * n, 64), 4), kCombineMaxBlocks);
    long long ldc64 = ldc;
    void *args[] = {&ws, &slice, &splits, &m, &n, &alpha, &beta, &C, &ldc64};
    return launch_raw(reinterpret_cast<const void *>(&splitk_combine_kernel), blocks, 256, args, s);
}

GemmArgs base_args(int m, int n, int k, float alpha, const float *A, int lda, const float *B,
                   int ldb, float beta, float *C, int ldc) {
    GemmArgs a;
    std::memset(&a, 0, sizeof(a));
    a.m = m; a.n = n; a.k = k;
    a.alpha = alpha; a.beta = beta;
    a.A = A; a.lda = lda; a.B = B; a.ldb = ldb; a.C = C; a.ldc = ldc;
    a.group_m = kGroupM;
    a.xcd_remap = 1;
    a.c_vec = aligned16(C) && ldc % 4 == 0;
    return a;
}

// Common prologue of the compute entry points.  Returns SUCCESS with
// *done = true when the call is complete without a GEMM kernel.
int prologue(int m, int n, int k, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, hipStream_t stream, bool *done, int ta = 0,
             int tb = 0) {
    *done = true;
    int st = check_sizes(m, n, k, lda, ldb, ldc, ta, tb);
    if (st) return st;
    st = check_pointers(m, n, k, alpha, A, B, C);
    if (st) return st;
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    st = check_device();
    if (st) return st;
    if (k == 0 || alpha == 0.f) return launch_scale(m, n, beta, C, ldc, stream);
    *done = false;
    return MI_SGEMM_SUCCESS;
}

// The full-k matrix-core kernel of configuration `id` (arguments checked),
// in the grouped, XCD-aware workgroup order unless `order` overrides it
// ({xcd_remap, group_m}, measured comparisons only).
struct TileOrder {
    int xcd_remap, group_m;
};
constexpr TileOrder kDefaultOrder{1, kGroupM};

int launch_full(int id, int ta, int tb, int m, int n, int k, float alpha, const float *A, int lda,
                const float *B, int ldb, float beta, float *C, int ldc, hipStream_t s,
                TileOrder order = kDefaultOrder) {
    const MfmaConfig &c = mfma_config(id);
    GemmArgs a = base_args(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
    a.xcd_remap = order.xcd_remap;
    a.group_m = order.group_m;
    a.tiles_m = (int)ceil_div(m, c.bm);
    a.tiles_n = (int)ceil_div(n, c.bn);
    const long long grid = (long long)a.tiles_m * a.tiles_n;
    return launch(c.full[ta][tb][vector_ok(A, lda, B, ldb)], grid, 64 * c.wgm * c.wgn, s, a);
}

int run_mfma(int config, int ta, int tb, int m, int n, int k, float alpha, const float *A,
             int lda, const float *B, int ldb, float beta, float *C, int ldc, void *stream,
             TileOrder order = kDefaultOrder) {
    if (config >= kNumMfmaConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool done;
    int st = prologue(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s, &done, ta, tb);
    if (st || done) return st;
    const int id = config < 0 ? choose_mfma_config(m, n, k) : config;
    return launch_full(id, ta, tb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s, order);
}

// VALU configurations: 0 the 256-thread tile of the worked example, 1 the
// same tile with two k groups (512 threads; see sgemm_valu.hpp).  Two k
// groups win when each CU gets at most one workgroup (back to back on one
// MI355X, TFLOP/s, 256 -> 512 threads: 2048^3 57.5 -> 77.6, 1024^2 x 8192
// 14.8 -> 23.3); with more tiles the 256-thread tile puts two workgroups on
// a CU and wins (4096^3 91.7 -> 87.9, 8192^3 88.0 -> 82.0).  Without 16-byte
// loads the two-group instance spills (the element loads need more
// registers), so it is not chosen there.
constexpr int kNumValuConfigs = 2;
constexpr long long kValuKGroupMaxTiles = 256;
int choose_valu_config(long long tiles, bool vec) {
    return vec && tiles <= kValuKGroupMaxTiles ? 1 : 0;
}

int run_valu(int config, int m, int n, int k, float alpha, const float *A, int lda,
             const float *B, int ldb, float beta, float *C, int ldc, void *stream) {
    if (config >= kNumValuConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
    hipStream_t s = static_cast<hipStream_t>(stream);
    bool done;
    int st = prologue(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s, &done);
    if (st || done) return st;
    GemmArgs a = base_args(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
    a.tiles_m = (int)ceil_div(m, ValuTile::BM);
    a.tiles_n = (int)ceil_div(n, ValuTile::BN);
    const long long grid = (long long)a.tiles_m * a.tiles_n;
    const bool vec = vector_ok(A, lda, B, ldb);
    const int id = config < 0 ? choose_valu_config(grid, vec) : config;
    KernelFn fn = id == 1 ? (vec ? &sgemm_valu_kernel<true, 2> : &sgemm_valu_kernel<false, 2>)
                          : (vec ? &sgemm_valu_kernel<true, 1> : &sgemm_valu_kernel<false, 1>);
    return launch(fn, grid, ValuTile::NT * (id == 1 ? 2 : 1), s, a);
}

// Stream-K: the persistent-grid kernel, then the fixup of shared tiles.
int launch_streamk(const SplitPlan &sp, int ta, int tb, int m, int n, int k, float alpha,
                   const float *A, int lda, const float *B, int ldb, float beta, float *C,
                   int ldc, void *ws, hipStream_t s) {
    float *wsa = reinterpret_cast<float *>((reinterpret_cast<uintptr_t>(ws) + kWsAlign - 1) &
                                           ~(uintptr_t)(kWsAlign - 1));
    const MfmaConfig &c = mfma_config(sp.config);
    GemmArgs a = base_args(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
    a.tiles_m = (int)ceil_div(m, c.bm);
    a.tiles_n = (int)ceil_div(n, c.bn);
    a.ws = wsa;
    a.sk_iters = sp.sk_iters;
    a.sk_ksteps = sp.sk_ksteps;
    a.sk_dp_tiles = (int)sp.sk_dp_tiles;
    int st = launch(c.streamk[ta][tb][vector_ok(A, lda, B, ldb)], sp.sk_dp_tiles + sp.sk_workers,
                    64 * c.wgm * c.wgn, s, a);
    if (st || sp.sk_workers < 2) return st;
    const float *wsc = wsa;
    long long iters = sp.sk_iters, ldc64 = ldc;
    int ksteps = sp.sk_ksteps, grid = sp.sk_workers, tile0 = a.sk_dp_tiles;
    int tm = a.tiles_m, tn = a.tiles_n, gm = a.group_m;
    void *args[] = {&wsc, &iters, &ksteps, &grid, &tile0, &tm, &tn, &gm, &m, &n, &alpha, &beta, &C, &ldc64};
    return launch_raw(c.fixup, (long long)(sp.sk_workers - 1) * kFixupSplit, kFixupThreads, args, s);
}

// use_scratch: the workspace is the static scratch (ws ignored): the
// automatic plan keeps within it, a forced plan beyond it is refused.
int run_splitk(int config, int ta, int tb, int m, int n, int k, float alpha, const float *A,
               int lda, const float *B, int ldb, float beta, float *C, int ldc, int splits,
               void *ws, size_t ws_bytes, void *stream, bool use_scratch = false) {
    if (config >= kNumMfmaConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
    int st = check_sizes(m, n, k, lda, ldb, ldc, ta, tb);
    if (st) return st;
    if (splits < 0 || splits > k) return MI_SGEMM_ERROR_INVALID_VALUE;
    st = check_pointers(m, n, k, alpha, A, B, C);
    if (st) return st;
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0 || alpha == 0.f) {
        st = check_device();
        return st ? st : launch_scale(m, n, beta, C, ldc, s);
    }
    const SplitPlan sp =
        plan_split(m, n, k, splits, config, true, use_scratch ? kScratchBytes : kAutoWorkspaceCap);
    if (use_scratch) {
        if (sp.bytes > kScratchBytes) return MI_SGEMM_ERROR_SCRATCH_LIMIT;
    } else if (sp.bytes > 0 && (!ws || ws_bytes < sp.bytes)) {
        return MI_SGEMM_ERROR_WORKSPACE;
    }
    st = check_device();
    if (st) return st;
    if (use_scratch && sp.bytes > 0) {
        ws = scratch_address();
        if (!ws) return MI_SGEMM_ERROR_LAUNCH;
    }
    const int id = sp.config;
    if (sp.sk_grid > 0) return launch_streamk(sp, ta, tb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws, s);
    // one slice: the full-k kernel, no workspace (the same sums and rounding
    // as the partial-plus-combine path would give)
    if (sp.splits == 1) return launch_full(id, ta, tb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s);

    float *wsa = reinterpret_cast<float *>((reinterpret_cast<uintptr_t>(ws) + kWsAlign - 1) &
                                           ~(uintptr_t)(kWsAlign - 1));
    const MfmaConfig &c = mfma_config(id);
    GemmArgs a = base_args(m, n, k, 1.f, A, lda, B, ldb, 0.f, nullptr, ldc);
    a.tiles_m = (int)ceil_div(m, c.bm);
    a.tiles_n = (int)ceil_div(n, c.bn);
    a.k_per_split = sp.k_per_split;
    a.ws = wsa;
    a.ws_slice = sp.slice;
    const long long grid = (long long)a.tiles_m * a.tiles_n * sp.splits;
    st = launch(c.split[ta][tb][vector_ok(A, lda, B, ldb)], grid, 64 * c.wgm * c.wgn, s, a);
    if (st) return st;

    return launch_combine(m, n, sp.splits, wsa, sp.slice, alpha, beta, C, ldc, s);
}

// Split-K without a workspace: C <- beta*C, then every (tile, slice)
// workgroup adds alpha * (its slice sum) into C with float atomics.
int run_splitk_atomic(int config, int m, int n, int k, float alpha, const float *A, int lda,
                      const float *B, int ldb, float beta, float *C, int ldc, int splits,
                      void *stream) {
    if (config >= kNumMfmaConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
    int st = check_sizes(m, n, k, lda, ldb, ldc);
    if (st) return st;
    if (splits < 0 || splits > k) return MI_SGEMM_ERROR_INVALID_VALUE;
    st = check_pointers(m, n, k, alpha, A, B, C);
    if (st) return st;
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0 || alpha == 0.f) return launch_scale(m, n, beta, C, ldc, s);
    const SplitPlan sp = plan_split(m, n, k, splits, config, false);  // slices only
    const int id = sp.config;
    if (sp.splits == 1) return launch_full(id, 0, 0, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, s);
    const MfmaConfig &c = mfma_config(id);
    GemmArgs a = base_args(m, n, k, alpha, A, lda, B, ldb, beta, C, ldc);
    a.tiles_m = (int)ceil_div(m, c.bm);
    a.tiles_n = (int)ceil_div(n, c.bn);
    a.k_per_split = sp.k_per_split;
    const long long grid = (long long)a.tiles_m * a.tiles_n * sp.splits;
    const int threads = 64 * c.wgm * c.wgn;
    // checked before C is scaled, so that a refused launch leaves C as it was
    if (!launch_fits(grid, threads)) return MI_SGEMM_ERROR_INVALID_VALUE;
    if (beta != 1.f) {
        st = launch_scale(m, n, beta, C, ldc, s);
        if (st) return st;
    }
    return launch(c.atomic[vector_ok(A, lda, B, ldb)], grid, threads, s, a);
}

// Stream-K with a forced grid (0: automatic) and configuration (< 0: the
// candidate the model prefers).
SplitPlan plan_streamk(int m, int n, int k, int config, int grid) {
    if (config >= 0) return make_sk_plan(m, n, k, config, grid);
    SplitPlan best{};
    double best_cost = 0.0;
    for (const Candidate &cand : kCandidates) {
        const SplitPlan sp = make_sk_plan(m, n, k, cand.id, grid);
        if (sp.sk_grid == 0) return sp;  // empty problem
        const double cost = sk_cost_us(m, n, sp, cand.efficiency);
        if (best.sk_grid == 0 || cost < best_cost * 0.99) {
            best = sp;
            best_cost = cost;
        }
    }
    return best;
}

int run_streamk(int config, int ta, int tb, int m, int n, int k, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc, int grid,
                void *ws, size_t ws_bytes, void *stream) {
    if (config >= kNumMfmaConfigs || grid < 0) return MI_SGEMM_ERROR_INVALID_VALUE;
    int st = check_sizes(m, n, k, lda, ldb, ldc, ta, tb);
    if (st) return st;
    st = check_pointers(m, n, k, alpha, A, B, C);
    if (st) return st;
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (k == 0 || alpha == 0.f) {
        st = check_device();
        return st ? st : launch_scale(m, n, beta, C, ldc, s);
    }
    const SplitPlan sp = plan_streamk(m, n, k, config, grid);
    if (sp.bytes > 0 && (!ws || ws_bytes < sp.bytes)) return MI_SGEMM_ERROR_WORKSPACE;
    st = check_device();
    if (st) return st;
    return launch_streamk(sp, ta, tb, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, ws, s);
}

// ---------------------------------------------------------------------------
// Array sum.
// ---------------------------------------------------------------------------
// Partial-pass grid: at least 16 inputs (one unrolled float4 round) per lane,
// at most 32 workgroups per CU (four waves of residency): a 1 GiB input then
// gives each lane 128 inputs, the fastest point of a sweep over 8 to 64
// workgroups per CU and unroll depths 4 to 16.
long long reduce_grid(long long n) {
    static_assert(32 * kCUs <= kFinalThreads * kFinalPer, "final pass covers every partial");
    long long g = ceil_div(n, (long long)kReduceThreads * 16);
    if (g > 32 * kCUs) g = 32 * kCUs;
    return g < 1 ? 1 : g;
}

}  // namespace
}  // namespace mi

using namespace mi;

extern "C" {

int mi_sgemm(int m, int n, int k, float alpha, const float *A, int lda, const float *B, int ldb,
             float beta, float *C, int ldc, void *stream) {
    return run_mfma(-1, 0, 0, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int mi_sgemm_ex(int trans_a, int trans_b, int m, int n, int k, float alpha, const float *A,
                int lda, const float *B, int ldb, float beta, float *C, int ldc, void *stream) {
    return run_mfma(-1, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int mi_sgemm_valu(int m, int n, int k, float alpha, const float *A, int lda, const float *B,
                  int ldb, float beta, float *C, int ldc, void *stream) {
    return run_valu(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream);
}

int mi_sgemm_with_config(int kernel, int config, int trans_a, int trans_b, int m, int n, int k,
                         float alpha, const float *A, int lda, const float *B, int ldb,
                         float beta, float *C, int ldc, void *stream) {
    if (kernel == MI_SGEMM_KERNEL_MFMA)
        return run_mfma(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                        stream);
    if (kernel == MI_SGEMM_KERNEL_VALU && trans_a == 0 && trans_b == 0)
        return run_valu(config, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, stream);
    return MI_SGEMM_ERROR_INVALID_VALUE;
}

int mi_sgemm_with_order(int config, int xcd_remap, int group_m, int trans_a, int trans_b, int m,
                        int n, int k, float alpha, const float *A, int lda, const float *B,
                        int ldb, float beta, float *C, int ldc, void *stream) {
    if ((xcd_remap != 0 && xcd_remap != 1) || group_m < 1) return MI_SGEMM_ERROR_INVALID_VALUE;
    return run_mfma(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                    stream, TileOrder{xcd_remap, group_m});
}

size_t mi_sgemm_splitk_workspace_bytes(int m, int n, int k, int splits) {
    return mi_sgemm_splitk_with_config_workspace_bytes(-1, m, n, k, splits);
}

int mi_sgemm_splitk(int m, int n, int k, float alpha, const float *A, int lda, const float *B,
                    int ldb, float beta, float *C, int ldc, int splits, void *ws,
                    size_t ws_bytes, void *stream) {
    return run_splitk(-1, 0, 0, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits, ws,
                      ws_bytes, stream);
}

int mi_sgemm_splitk_ex(int trans_a, int trans_b, int m, int n, int k, float alpha,
                       const float *A, int lda, const float *B, int ldb, float beta, float *C,
                       int ldc, int splits, void *ws, size_t ws_bytes, void *stream) {
    return run_splitk(-1, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                      ws, ws_bytes, stream);
}

int mi_sgemm_splitk_noalloc(int trans_a, int trans_b, int m, int n, int k, float alpha,
                            const float *A, int lda, const float *B, int ldb, float beta, float *C,
                            int ldc, int splits, void *stream) {
    return run_splitk(-1, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits,
                      nullptr, 0, stream, true);
}

int mi_sgemm_splitk_with_config(int config, int trans_a, int trans_b, int m, int n, int k,
                                float alpha, const float *A, int lda, const float *B, int ldb,
                                float beta, float *C, int ldc, int splits, void *ws,
                                size_t ws_bytes, void *stream) {
    return run_splitk(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                      splits, ws, ws_bytes, stream);
}

int mi_sgemm_splitk_atomic(int m, int n, int k, float alpha, const float *A, int lda,
                           const float *B, int ldb, float beta, float *C, int ldc, int splits,
                           void *stream) {
    return run_splitk_atomic(-1, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc, splits, stream);
}

int mi_sgemm_streamk(int config, int trans_a, int trans_b, int m, int n, int k, float alpha,
                     const float *A, int lda, const float *B, int ldb, float beta, float *C,
                     int ldc, int grid, void *ws, size_t ws_bytes, void *stream) {
    return run_streamk(config, trans_a, trans_b, m, n, k, alpha, A, lda, B, ldb, beta, C, ldc,
                       grid, ws, ws_bytes, stream);
}

size_t mi_sgemm_streamk_workspace_bytes(int config, int m, int n, int k, int grid) {
    if (m < 0 || n < 0 || k < 0 || grid < 0 || config >= kNumMfmaConfigs) return 0;
    return plan_streamk(m, n, k, config, grid).bytes;
}

size_t mi_sgemm_splitk_with_config_workspace_bytes(int config, int m, int n, int k, int splits) {
    if (m < 0 || n < 0 || k < 0 || splits < 0 || splits > k || config >= kNumMfmaConfigs)
        return 0;
    return plan_split(m, n, k, splits, config).bytes;
}

int mi_sgemm_splitk_combine(int m, int n, int splits, const float *ws, long long slice,
                            float alpha, float beta, float *C, int ldc, void *stream) {
    if (m < 0 || n < 0 || splits < 0) return MI_SGEMM_ERROR_INVALID_VALUE;
    if (ldc < (n > 1 ? n : 1)) return MI_SGEMM_ERROR_INVALID_LD;
    if (m == 0 || n == 0) return MI_SGEMM_SUCCESS;
    if (!C || (splits > 0 && alpha != 0.f && !ws)) return MI_SGEMM_ERROR_NULL_POINTER;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (splits == 0 || alpha == 0.f) {
        const int st = check_device();
        return st ? st : launch_scale(m, n, beta, C, ldc, s);
    }
    // every float4 a lane reads lies inside its slice
    const long long mn = (long long)m * n;
    if (slice % 4 != 0 || slice < ceil_div(mn, 4) * 4 || !aligned16(ws))
        return MI_SGEMM_ERROR_INVALID_VALUE;
    const int st = check_device();
    return st ? st : launch_combine(m, n, splits, ws, slice, alpha, beta, C, ldc, s);
}

size_t mi_reduce_sum_workspace_bytes(long long n) {
    if (n <= 0) return 0;
    return (size_t)reduce_grid(n) * sizeof(float);
}

long long mi_reduce_sum_max_additions(long long n) {
    if (n <= 0) return 0;
    const long long g = reduce_grid(n);
    // groups of four per lane: workgroups take ceil(groups / g) each
    const long long per_acc = ceil_div(ceil_div(n >> 2, g), kReduceThreads);
    // per accumulator (+1 for a trailing element), 2 levels over the four
    // accumulators, 6 in the wave, 2 over the waves; then the final pass:
    // kFinalPer - 1 in a lane, 6 in the wave, 6 over the per-wave sums.
    return per_acc + 1 + 2 + 6 + 2 + (kFinalPer - 1) + 6 + 6;
}

int mi_reduce_sum(long long n, const float *x, float *out, void *ws, size_t ws_bytes,
                  void *stream) {
    if (n < 0) return MI_SGEMM_ERROR_INVALID_VALUE;
    if (!out || (n > 0 && !x)) return MI_SGEMM_ERROR_NULL_POINTER;
    const long long g = n > 0 ? reduce_grid(n) : 0;
    if (g > 0 && (!ws || ws_bytes < (size_t)g * sizeof(float))) return MI_SGEMM_ERROR_WORKSPACE;
    int st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    float *partials = static_cast<float *>(ws);
    if (g > 0) {
        const bool vec = (reinterpret_cast<uintptr_t>(x) & 15u) == 0;
        long long per = ceil_div(n >> 2, g);  // groups of four per workgroup
        void *args[] = {&x, &n, &per, &partials};
        st = launch_raw(vec ? reinterpret_cast<const void *>(&reduce_partial_kernel<true>)
                            : reinterpret_cast<const void *>(&reduce_partial_kernel<false>),
                        g, kReduceThreads, args, s);
        if (st) return st;
    }
    int count = (int)g;
    const float *pc = partials;
    void *args[] = {&pc, &count, &out};
    return launch_raw(reinterpret_cast<const void *>(&reduce_final_kernel), 1, kFinalThreads,
                      args, s);
}

int mi_clock_probe(unsigned long long *ticks, int workgroups, int spin_us, int *ref_khz,
                   void *stream) {
    if (workgroups < 1 || workgroups > kClockProbeMaxWorkgroups || spin_us < 1 ||
        spin_us > 100000)
        return MI_SGEMM_ERROR_INVALID_VALUE;
    if (!ticks || !ref_khz) return MI_SGEMM_ERROR_NULL_POINTER;
    int st = check_device();
    if (st) return st;
    int dev = 0, khz = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        khz <= 0)
        return MI_SGEMM_ERROR_DEVICE;
    *ref_khz = khz;
    long long spin = (long long)spin_us * khz / 1000;
    if (spin < 1) spin = 1;
    void *args[] = {&ticks, &spin};
    return launch_raw(reinterpret_cast<const void *>(&clock_probe_kernel), workgroups, 64, args,
                      static_cast<hipStream_t>(stream));
}

int mi_fma_rate_probe(int loop, float *out, int workgroups, int iters, void *stream) {
    if ((loop != kFmaOuter && loop != kFmaScalar) || workgroups < 1 || workgroups > 65536 ||
        iters < 1 || iters > 1000000)
        return MI_SGEMM_ERROR_INVALID_VALUE;
    if (!out) return MI_SGEMM_ERROR_NULL_POINTER;
    const int st = check_device();
    if (st) return st;
    hipStream_t s = static_cast<hipStream_t>(stream);
    if (loop == kFmaOuter) {
        void *args[] = {&out, &iters};
        return launch_raw(reinterpret_cast<const void *>(&fma_outer_kernel), workgroups, 256,
                          args, s);
    }
    float a = 0.999f, b = 1e-3f;
    void *args[] = {&out, &iters, &a, &b};
    return launch_raw(reinterpret_cast<const void *>(&fma_scalar_kernel), workgroups, 256, args, s);
}

const char *mi_status_string(int status) {
    switch (status) {
        case MI_SGEMM_SUCCESS: return "success";
        case MI_SGEMM_ERROR_INVALID_VALUE: return "invalid value (size, split count or id)";
        case MI_SGEMM_ERROR_INVALID_LD: return "leading dimension smaller than the row width";
        case MI_SGEMM_ERROR_NULL_POINTER: return "null pointer for an operand that is used";
        case MI_SGEMM_ERROR_WORKSPACE: return "workspace missing or too small";
        case MI_SGEMM_ERROR_LAUNCH: return "kernel launch failed";
        case MI_SGEMM_ERROR_DEVICE: return "no current gfx950 device";
        case MI_SGEMM_ERROR_SCRATCH_LIMIT:
            return "the plan needs more than the 64 MiB static scratch of mi_sgemm_splitk_noalloc";
        default: return "unknown status";
    }
}

int mi_sgemm_config_count(int kernel) {
    if (kernel == MI_SGEMM_KERNEL_MFMA) return kNumMfmaConfigs;
    if (kernel == MI_SGEMM_KERNEL_VALU) return kNumValuConfigs;
    if (kernel == MI_SGEMM_KERNEL_SPLITK || kernel == MI_SGEMM_KERNEL_SPLITK_ATOMIC)
        return kNumMfmaConfigs;
    return 0;
}

int mi_sgemm_get_plan(int kernel, int config, int m, int n, int k, int splits,
                      mi_sgemm_plan *plan) {
    if (!plan || m < 0 || n < 0 || k < 0) return MI_SGEMM_ERROR_INVALID_VALUE;
    std::memset(plan, 0, sizeof(*plan));
    plan->kernel = kernel;
    plan->group_m = kGroupM;
    plan->vector_loads = 1;
    plan->splits = 1;
    plan->k_per_split = k;
    long long sk_workgroups = 0;
    if (kernel == MI_SGEMM_KERNEL_VALU) {
        if (config >= kNumValuConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
        const long long tiles = ceil_div(m, ValuTile::BM) * ceil_div(n, ValuTile::BN);
        plan->config = config < 0 ? choose_valu_config(tiles, true) : config;
        plan->tile_m = ValuTile::BM; plan->tile_n = ValuTile::BN; plan->tile_k = ValuTile::BK;
        plan->micro_m = ValuTile::RM; plan->micro_n = ValuTile::RN;
        plan->threads = ValuTile::NT * (plan->config == 1 ? 2 : 1);
        plan->small_iterations = ValuTile::BK;
        plan->fma_per_small_iteration = ValuTile::RM * ValuTile::RN;
        plan->outputs_per_thread = ValuTile::RM * ValuTile::RN;
    } else if (kernel == MI_SGEMM_KERNEL_MFMA || kernel == MI_SGEMM_KERNEL_SPLITK ||
               kernel == MI_SGEMM_KERNEL_SPLITK_ATOMIC) {
        int id;
        const bool split = kernel != MI_SGEMM_KERNEL_MFMA;
        SplitPlan sp{};
        if (split) {
            if (config >= kNumMfmaConfigs || splits < 0 || splits > k)
                return MI_SGEMM_ERROR_INVALID_VALUE;
            sp = plan_split(m, n, k, splits, config, kernel == MI_SGEMM_KERNEL_SPLITK);
            id = (m > 0 && n > 0 && k > 0) ? sp.config
                                           : (config < 0 ? choose_mfma_config(m, n, k) : config);
        } else {
            if (config >= kNumMfmaConfigs) return MI_SGEMM_ERROR_INVALID_VALUE;
            id = config < 0 ? choose_mfma_config(m, n, k) : config;
        }
        const MfmaConfig &c = mfma_config(id);
        plan->config = id;
        plan->tile_m = c.bm; plan->tile_n = c.bn; plan->tile_k = c.bk;
        plan->micro_m = c.bm / c.wgm; plan->micro_n = c.bn / c.wgn;
        plan->threads = 64 * c.wgm * c.wgn;
        plan->small_iterations = c.bk / 2;
        plan->fma_per_small_iteration = (plan->micro_m / 32) * (plan->micro_n / 32);
        plan->outputs_per_thread = plan->micro_m * plan->micro_n / 64;
        if (split) {
            plan->stream_k_grid = kernel == MI_SGEMM_KERNEL_SPLITK ? sp.sk_grid : 0;
            if (plan->stream_k_grid > 0) sk_workgroups = sp.sk_dp_tiles + sp.sk_workers;
            plan->splits = sp.splits;
            plan->k_per_split = sp.k_per_split;
            plan->workspace_bytes = kernel == MI_SGEMM_KERNEL_SPLITK ? sp.bytes : 0;
        }
    } else {
        return MI_SGEMM_ERROR_INVALID_VALUE;
    }
    plan->tiles_m = (int)ceil_div(m, plan->tile_m);
    plan->tiles_n = (int)ceil_div(n, plan->tile_n);
    plan->workgroups = sk_workgroups > 0
                           ? sk_workgroups
                           : (long long)plan->tiles_m * plan->tiles_n * (plan->splits > 0 ? plan->splits : 1);
    plan->big_iterations = (int)ceil_div(plan->k_per_split, plan->tile_k);
    plan->a_elements_per_big_iteration = plan->tile_m * plan->tile_k;
    plan->b_elements_per_big_iteration = plan->tile_k * plan->tile_n;
    return MI_SGEMM_SUCCESS;
}

}  // extern "C"
