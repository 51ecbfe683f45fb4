// mfma_configs.hpp -- the tile configurations of the matrix-core kernel and
// the launch table of each one.  The kernel instances of configuration N are
// compiled in their own translation unit (mfma_cfg.hip built with
// -DMI_CFG_ID=N), so the configurations build in parallel; the host code
// reaches them through mfma_config(id).
#pragma once

#include <hip/hip_runtime.h>

#include "sgemm_mfma.hpp"
#include "streamk.hpp"

namespace mi {

using KernelFn = void (*)(GemmArgs);

// Kernel tables are indexed [trans_a][trans_b][vector loads].
struct MfmaConfig {
    int bm, bn, bk, wgm, wgn;
    int stages;    // LDS buffers in the ring
    int max_wgs;   // workgroups per CU the register budget allows (0: no limit beyond LDS and waves)
    KernelFn full[2][2][2];   // full-k kernels
    KernelFn split[2][2][2];  // split-K partial kernels
    KernelFn atomic[2];       // split-K kernels adding into C atomically (operands as given)
    KernelFn streamk[2][2][2];  // stream-K kernels
    const void *fixup;          // stream-K fixup for this tile size
};

template <class T, int MODE, bool TA, bool TB>
constexpr void fill_pair(KernelFn (&f)[2]) {
    f[0] = &sgemm_mfma_kernel<T, false, MODE, TA, TB>;
    f[1] = &sgemm_mfma_kernel<T, true, MODE, TA, TB>;
}

template <class T, int MODE>
constexpr void fill_table(KernelFn (&f)[2][2][2]) {
    fill_pair<T, MODE, false, false>(f[0][0]);
    fill_pair<T, MODE, false, true>(f[0][1]);
    fill_pair<T, MODE, true, false>(f[1][0]);
    fill_pair<T, MODE, true, true>(f[1][1]);
}

template <class T>
constexpr MfmaConfig make_cfg() {
    MfmaConfig c{T::BM, T::BN, T::BK, T::WGM, T::WGN, T::STAGES, T::WGS > 1 ? T::WGS : 0,
                 {}, {}, {}, {}, nullptr};
    fill_table<T, kFull>(c.full);
    fill_table<T, kPartial>(c.split);
    fill_pair<T, kAtomic, false, false>(c.atomic);
    fill_table<T, kStreamK>(c.streamk);
    c.fixup = reinterpret_cast<const void *>(&streamk_fixup_kernel<T::BM, T::BN>);
    return c;
}

// Configuration ids: MfmaTile<BM, BN, BK, waves along m, waves along n[, buffers]>.
template <int ID> struct TileOf;
template <> struct TileOf<0> { using type = MfmaTile<128, 128, 16, 2, 2>; };
template <> struct TileOf<1> { using type = MfmaTile<128, 128, 32, 2, 2>; };
template <> struct TileOf<2> { using type = MfmaTile<128, 128, 16, 2, 4>; };
template <> struct TileOf<3> { using type = MfmaTile<128, 128, 32, 2, 4>; };
template <> struct TileOf<4> { using type = MfmaTile<256, 128, 16, 2, 4>; };
template <> struct TileOf<5> { using type = MfmaTile<128, 256, 16, 2, 4>; };
template <> struct TileOf<6> { using type = MfmaTile<64, 64, 32, 2, 2>; };
template <> struct TileOf<7> { using type = MfmaTile<256, 128, 32, 2, 4>; };
template <> struct TileOf<8> { using type = MfmaTile<128, 64, 32, 2, 2>; };
// 16 waves, one workgroup per CU: a four-buffer ring (128 KB of LDS)
template <> struct TileOf<9> { using type = MfmaTile<128, 128, 32, 4, 4, 4>; };
// two-buffer rings, two workgroups per CU
template <> struct TileOf<10> { using type = MfmaTile<128, 128, 16, 2, 4, 2>; };
template <> struct TileOf<11> { using type = MfmaTile<128, 128, 32, 4, 2, 2>; };
// 64 x 64 x 16 built for six workgroups per CU
template <> struct TileOf<12> { using type = MfmaTile<64, 64, 16, 2, 2, 3, 6>; };
// the same tile with a four-buffer ring, four workgroups per CU
template <> struct TileOf<13> { using type = MfmaTile<64, 64, 16, 2, 2, 4, 4>; };
// 8 waves, two workgroups per CU, a four-buffer ring (64 KB of LDS each)
template <> struct TileOf<14> { using type = MfmaTile<128, 128, 16, 4, 2, 4, 2>; };
constexpr int kNumMfmaConfigs = 15;

// One table per configuration, each defined (constant-initialised) in its
// own build of mfma_cfg.hip.
extern const MfmaConfig kMfmaConfig0, kMfmaConfig1, kMfmaConfig2, kMfmaConfig3, kMfmaConfig4,
    kMfmaConfig5, kMfmaConfig6, kMfmaConfig7, kMfmaConfig8, kMfmaConfig9, kMfmaConfig10,
    kMfmaConfig11, kMfmaConfig12, kMfmaConfig13, kMfmaConfig14;

}  // namespace mi
