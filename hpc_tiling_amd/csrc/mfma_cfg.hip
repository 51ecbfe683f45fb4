// mfma_cfg.hip -- the matrix-core kernel instances and launch table of one
// tile configuration; built once per configuration with -DMI_CFG_ID=<id>.
#include "mfma_configs.hpp"

#ifndef MI_CFG_ID
#error "build with -DMI_CFG_ID=<configuration id>"
#endif

#define MI_CFG_NAME2(id) kMfmaConfig##id
#define MI_CFG_NAME(id) MI_CFG_NAME2(id)

namespace mi {
static_assert(MI_CFG_ID >= 0 && MI_CFG_ID < kNumMfmaConfigs, "unknown configuration id");
extern const MfmaConfig MI_CFG_NAME(MI_CFG_ID) = make_cfg<TileOf<MI_CFG_ID>::type>();
}  // namespace mi
