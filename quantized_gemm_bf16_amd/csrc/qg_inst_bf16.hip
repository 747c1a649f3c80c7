// Explicit instantiations of the bf16 kernels listed in qg_kernel_list.inc.
#include "qg_w4.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS)
#undef QG_TILE_BF16
#undef QG_SKINNY_BF16
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB) \
  template hipError_t launch_tile<TileCfg<El::BF16, BM, BN, WM, WN, ST, RB>>(const Args&, int, hipStream_t);
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS) \
  template hipError_t launch_skinny<SkinnyCfg<El::BF16, BN, NW, MT, DP, BB, NS>>(const Args&, int, hipStream_t);
#define QG_W4(BM, BN, NW, ST) template hipError_t launch_w4<W4Cfg<BM, BN, NW, ST>>(const Args&, int, hipStream_t);
#define QG_F8(BM, BN, WM, WN, ST)
#include "qg_kernel_list.inc"
}  // namespace qg
