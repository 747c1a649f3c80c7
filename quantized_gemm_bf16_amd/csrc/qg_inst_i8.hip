// Explicit instantiations of the i8 kernels listed in qg_kernel_list.inc.
#include "qg_skinny.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS)
#undef QG_TILE_I8
#undef QG_SKINNY_I8
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB) \
  template hipError_t launch_tile<TileCfg<El::I8, BM, BN, WM, WN, ST, RB>>(const Args&, int, hipStream_t);
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS) \
  template hipError_t launch_skinny<SkinnyCfg<El::I8, BN, NW, MT, DP, BB, NS>>(const Args&, int, hipStream_t);
#define QG_W4(MT, BN, WN, WK, ST)
#define QG_F8(BM, BN, WM, WN, ST)
#include "qg_kernel_list.inc"
}  // namespace qg
