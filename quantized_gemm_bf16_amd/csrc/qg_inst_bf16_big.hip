// Explicit instantiations of the 256 x 256 bf16 tile kernels listed in
// qg_kernel_list.inc (QG_TILE_BF16_BIG).
#include "qg_tile.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS)
#undef QG_TILE_BF16_BIG
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB) \
  template hipError_t launch_tile<TileCfg<El::BF16, BM, BN, WM, WN, ST, RB>>(const Args&, int, hipStream_t);
#define QG_W4(MT, BN, WN, WK, ST)
#define QG_F8(BM, BN, WM, WN, ST)
#include "qg_kernel_list.inc"
}  // namespace qg
