// Explicit instantiations of the W4A16 kernels listed in qg_kernel_list.inc.
#include "qg_w4.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS)
#define QG_W4(MT, BN, WN, WK, ST) \
  template hipError_t launch_w4<W4Cfg<MT, BN, WN, WK, ST>>(const Args&, int, hipStream_t);
#define QG_F8(BM, BN, WM, WN, ST)
#include "qg_kernel_list.inc"
}  // namespace qg
