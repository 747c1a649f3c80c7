// Explicit instantiations of the block-scaled fp8 kernels listed in
// qg_kernel_list.inc.
#include "qg_fp8.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS)
#define QG_W4(MT, BN, WN, WK, ST)
#define QG_F8(BM, BN, WM, WN, ST) \
  template hipError_t launch_f8<F8Cfg<BM, BN, WM, WN, ST>>(const Args&, int, hipStream_t);
#include "qg_kernel_list.inc"
}  // namespace qg
