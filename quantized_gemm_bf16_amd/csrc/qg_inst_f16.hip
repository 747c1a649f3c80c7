// Explicit instantiations of the f16 tile kernels listed in qg_kernel_list.inc.
#include "qg_tile.hpp"

namespace qg {
#define QG_TILE_BF16(BM, BN, WM, WN, ST)
#define QG_TILE_F16(BM, BN, WM, WN, ST)
#define QG_TILE_I8(BM, BN, WM, WN, ST)
#undef QG_TILE_F16
#define QG_TILE_F16(BM, BN, WM, WN, ST) \
  template hipError_t launch_tile<TileCfg<El::F16, BM, BN, WM, WN, ST>>(const Args&, int, hipStream_t);
#include "qg_kernel_list.inc"
}  // namespace qg
