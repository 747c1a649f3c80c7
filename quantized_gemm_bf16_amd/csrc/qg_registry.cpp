// The kernel registry table ("all registered GEMM kernels for the current
// device", page "InternLM Lmdeploy Gemm Interface", Description).
#include "qg_registry.hpp"
#include "qg_tile.hpp"

namespace qg {

#define QG_DECL(E, BM, BN, WM, WN, ST) \
  extern template hipError_t launch_tile<TileCfg<El::E, BM, BN, WM, WN, ST>>(const Args&, int, hipStream_t);
#define QG_TILE_BF16(BM, BN, WM, WN, ST) QG_DECL(BF16, BM, BN, WM, WN, ST)
#define QG_TILE_F16(BM, BN, WM, WN, ST) QG_DECL(F16, BM, BN, WM, WN, ST)
#define QG_TILE_I8(BM, BN, WM, WN, ST) QG_DECL(I8, BM, BN, WM, WN, ST)
#include "qg_kernel_list.inc"
#undef QG_TILE_BF16
#undef QG_TILE_F16
#undef QG_TILE_I8

#define QG_ENTRY(E, DT, BM, BN, WM, WN, ST)                                                                   \
  {"tile_" #E "_" #BM "x" #BN "_w" #WM "x" #WN "_s" #ST, FAM_TILE, DT, BM, BN,                               \
   TileCfg<El::E, BM, BN, WM, WN, ST>::BK, ST, TileCfg<El::E, BM, BN, WM, WN, ST>::NT, BM * BN * 4,         \
   &launch_tile<TileCfg<El::E, BM, BN, WM, WN, ST>>},
#define QG_TILE_BF16(BM, BN, WM, WN, ST) QG_ENTRY(BF16, DT_BF16, BM, BN, WM, WN, ST)
#define QG_TILE_F16(BM, BN, WM, WN, ST) QG_ENTRY(F16, DT_F16, BM, BN, WM, WN, ST)
#define QG_TILE_I8(BM, BN, WM, WN, ST) QG_ENTRY(I8, DT_I8, BM, BN, WM, WN, ST)

// (not const: a const table would also be placed in device constant memory)
KernelInfo kKernels[] = {
#include "qg_kernel_list.inc"
};
extern const int kNumKernels;
const int kNumKernels = sizeof(kKernels) / sizeof(kKernels[0]);

}  // namespace qg
