// The kernel registry table ("all registered GEMM kernels for the current
// device", page "InternLM Lmdeploy Gemm Interface", Description).
#include "qg_registry.hpp"
#include "qg_w4.hpp"
#include "qg_fp8.hpp"

namespace qg {

#define QG_DECL(E, BM, BN, WM, WN, ST, RB) \
  extern template hipError_t launch_tile<TileCfg<El::E, BM, BN, WM, WN, ST, RB>>(const Args&, int, hipStream_t);
#define QG_DECL_SK(E, BN, NW, MT, DP, BB, NS) \
  extern template hipError_t launch_skinny<SkinnyCfg<El::E, BN, NW, MT, DP, BB, NS>>(const Args&, int, hipStream_t);
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB) QG_DECL(BF16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB) QG_DECL(BF16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB) QG_DECL(F16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB) QG_DECL(I8, BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS) QG_DECL_SK(BF16, BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS) QG_DECL_SK(F16, BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS) QG_DECL_SK(I8, BN, NW, MT, DP, BB, NS)
#define QG_W4(MT, BN, WN, WK, ST) \
  extern template hipError_t launch_w4<W4Cfg<MT, BN, WN, WK, ST>>(const Args&, int, hipStream_t);
#define QG_F8(BM, BN, WM, WN, ST) \
  extern template hipError_t launch_f8<F8Cfg<BM, BN, WM, WN, ST>>(const Args&, int, hipStream_t);
#include "qg_kernel_list.inc"
#undef QG_W4
#undef QG_F8
#undef QG_TILE_BF16
#undef QG_TILE_BF16_BIG
#undef QG_TILE_F16
#undef QG_TILE_I8
#undef QG_SKINNY_BF16
#undef QG_SKINNY_F16
#undef QG_SKINNY_I8

#define QG_ENTRY(E, DT, BM, BN, WM, WN, ST, RB)                                                          \
  {"tile_" #E "_" #BM "x" #BN "x" #RB "b_w" #WM "x" #WN "_s" #ST, FAM_TILE, DT, BM, BN,                 \
   TileCfg<El::E, BM, BN, WM, WN, ST, RB>::BK, ST, TileCfg<El::E, BM, BN, WM, WN, ST, RB>::NT, BM * BN * 4, \
   &launch_tile<TileCfg<El::E, BM, BN, WM, WN, ST, RB>>},
#define QG_ENTRY_SK(E, DT, BN, NW, MT, DP, BB, NS)                                                                  \
  {"skinny_" #E "_" #MT "x16x" #BN "x" #BB "b_w" #NW "_d" #DP "_n" #NS, FAM_SKINNY, DT, 16 * MT, BN,                          \
   SkinnyCfg<El::E, BN, NW, MT, DP, BB, NS>::BK, DP, SkinnyCfg<El::E, BN, NW, MT, DP, BB, NS>::NT, 16 * MT * BN * 4,        \
   &launch_skinny<SkinnyCfg<El::E, BN, NW, MT, DP, BB, NS>>},
#define QG_TILE_BF16(BM, BN, WM, WN, ST, RB) QG_ENTRY(BF16, DT_BF16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_BF16_BIG(BM, BN, WM, WN, ST, RB) QG_ENTRY(BF16, DT_BF16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_F16(BM, BN, WM, WN, ST, RB) QG_ENTRY(F16, DT_F16, BM, BN, WM, WN, ST, RB)
#define QG_TILE_I8(BM, BN, WM, WN, ST, RB) QG_ENTRY(I8, DT_I8, BM, BN, WM, WN, ST, RB)
#define QG_SKINNY_BF16(BN, NW, MT, DP, BB, NS) QG_ENTRY_SK(BF16, DT_BF16, BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_F16(BN, NW, MT, DP, BB, NS) QG_ENTRY_SK(F16, DT_F16, BN, NW, MT, DP, BB, NS)
#define QG_SKINNY_I8(BN, NW, MT, DP, BB, NS) QG_ENTRY_SK(I8, DT_I8, BN, NW, MT, DP, BB, NS)

#define QG_W4(MT, BN, WN, WK, ST)                                                                     \
  {"w4_BF16_" #MT "x16x" #BN "_w" #WN "x" #WK "_s" #ST, FAM_W4, DT_BF16, 16 * MT, BN,                     \
   W4Cfg<MT, BN, WN, WK, ST>::BK, ST, W4Cfg<MT, BN, WN, WK, ST>::NT, 16 * MT * BN * 4,                   \
   &launch_w4<W4Cfg<MT, BN, WN, WK, ST>>},

#define QG_F8(BM, BN, WM, WN, ST)                                                                         \
  {"f8_E4M3_" #BM "x" #BN "_w" #WM "x" #WN "_s" #ST, FAM_F8, DT_E4M3, BM, BN, 128, ST, WM * WN * 64, BM * BN * 4, \
   &launch_f8<F8Cfg<BM, BN, WM, WN, ST>>},

// (not const: a const table would also be placed in device constant memory)
KernelInfo kKernels[] = {
#include "qg_kernel_list.inc"
};
extern const int kNumKernels;
const int kNumKernels = sizeof(kKernels) / sizeof(kKernels[0]);

}  // namespace qg
