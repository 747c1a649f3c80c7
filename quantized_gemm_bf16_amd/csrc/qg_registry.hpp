// Kernel registry: every precompiled gfx950 kernel instance with its traits.
#pragma once
#include <hip/hip_runtime.h>
#include "qg_args.hpp"

namespace qg {

enum KernelFamily : int { FAM_TILE = 0, FAM_SKINNY = 1, FAM_W4 = 2, FAM_F8 = 3 };

typedef hipError_t (*LaunchFn)(const Args& a, int grid, hipStream_t s);

struct KernelInfo {
  const char* name;
  int family;      // KernelFamily
  int in_type;     // DType of A (and B, except u4)
  int bm, bn, bk;  // output tile and k-tile (elements)
  int stages;
  int threads;
  int slot_bytes;  // bytes of one partial tile (BM*BN*4)
  LaunchFn launch;
};

extern KernelInfo kKernels[];
extern const int kNumKernels;

}  // namespace qg
