// Kernel argument block shared by the host engine and the gfx950 kernels.
#pragma once
#include <stdint.h>

namespace qg {

enum Mode : int32_t { MODE_DP = 0, MODE_SPLITK = 1, MODE_STREAMK = 2, MODE_GROUPED = 3 };

enum EpiFlag : int32_t { EPI_BIAS = 1, EPI_RELU = 2, EPI_GELU = 4, EPI_QUANT_I8 = 8 };

enum DType : int32_t { DT_F32 = 0, DT_F16 = 1, DT_BF16 = 2, DT_E4M3 = 3, DT_I8 = 4, DT_I32 = 5, DT_U4 = 6 };

struct Args {
  // operands (device pointers)
  const void* A;
  const void* B;
  const void* C;
  void* D;
  const void* U;        // fp8: A scales fp32 [M, ldu]
  const void* V;        // int4: fp16 [N, ldv]; fp8: fp32 [N/128, ldv] per group
  const int32_t* offsets;  // grouped: E + 1 row offsets
  int64_t lda, ldb, ldc, ldd, ldu, ldv;  // elements (B: words for u4)
  int64_t b_batch, v_batch;              // grouped strides (elements / words)
  int32_t M, N, K;
  int32_t E;                             // grouped: number of experts
  float alpha, beta;
  int32_t c_type;                        // DType of C, -1 = C not read
  int32_t d_type;                        // DType of D
  int32_t zero_point;                    // int4
  int32_t group_k;                       // int4 scale group along K

  // epilogue (flags as in the C ABI's qg_epilogue)
  int32_t epi;
  int32_t int_scaled;                    // int8 sums scaled by U[m*ldu] * V[n*ldv] (w8a8)
  int32_t bias_type;
  const void* bias;                      // N values, or null
  const float* row_scale;                // output quantisation: one per row of D
  float out_zero_point;

  // work division
  int32_t mode;
  int32_t tiles_m, tiles_n;  // DP/split/stream: exact; grouped: tiles_n only
  int32_t iters;             // k-iterations (k-tiles) per output tile
  int32_t splits, iters_per_split;
  int32_t programs;          // stream-K: programs (one per workgroup)
  int32_t dp_tiles;          // stream-K: leading tiles taken whole, round-robin
  int32_t sk_work;           // stream-K: k-iterations of the remaining tiles, shared evenly
  int32_t group_m;           // tile-order super-group height (in tiles)
  int32_t grid;              // workgroups launched
  int32_t* counters;         // barriers workspace: one int32 per output tile
  void* partials;            // partials workspace

  // measurement (split-K only, set by qg_run_timed; null otherwise): 8
  // timestamps per split-K unit, see Sched::run_splitk
  uint64_t* stamps;
};

}  // namespace qg
