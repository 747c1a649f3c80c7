// Measurement kernels and host loops of libqgceil.so (see include/qgceil.h):
// the chip's sustained MFMA rate and shader clock, its sustained streaming
// read rate, and the host cost of a launch, measured in the benchmark's own
// process next to the GEMM kernels they bound.
#include <hip/hip_runtime.h>

#include <chrono>

#include "../../include/qgceil.h"

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kMfmaThreads = 512;
constexpr int kMfmaLds = 96 * 1024;  // > 80 KiB: one workgroup per CU
constexpr int kStreamThreads = 256;
constexpr int kStreamLoads = 8;      // 16-byte loads in flight per thread

__global__ __launch_bounds__(kMfmaThreads) void mfma_loop(int iters, float* sink, uint64_t* clk) {
  __shared__ char lds[kMfmaLds];
  const int t = threadIdx.x;
  // operands that depend on the thread, so the loop cannot be folded
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((t + j) & 7) * 0.125f);
    b[j] = (__bf16)((float)((t * 3 + j) & 7) * -0.0625f);
  }
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  if (t == 0) ((volatile char*)lds)[blockIdx.x % kMfmaLds] = 1;  // keeps the LDS allocation
  __syncthreads();
  const uint64_t t0 = __builtin_readcyclecounter();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < iters; ++i) {
    c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
  }
  const uint64_t t1 = __builtin_readcyclecounter();
  const uint64_t r1 = __builtin_amdgcn_s_memrealtime();
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  if (t == 0) {
    sink[blockIdx.x] = s + (float)((volatile char*)lds)[blockIdx.x % kMfmaLds];
    clk[2 * blockIdx.x] = t1 - t0;
    clk[2 * blockIdx.x + 1] = r1 - r0;
  }
}

// Values the compiler cannot fold: the loop below must keep its constants
// in registers (as the int4 unpack does) and its fp16 operand live.
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_sgpr() {
  uint32_t r;
  asm("s_mov_b32 %0, %1" : "=s"(r) : "i"(V));
  return r;
}
template <uint32_t V>
__device__ __forceinline__ uint32_t opaque_vgpr() {
  uint32_t r;
  asm("v_mov_b32 %0, %1" : "=v"(r) : "i"(V));
  return r;
}

// One round: four slots of one MFMA (MODE bit 0) and four VALU instructions
// (MODE bit 1). The eight VALU chains advance once every other slot, so a
// chain's next instruction is eight instructions after its last one.
template <int MODE, int KIND>
__global__ __launch_bounds__(kMfmaThreads) void issue_mix(int iters, float* sink, uint64_t* clk) {
  __shared__ char lds[kMfmaLds];
  const int t = threadIdx.x;
  bf16x8 a, b;
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    a[j] = (__bf16)((float)((t + j) & 7) * 0.125f);
    b[j] = (__bf16)((float)((t * 3 + j) & 7) * -0.0625f);
  }
  f32x4 acc[4] = {};
  float x[8];
  uint32_t u[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    x[j] = (float)t * 1e-3f + (float)j;
    u[j] = (uint32_t)t * 0x9E3779B9u + (uint32_t)j;
  }
  const float y = __builtin_bit_cast(float, opaque_vgpr<0x3f7fbe77u>());  // 0.999
  const float z = __builtin_bit_cast(float, opaque_vgpr<0x38d1b717u>());  // 1e-4
  _Float16 h = (_Float16)(float)__builtin_bit_cast(float, opaque_vgpr<0x3c000000u>());  // 2^-7
  const uint32_t m = opaque_sgpr<0x000F000Fu>(), c = opaque_vgpr<0x43004300u>();
  const uint32_t sel = opaque_sgpr<0x0C040C00u>();
  if (t == 0) ((volatile char*)lds)[blockIdx.x % kMfmaLds] = 1;  // keeps the LDS allocation
  __syncthreads();
  const uint64_t t0 = __builtin_readcyclecounter();
  for (int i = 0; i < iters; ++i) {
    // the fp16 operand as a new value each round (the statement emits
    // nothing), so that the conversion is not hoisted out of the loop and the
    // multiply-adds stay mixed-precision instructions
    if constexpr (KIND == 2) asm volatile("" : "+v"(h));
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if constexpr (MODE & 1)
        acc[q] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc[q], 0, 0, 0);
      if constexpr (MODE & 2) {
        const int j0 = (q & 1) * 4;
        if constexpr (KIND == 1) {
#pragma unroll
          for (int j = j0; j < j0 + 2; ++j) u[j] = (__builtin_amdgcn_perm(u[j], u[j], sel) & m) | c;
        } else {
#pragma unroll
          for (int j = j0; j < j0 + 4; ++j)
            x[j] = KIND == 0 ? __builtin_fmaf(x[j], y, z) : __builtin_fmaf((float)h, x[j], y);
        }
      }
    }
  }
  // until every wave is done: the older wave of a SIMD wins the issue
  // arbitration and finishes first, so one wave's own time would undercount
  __syncthreads();
  const uint64_t t1 = __builtin_readcyclecounter();
  float s = 0.f;
#pragma unroll
  for (int q = 0; q < 4; ++q) s += acc[q][0] + acc[q][3];
#pragma unroll
  for (int j = 0; j < 8; ++j) s += x[j] + (float)(u[j] & 1);
  if (t == 0) {
    sink[blockIdx.x] = s + (float)((volatile char*)lds)[blockIdx.x % kMfmaLds];
    clk[blockIdx.x] = t1 - t0;
  }
}

// Workgroup g reads the 32 KiB blocks g, g + grid, ... : each thread loads
// kStreamLoads 16-byte pieces 4 KiB apart, all lanes together whole 4 KiB
// spans, and folds them into one dword. Buffer loads past `bytes` return
// zero, so the tail needs no branch.
__global__ __launch_bounds__(kStreamThreads) void stream_read(const char* src, uint32_t bytes, uint32_t* sink) {
  constexpr uint32_t kBlockBytes = kStreamThreads * kStreamLoads * 16;
  const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc((void*)src, (short)0, (int)bytes, 0x00020000);
  i32x4 acc = {0, 0, 0, 0};
  for (uint64_t off = (uint64_t)blockIdx.x * kBlockBytes; off < bytes; off += (uint64_t)gridDim.x * kBlockBytes) {
    i32x4 v[kStreamLoads];
#pragma unroll
    for (int j = 0; j < kStreamLoads; ++j)
      v[j] = __builtin_bit_cast(i32x4, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (uint32_t)off + (uint32_t)(j * kStreamThreads + threadIdx.x) * 16, 0, 0));
#pragma unroll
    for (int j = 0; j < kStreamLoads; ++j) acc ^= v[j];
  }
  sink[(size_t)blockIdx.x * kStreamThreads + threadIdx.x] = (uint32_t)(acc[0] ^ acc[1] ^ acc[2] ^ acc[3]);
}

__global__ void empty_kernel() {}

// An empty kernel with a 256-byte argument block: the runtime copies the
// arguments of every launch, so this is the launch floor for a kernel that
// takes arguments (the GEMM kernels take one block of about that size).
struct ArgBlock {
  char bytes[256];
};
__global__ void empty_args_kernel(const ArgBlock) {}

int launched() {
  if (hipGetLastError() != hipSuccess) return QG_ERR_HIP;
  return QG_OK;
}

}  // namespace

extern "C" {

int qgc_mfma_loop(int grid, int iters, float* sink, uint64_t* clk, hipStream_t stream) {
  if (grid < 1 || grid > 65535 || iters < 1 || iters > (1 << 20) || !sink || !clk) return QG_ERR_INVALID_ARG;
  hipLaunchKernelGGL(mfma_loop, dim3(grid), dim3(kMfmaThreads), 0, stream, iters, sink, clk);
  return launched();
}

int qgc_stream_read(const void* src, size_t bytes, int grid, uint32_t* sink, hipStream_t stream) {
  if (!src || !sink || bytes == 0 || bytes % 16 || bytes >= (size_t(1) << 31) ||
      (reinterpret_cast<uintptr_t>(src) & 15) || grid < 1 || grid > 65535)
    return QG_ERR_INVALID_ARG;
  hipLaunchKernelGGL(stream_read, dim3(grid), dim3(kStreamThreads), 0, stream, (const char*)src, (uint32_t)bytes,
                     sink);
  return launched();
}

int qgc_issue_mix(int mode, int kind, int grid, int iters, float* sink, uint64_t* clk, hipStream_t stream) {
  if (mode < 1 || mode > 3 || kind < 0 || kind > 2 || grid < 1 || grid > 65535 || iters < 1 || iters > (1 << 20) ||
      !sink || !clk)
    return QG_ERR_INVALID_ARG;
  void (*k)(int, float*, uint64_t*) = nullptr;
  if (mode == 1) k = issue_mix<1, 0>;
  else if (mode == 2) k = kind == 0 ? issue_mix<2, 0> : (kind == 1 ? issue_mix<2, 1> : issue_mix<2, 2>);
  else k = kind == 0 ? issue_mix<3, 0> : (kind == 1 ? issue_mix<3, 1> : issue_mix<3, 2>);
  hipLaunchKernelGGL(k, dim3(grid), dim3(kMfmaThreads), 0, stream, iters, sink, clk);
  return launched();
}

int qgc_empty(hipStream_t stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  return launched();
}

int qgc_host_us_per_call(qgc_run_fn fn, int n, qg_handle* h, const qg_operation* op, float alpha, const void* A,
                         const qg_layout* Adesc, const void* U, const qg_layout* Udesc, const void* B,
                         const qg_layout* Bdesc, const void* V, const qg_layout* Vdesc, float beta, const void* C,
                         const qg_layout* Cdesc, void* D, const qg_layout* Ddesc, const qg_workspace* ws,
                         hipStream_t stream, double* us_per_call) {
  if (!fn || n < 1 || !us_per_call) return QG_ERR_INVALID_ARG;
  const auto t0 = std::chrono::steady_clock::now();
  for (int i = 0; i < n; ++i) {
    const int st = fn(h, op, alpha, A, Adesc, U, Udesc, B, Bdesc, V, Vdesc, beta, C, Cdesc, D, Ddesc, ws, stream);
    if (st != QG_OK) return st;
  }
  const auto t1 = std::chrono::steady_clock::now();
  *us_per_call = std::chrono::duration<double, std::micro>(t1 - t0).count() / n;
  return QG_OK;
}

int qgc_host_us_per_empty(int n, int arg_bytes, hipStream_t stream, double* us_per_call) {
  if (n < 1 || !us_per_call || !(arg_bytes == 0 || arg_bytes == (int)sizeof(ArgBlock))) return QG_ERR_INVALID_ARG;
  ArgBlock blk = {};
  const auto t0 = std::chrono::steady_clock::now();
  if (arg_bytes == 0) {
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, stream);
  } else {
    for (int i = 0; i < n; ++i) hipLaunchKernelGGL(empty_args_kernel, dim3(1), dim3(64), 0, stream, blk);
  }
  const auto t1 = std::chrono::steady_clock::now();
  if (hipGetLastError() != hipSuccess) return QG_ERR_HIP;
  *us_per_call = std::chrono::duration<double, std::micro>(t1 - t0).count() / n;
  return QG_OK;
}

}  // extern "C"
