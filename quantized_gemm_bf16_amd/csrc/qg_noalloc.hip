// qg_run_noalloc: qg_run for callers that cannot allocate device memory
// (code under HIP graph capture, tight serving loops, harnesses that forbid
// allocation). The split-K / stream-K workspace comes from a file-scope
// device array instead of the caller: each GPU holds its own copy of
// `scratch` (loaded with the library's code object, kept until the process
// ends). Host code never passes the array's name to a kernel -- in host code
// that name is a host-side stand-in, not a device address. Its device
// address is looked up once per device with hipGetSymbolAddress and only
// that address is used afterwards.
#include <hip/hip_runtime.h>

#include <mutex>

#include "../../include/qgemm.h"

namespace {

constexpr size_t kNoAllocBarriers = size_t(64) << 10;  // 16384 arrival counters
constexpr size_t kNoAllocPartials = size_t(16) << 20;  // partial tiles
constexpr size_t kNoAllocBytes = kNoAllocBarriers + kNoAllocPartials;

static __device__ __align__(256) char scratch[kNoAllocBytes];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices] = {};  // device address of `scratch` on each device

// Zeroes n 32-bit words (the arrival counters must start at zero; every run
// leaves them zero again). A kernel rather than hipMemsetAsync, so that a
// first call made under graph capture records no memset node.
__global__ void clear_words(int* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0;
}

// Device address of this device's scratch array; the first call on a device
// looks it up and clears the counters on `stream`.
int scratch_for(int dev, hipStream_t stream, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return QG_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> g(g_mu);
  if (!g_ptr[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) {
      (void)hipGetLastError();
      return QG_ERR_HIP;
    }
    const int words = (int)(kNoAllocBarriers / 4);
    hipLaunchKernelGGL(clear_words, dim3(16), dim3(256), 0, stream, (int*)ptr, words);
    if (hipGetLastError() != hipSuccess) return QG_ERR_HIP;
    g_ptr[dev] = ptr;
  }
  *out = g_ptr[dev];
  return QG_OK;
}

}  // namespace

extern "C" {

size_t qg_noalloc_barriers_size(void) { return kNoAllocBarriers; }
size_t qg_noalloc_partials_size(void) { return kNoAllocPartials; }

int qg_run_noalloc(qg_handle* h, const qg_operation* op, float alpha, const void* A, const qg_layout* Adesc,
                   const void* U, const qg_layout* Udesc, const void* B, const qg_layout* Bdesc, const void* V,
                   const qg_layout* Vdesc, float beta, const void* C, const qg_layout* Cdesc, void* D,
                   const qg_layout* Ddesc, hipStream_t stream) {
  if (!h || !op) return QG_ERR_INVALID_ARG;
  // measuring creates events and synchronises: not for this entry point
  if (op->policy == QG_POLICY_MEASURE) return QG_ERR_UNSUPPORTED;
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return QG_ERR_HIP;
  }
  void* ptr = nullptr;
  const int st = scratch_for(dev, stream, &ptr);
  if (st != QG_OK) return st;
  qg_workspace ws;
  ws.barriers = ptr;
  ws.barriers_size = kNoAllocBarriers;
  ws.partials = (char*)ptr + kNoAllocBarriers;
  ws.partials_size = kNoAllocPartials;
  // qg_run allocates nothing; a plan needing more workspace than the scratch
  // array holds is refused with QG_ERR_WORKSPACE
  return qg_run(h, op, alpha, A, Adesc, U, Udesc, B, Bdesc, V, Vdesc, beta, C, Cdesc, D, Ddesc, &ws, stream);
}

}  // extern "C"
