// gemm_run_noalloc: gemm_run for callers that cannot allocate device memory (code under
// HIP graph capture, tight serving loops, harnesses that forbid hipMalloc). The split-K
// workspace (arrival counters, then fp32 partial tiles) is a file-scope device array of
// kNoallocBytes per GPU instead of a caller buffer. Each GPU holds its own copy until the
// process ends; its address on a device is taken once, with that device current, from
// hipGetSymbolAddress, and only that address is ever passed to kernels.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "../../include/dgemm.h"

namespace {

constexpr size_t kNoallocBytes = GEMM_NOALLOC_WORKSPACE_BYTES;
constexpr int kCounterWords = 64 * 1024 / 4;   // the workspace's arrival counters
constexpr int kMaxDevices = 64;

__device__ __align__(256) unsigned char scratch[kNoallocBytes];

// Zero n 32-bit words (a kernel, so that a caller's graph capture records no memset node).
__global__ void zero_words(uint32_t* p, int n) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) p[i] = 0u;
}

std::mutex g_mu;
void* g_scratch[kMaxDevices];   // device address of `scratch` on each device, once set up

// Device address of this device's scratch array. The first call on a device resolves it and
// clears the arrival counters on `stream` (every completed run leaves them zero again).
int scratch_for(int dev, hipStream_t stream, void** out) {
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_scratch[dev]) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return GEMM_ERR_HIP;
    hipLaunchKernelGGL(zero_words, dim3(kCounterWords / 256), dim3(256), 0, stream,
                       static_cast<uint32_t*>(ptr), kCounterWords);
    if (hipGetLastError() != hipSuccess) return GEMM_ERR_HIP;
    g_scratch[dev] = ptr;
  }
  *out = g_scratch[dev];
  return GEMM_OK;
}

}  // namespace

extern "C" int gemm_run_noalloc(gemm_plan_t plan, const void* A, const void* B,
                                const void* scales, void* C, void* stream) {
  if (!plan || !A || !B || !C) return GEMM_ERR_INVALID_ARG;
  size_t need = 0;
  int st = gemm_workspace_size(plan, &need);
  if (st != GEMM_OK) return st;
  if (need > kNoallocBytes) return GEMM_ERR_WORKSPACE_TOO_SMALL;
  if (need == 0) return gemm_run(plan, A, B, scales, C, nullptr, 0, stream);
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return GEMM_ERR_NO_DEVICE;
  void* ws = nullptr;
  st = scratch_for(dev, static_cast<hipStream_t>(stream), &ws);
  if (st != GEMM_OK) return st;
  return gemm_run(plan, A, B, scales, C, ws, kNoallocBytes, stream);
}
