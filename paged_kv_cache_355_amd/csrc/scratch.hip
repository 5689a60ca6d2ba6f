// The workspace of pa_decode_noalloc, for callers that cannot allocate device
// memory (code under HIP graph capture, tight serving loops): a file-scope
// device array that every GPU the library runs on holds until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// only stands in for the symbol); it looks up the array's device address once
// per device and uses that address everywhere.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <mutex>

#include "launch.h"

namespace pa {
namespace {

static __device__ __align__(256) char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];   // device address of `scratch`, per device

constexpr int kZeroThreads = 256;

__global__ __launch_bounds__(kZeroThreads) void zero_kernel(uint4* __restrict__ p, int64_t n16) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * kZeroThreads;
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kZeroThreads + threadIdx.x; i < n16; i += stride)
    p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

hipError_t scratch_buffer(void** ptr) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));   // with `dev` current: its copy of the array
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

hipError_t launch_zero(void* p, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0) return hipSuccess;
  if (bytes % 16 != 0) return hipErrorInvalidValue;
  const int64_t n16 = bytes / 16;
  const int64_t blocks = std::min<int64_t>((n16 + kZeroThreads - 1) / kZeroThreads, 1024);
  hipLaunchKernelGGL(zero_kernel, dim3(static_cast<uint32_t>(blocks)), dim3(kZeroThreads), 0, stream,
                     static_cast<uint4*>(p), n16);
  return hipGetLastError();
}

}  // namespace pa
