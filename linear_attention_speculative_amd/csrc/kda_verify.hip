// Launch dispatch of the fused short-conv update + speculative verify (the
// kernels are in kda_verify_kernels.hpp, instantiated per head dim in
// kda_verify_d*.hip), the counter reset kernel, and the per-GPU scratch
// array of the allocation-free verify entry point.
#include <mutex>

#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

__global__ void kda_reset_kernel(int32_t* counter, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counter[i] = 0;
}

}  // namespace

// Work counters of the allocation-free verify entry point: the ticket
// counter and one arrival counter per (request, head), in one array per GPU
// that lives until the process ends.  Every launch that uses it leaves it
// at zero again.
static __device__ __align__(256) int32_t scratch[kScratchCounters];

int scratch_counters(hipStream_t stream, int32_t** out) {
  static std::mutex mu;
  static int32_t* ptr[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return int(e);
  if (dev < 0 || dev >= 64) return int(hipErrorInvalidDevice);
  std::lock_guard<std::mutex> lock(mu);
  if (ptr[dev] == nullptr) {
    // Once per device, with it current: the array's device address (its
    // name in host code is only a handle, not an address).
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return int(e);
    // cleared with a kernel (no memset node, should the caller capture it)
    hipLaunchKernelGGL(kda_reset_kernel, dim3(1), dim3(256), 0, stream,
                       static_cast<int32_t*>(a), kScratchCounters);
    e = hipGetLastError();
    if (e != hipSuccess) return int(e);
    ptr[dev] = static_cast<int32_t*>(a);
  }
  *out = ptr[dev];
  return 0;
}

int launch_verify(const VerifyParams& p, int D, bool act_bf16, int schedule,
                  int grid, hipStream_t stream) {
  switch (D) {
    case 16: return launch_verify_dim<16>(p, act_bf16, schedule, grid, stream);
    case 32: return launch_verify_dim<32>(p, act_bf16, schedule, grid, stream);
    case 64: return launch_verify_dim<64>(p, act_bf16, schedule, grid, stream);
    case 128:
      return launch_verify_dim<128>(p, act_bf16, schedule, grid, stream);
    default: return int(hipErrorInvalidValue);
  }
}

int launch_reset_counter(int32_t* counter, int n, hipStream_t stream) {
  hipLaunchKernelGGL(kda_reset_kernel, dim3(1), dim3(64), 0, stream, counter,
                     n);
  return int(hipGetLastError());
}

}  // namespace kda
