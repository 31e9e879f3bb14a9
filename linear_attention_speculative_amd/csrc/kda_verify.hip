// Launch dispatch of the fused short-conv update + speculative verify (the
// kernels are in kda_verify_kernels.hpp, instantiated per head dim in
// kda_verify_d*.hip) and the counter reset kernel.
#include "kda_device.hpp"
#include "kda_internal.hpp"

namespace kda {
namespace {

__global__ void kda_reset_kernel(int32_t* counter, int n) {
  for (int i = threadIdx.x; i < n; i += blockDim.x) counter[i] = 0;
}

}  // namespace

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
