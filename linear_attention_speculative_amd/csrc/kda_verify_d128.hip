// Verify kernels of head dim 128 (templates in kda_verify_kernels.hpp; one
// translation unit per head dim so that they compile in parallel).
#include "kda_verify_kernels.hpp"

namespace kda {

template <>
int launch_verify_dim<128>(const VerifyParams& p, bool act_bf16, int schedule,
                          int grid, hipStream_t stream) {
  return act_bf16 ? launch_q<128, true>(p, schedule, grid, stream)
                  : launch_q<128, false>(p, schedule, grid, stream);
}

}  // namespace kda
