// Weight gradients of the expert MLP as K-grouped GroupGemms: for each expert,
// C_e = A_e^T B_e with the reduction over the group's rows (dW1 = Xg^T dgu,
// dW2 = y^T dY2), fp32 output.
#include "internal.hpp"

namespace moe {

moe_status_t launch_group_gemm_wgrad(const GemmArgs& a, int grid, hipStream_t s) {
  if (grid < 1) return MOE_OK;    // no experts: nothing to write
  hipLaunchKernelGGL((group_gemm_kernel<EPI_WGRAD, BL_KN>), dim3(grid), dim3(64 * gm_waves(EPI_WGRAD, BL_KN, AT_BF16)), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
