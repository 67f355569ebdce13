// Instantiation of the persistent grouped GEMM for the plain GroupGemm on a
// tile-blocked packed weight (FC2, dX).
#include "internal.hpp"

namespace moe {

template <int EPI, int BLAY>
static moe_status_t launch_one(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI, BLAY>), dim3(grid), dim3(64 * gm_waves(EPI, BLAY, AT_BF16)), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t launch_group_gemm_bwd(int epi, int blay, const GemmArgs& a, int grid, hipStream_t s) {
  if (epi == EPI_STORE && blay == BL_PACKED) return launch_one<EPI_STORE, BL_PACKED>(a, grid, s);
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
