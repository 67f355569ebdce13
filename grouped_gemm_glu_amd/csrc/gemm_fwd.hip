// Instantiations of the persistent grouped GEMM for the plain GroupGemm on the
// two unpacked weight orientations (N-contiguous [K][N] and K-contiguous
// [N][K]).
#include "internal.hpp"

namespace moe {

template <int EPI, int BLAY>
static moe_status_t launch_one(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI, BLAY>), dim3(grid), dim3(64 * gm_waves(EPI, BLAY, AT_BF16)), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t launch_group_gemm_fwd(int epi, int blay, const GemmArgs& a, int grid, hipStream_t s) {
  if (epi == EPI_STORE && blay == BL_KN) return launch_one<EPI_STORE, BL_KN>(a, grid, s);
  if (epi == EPI_STORE && blay == BL_NK) return launch_one<EPI_STORE, BL_NK>(a, grid, s);
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
