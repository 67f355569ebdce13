// Instantiations of the persistent grouped GEMM used by the backward pass:
// dgrad + dGLU (W2 [I][H] read as the K-contiguous W2^T) and dX (packed W1
// read transposed, N-contiguous, with the gate/up K remap).
#include "internal.hpp"

namespace moe {

template <int EPI, int BLAY>
static moe_status_t launch_one(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI, BLAY>), dim3(grid), dim3(GM_NT), 0, s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t launch_group_gemm_bwd(int epi, int blay, const GemmArgs& a, int grid, hipStream_t s) {
  if (epi == EPI_DGLU && blay == BL_NK) return launch_one<EPI_DGLU, BL_NK>(a, grid, s);
  if (epi == EPI_STORE && blay == BL_W1T) return launch_one<EPI_STORE, BL_W1T>(a, grid, s);
  return MOE_ERR_UNSUPPORTED;
}

}  // namespace moe
