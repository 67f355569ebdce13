// The block-scaled MXFP8 x MXFP8 GroupGemms on v_mfma_scale_f32_32x32x64_f8f6f4:
// GroupGemm + Quantize (activations quantised row-wise along K, the weight
// quantised along K and tile-blocked offline) and FC1 + GLU on the
// gate/up-repacked MXFP8 W1.
#include "internal.hpp"

namespace moe {

moe_status_t launch_group_gemm_mx(const GemmArgs& a, int grid, hipStream_t s) {
  hipLaunchKernelGGL((group_gemm_kernel<EPI_STORE, BL_PACKED, AT_MX>), dim3(grid), dim3(GM_NT), 0,
                     s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

moe_status_t launch_group_gemm_mx_glu(const GemmArgs& a, int epi, int grid, hipStream_t s) {
  if (epi == EPI_GLU)
    hipLaunchKernelGGL((group_gemm_kernel<EPI_GLU, BL_PACKED, AT_MX>), dim3(grid), dim3(GM_NT), 0, s, a);
  else
    hipLaunchKernelGGL((group_gemm_kernel<EPI_GLU_MX, BL_PACKED, AT_MX>), dim3(grid), dim3(GM_NT), 0,
                       s, a);
  return hipGetLastError() == hipSuccess ? MOE_OK : MOE_ERR_LAUNCH;
}

}  // namespace moe
